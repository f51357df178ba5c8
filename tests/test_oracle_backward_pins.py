"""Pins of the oracle's block-sparse attention backward.

Checked against finite differences of the forward with the lists held
fixed, against torch autograd of scaled_dot_product_attention (float64, CPU)
where every key block is selected, and against two identities that hold for
any lists: the key gradients of one query row sum to zero (a softmax row's
Jacobian annihilates constants), so dK sums to zero over all key tokens;
and each row of P sums to one, so dV summed over key tokens equals dO summed
over query tokens. Planted mistakes in a copy of the oracle must fail.
"""
from __future__ import annotations

import inspect
import math

import numpy as np
import pytest
import torch

from oracle import lcsa_oracle as O


def tiny(T=4, H=16, W=16, NH=2, D=8, seed=5):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((1, T, H, W, NH, D)) for _ in range(4))


def some_lists(nq, NH, seed=0, k=3):
    """Fixed per-row lists: ascending, non-empty, varied lengths."""
    rng = np.random.default_rng(seed)
    return [[sorted(rng.choice(nq, size=int(rng.integers(1, k + 1)), replace=False).tolist())
             for _ in range(nq)] for _ in range(NH)]


def forward(q, k, v, sel, scale):
    qb, kb, vb = O.partition(q), O.partition(k), O.partition(v)
    ob = np.zeros_like(qb)
    for h in range(q.shape[4]):
        for i in range(qb.shape[2]):
            ob[0, h, i], _ = O.sparse_attention_row(qb[0, h, i], kb[0, h], vb[0, h],
                                                    np.array(sel[0][h][i]), scale)
    return ob


def test_matches_finite_differences():
    q, k, v, g = tiny()
    scale = 1 / math.sqrt(8)
    nq = 2 * 2 * 2
    sel = [some_lists(nq, 2)]
    dq, dk, dv = O.sparse_attention_backward(q, k, v, g, sel, scale)
    gb = O.partition(g)
    loss = lambda qq, kk, vv: float((forward(qq, kk, vv, sel, scale) * gb).sum())
    rng = np.random.default_rng(9)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        gflat = O.unpartition(grad, 4, 16, 16)
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if n == name else a for n, a in (("q", q), ("k", k), ("v", v))]
            args_m = [xm if n == name else a for n, a in (("q", q), ("k", k), ("v", v))]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - gflat[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, gflat[idx])


def test_all_keys_selected_matches_torch_autograd():
    q, k, v, g = tiny(T=2, H=16, W=24, NH=2, D=16)
    nq = 6
    sel = [[list(range(nq)) for _ in range(nq)] for _ in range(2)]
    dq, dk, dv = O.sparse_attention_backward(q, k, v, g, [sel])
    # block order inside a block does not matter for dense attention: compare
    # in token layout against SDPA over the whole token sequence
    L = 2 * 16 * 24
    tq, tk, tv = (torch.tensor(x.reshape(L, 2, 16).transpose(1, 0, 2), requires_grad=True)
                  for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0]
    out.backward(torch.tensor(g.reshape(L, 2, 16).transpose(1, 0, 2)))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        tok = O.unpartition(mine, 2, 16, 24).reshape(L, 2, 16).transpose(1, 0, 2)
        assert np.allclose(tok, ref.numpy(), rtol=0, atol=1e-12)


def test_identities_hold_for_any_lists():
    q, k, v, g = tiny(T=6, H=16, W=16, NH=3, D=8, seed=11)
    nq = 3 * 4
    sel = [some_lists(nq, 3, seed=4, k=5)]
    dq, dk, dv = O.sparse_attention_backward(q, k, v, g, sel)
    gb = O.partition(g)
    for h in range(3):
        assert np.allclose(dk[0, h].sum(axis=(0, 1)), 0.0, atol=1e-12)
        assert np.allclose(dv[0, h].sum(axis=(0, 1)), gb[0, h].sum(axis=(0, 1)), atol=1e-12)


def test_rows_subset_gives_those_rows():
    q, k, v, g = tiny()
    sel = [some_lists(8, 2, seed=2)]
    full = O.sparse_attention_backward(q, k, v, g, sel)
    rows = {(0, 1, 3), (0, 0, 5)}
    part = O.sparse_attention_backward(q, k, v, g, sel, rows=rows)
    for (b, h, i) in rows:
        assert np.array_equal(part[0][b, h, i], full[0][b, h, i])
    # key blocks selected only by the given rows get their full gradient
    for h in range(2):
        users = {}
        for i in range(8):
            for j in sel[0][h][i]:
                users.setdefault(j, set()).add(i)
        for j, us in users.items():
            if all((0, h, i) in rows for i in us):
                assert np.allclose(part[1][0, h, j], full[1][0, h, j], rtol=0, atol=1e-14)


def planted(old: str, new: str):
    src = inspect.getsource(O.sparse_attention_backward)
    assert old in src
    ns = dict(vars(O))
    exec(src.replace(old, new), ns)
    return ns["sparse_attention_backward"]


@pytest.mark.parametrize("old,new", [
    ("dP - (P * dP).sum(axis=1, keepdims=True)", "dP"),            # Jacobian term dropped
    ("dq[b, h, i] = scale * (dS @ K)", "dq[b, h, i] = dS @ K"),   # scale dropped
    ("gV = P.T @ dO", "gV = dS.T @ dO"),                           # dS in place of P
    ("dP = dO @ V.T", "dP = dO @ K.T"),                            # K in place of V
])
def test_planted_mistakes_are_caught(old, new):
    q, k, v, g = tiny(T=2, H=16, W=24, NH=1, D=16)
    sel = [[[list(range(6)) for _ in range(6)]]]
    bad = planted(old, new)(q, k, v, g, sel)
    good = O.sparse_attention_backward(q, k, v, g, sel)
    assert any(not np.allclose(b_, g_, rtol=0, atol=1e-6) for b_, g_ in zip(bad, good))
    # and the autograd pin itself fails for the mutant
    L = 2 * 16 * 24
    tq, tk, tv = (torch.tensor(x.reshape(L, 1, 16).transpose(1, 0, 2), requires_grad=True)
                  for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0]
    out.backward(torch.tensor(g.reshape(L, 1, 16).transpose(1, 0, 2)))
    refs = (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())
    mism = 0
    for mine, ref in zip(bad, refs):
        tok = O.unpartition(mine, 2, 16, 24).reshape(L, 1, 16).transpose(1, 0, 2)
        mism += not np.allclose(tok, ref, rtol=0, atol=1e-9)
    assert mism > 0
