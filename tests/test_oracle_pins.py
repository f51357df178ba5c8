"""Pins of the float64 oracle against what the pages and mathematics fix.

None of these compares the oracle with itself: each check is a closed form,
an invariant, a special case that reduces to a textbook or library routine,
values computed by hand from the pages' rules (tests/golden/k_table.json), or
the independent token-space brute force in tests/bruteforce.py.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import lcsa_oracle as O
from bruteforce import bp_window, bt_window, lcsa_bruteforce
from block_sparse_attention_03_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_tokens(rng, B, T, H, W, NH, D):
    return rng.standard_normal((B, T, H, W, NH, D))


# ---------------------------------------------------------------- partition

def test_partition_roundtrip_bitwise():
    rng = np.random.default_rng(1)
    x = rand_tokens(rng, 2, 6, 16, 24, 3, 5)
    xb = O.partition(x)
    assert xb.shape == (2, 3, 3 * 2 * 3, 128, 5)
    assert np.array_equal(O.unpartition(xb, 6, 16, 24), x)


def test_partition_blocks_are_2x8x8_windows():
    """Every block holds exactly the tokens of one 2x8x8 window, blocks in
    (bt, by, bx) order, tokens inside in (dt, dy, dx) row-major order."""
    T, H, W = 4, 16, 24
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    code = (t * 1000 + y) * 1000 + x                       # unique per token
    xin = code[None, :, :, :, None, None].astype(np.float64)
    xb = O.partition(xin)[0, 0, :, :, 0]                    # [nblk][128]
    nby, nbx = H // 8, W // 8
    seen = set()
    for n in range(xb.shape[0]):
        bt, rem = divmod(n, nby * nbx)
        by, bx = divmod(rem, nbx)
        for tau in range(128):
            dt, r2 = divmod(tau, 64)
            dy, dx = divmod(r2, 8)
            c = int(xb[n, tau])
            tt, yy, xx = c // 1000000, (c // 1000) % 1000, c % 1000
            assert (tt, yy, xx) == (2 * bt + dt, 8 * by + dy, 8 * bx + dx)
            seen.add(c)
    assert len(seen) == T * H * W                           # a bijection


def test_partition_rejects_partial_windows():
    for shape in [(1, 3, 16, 16, 1, 4), (1, 4, 12, 16, 1, 4), (1, 4, 16, 20, 1, 4)]:
        with pytest.raises(ValueError):
            O.partition(np.zeros(shape))


# ---------------------------------------------------------------- pooling

def test_pool_constant_block():
    # dyadic constants: every partial sum is exact, so the mean is c exactly
    rng = np.random.default_rng(2)
    c = rng.integers(-4096, 4096, size=(1, 2, 6, 1, 4)) / 1024.0
    xb = np.broadcast_to(c, (1, 2, 6, 128, 4)).copy()
    assert np.array_equal(O.pool(xb), xb[:, :, :, 0, :])


def test_pool_linear_field_is_value_at_block_centre():
    """A field linear in (t, y, x) pools to its value at the window centre
    (2bt+0.5, 8by+3.5, 8bx+3.5)."""
    T, H, W = 4, 16, 24
    a, by_, bx_, c0 = 0.3, -0.7, 0.25, 1.5
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    f = (a * t + by_ * y + bx_ * x + c0)[None, :, :, :, None, None]
    p = O.pool(O.partition(f))[0, 0, :, 0]
    nby, nbx = H // 8, W // 8
    for n in range(p.shape[0]):
        bt, rem = divmod(n, nby * nbx)
        by, bx = divmod(rem, nbx)
        want = a * (2 * bt + 0.5) + by_ * (8 * by + 3.5) + bx_ * (8 * bx + 3.5) + c0
        assert abs(p[n] - want) < 1e-12


def test_pool_linearity():
    rng = np.random.default_rng(3)
    x1, x2 = rng.standard_normal((2, 1, 3, 4, 128, 6))
    lhs = O.pool(2.5 * x1 - 1.25 * x2)
    rhs = 2.5 * O.pool(x1) - 1.25 * O.pool(x2)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- windows / mask

@pytest.mark.parametrize("n", list(range(1, 31)))
@pytest.mark.parametrize("r", [1, 3, 5, 11, 13])
def test_windows_match_independent_definitions(n, r):
    for i in range(n):
        assert set(O.window_1d(i, n, r, O.BORDER_PRESERVED)) == bp_window(i, n, r)
        assert set(O.window_1d(i, n, r, O.BORDER_TRUNCATED)) == bt_window(i, n, r)


@pytest.mark.parametrize("n", [1, 2, 5, 6, 11, 12, 21, 30])
def test_window_properties(n):
    r = 11
    for i in range(n):
        bp = list(O.window_1d(i, n, r, O.BORDER_PRESERVED))
        bt = list(O.window_1d(i, n, r, O.BORDER_TRUNCATED))
        assert i in bp and i in bt                      # include_self
        assert len(bp) == min(r, n)                     # fixed size, shifted inside
        assert bp == list(range(bp[0], bp[0] + len(bp))) and 0 <= bp[0] and bp[-1] < n
        assert len(bt) == min(i + 5, n - 1) - max(i - 5, 0) + 1
        if 5 <= i <= n - 6:                             # interior: both centred
            assert bp == bt == list(range(i - 5, i + 6))


def test_allowed_counts_closed_form_and_golden():
    g = json.load(open(os.path.join(GOLDEN, "k_table.json")))
    p = O.SelectParams(local_range=11)
    for case in g["allowed_counts"]:
        nby, nbx = case["nby"], case["nbx"]
        for vis, want in zip(case["key_tbs_visible"], case["allowed"]):
            # query TB = vis-1 sees TBs 0..vis-1
            m = O.allowed_mask([vis - 1], list(range(vis)), nby, nbx, p)
            counts = m.sum(axis=1)
            assert np.all(counts == min(11, nby) * min(11, nbx) * vis)
            assert counts.max() == want


def test_allowed_counts_bt_closed_form():
    p = O.SelectParams(local_range=11, border=O.BORDER_TRUNCATED)
    nby, nbx = 12, 21
    m = O.allowed_mask([2], [0, 1, 2, 3], nby, nbx, p)   # TB 3 is in the future
    for i in range(nby * nbx):
        by, bx = divmod(i, nbx)
        cy = min(by + 5, nby - 1) - max(by - 5, 0) + 1
        cx = min(bx + 5, nbx - 1) - max(bx - 5, 0) + 1
        assert m[i].sum() == cy * cx * 3


def test_causality_never_future():
    p = O.SelectParams(local_range=31)
    m = O.allowed_mask([0, 1, 2], [0, 1, 2], 2, 3, p)
    nS = 6
    for i in range(18):
        for j in range(18):
            assert m[i, j] == (j // nS <= i // nS)


# ---------------------------------------------------------------- softmax / top-k

def test_softmax_rows_sum_to_one_and_match_scipy():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((20, 40)) * 3
    allowed = rng.random((20, 40)) < 0.4
    allowed[:, 0] = True
    s = np.where(allowed, s, -np.inf)
    p = O.softmax_rows(s)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[~allowed] == 0)
    for i in range(20):
        ref = scipy.special.softmax(s[i, allowed[i]])
        assert np.allclose(p[i, allowed[i]], ref, rtol=1e-13, atol=1e-15)


def test_k_table_golden():
    g = json.load(open(os.path.join(GOLDEN, "k_table.json")))
    for case in g["k_rows"]:
        if "topk_fixed" in case:
            p = O.SelectParams(topk_fixed=case["topk_fixed"])
        else:
            num, den = case["ratio"]
            p = O.SelectParams(ratio_num=num, ratio_den=den,
                               scale_by_resolution=case["scale"])
            if case["scale"]:
                p.out_h, p.out_w = case["out"]
        for n, k in zip(case["n_allowed"], case["k"]):
            assert O.topk_count(n, 10 ** 6, p) == k, case["name"]


def test_k_rule_edges():
    p = O.SelectParams(ratio_num=1, ratio_den=5)
    assert O.topk_count(0, 10, p) == 0
    assert O.topk_count(1, 10, p) == 1          # floor 0 -> clamped to 1
    assert O.topk_count(4, 10, p) == 1
    assert O.topk_count(5, 10, p) == 1
    assert O.topk_count(10, 10, p) == 2
    p_all = O.SelectParams(ratio_num=1, ratio_den=1)
    assert O.topk_count(7, 10, p_all) == 7
    p_base = O.SelectParams(ratio_num=1, ratio_den=5, ratio_base=1)
    assert O.topk_count(30, 1000, p_base) == 30  # 200 clamped to allowed
    assert O.topk_count(30, 100, p_base) == 20
    assert O.topk_count(3, 10, O.SelectParams(topk_fixed=5)) == 3


def test_topk_threshold_property_and_count():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((30, 50))
    allowed = rng.random((30, 50)) < 0.5
    allowed[:, 3] = True
    s = np.where(allowed, s, -np.inf)
    p = O.SelectParams(ratio_num=1, ratio_den=3)
    sel, ks = O.select_topk(s, p)
    for i in range(30):
        na = allowed[i].sum()
        assert ks[i] == max(1, min(na // 3, na)) and len(sel[i]) == ks[i]
        assert np.all(allowed[i, sel[i]])
        rest = np.setdiff1d(np.nonzero(allowed[i])[0], sel[i])
        if len(rest):
            assert s[i, sel[i]].min() >= s[i, rest].max()
        assert np.all(np.diff(sel[i]) > 0)


def test_topk_all_equal_scores_takes_lowest_indices():
    s = np.zeros((3, 10))
    s[:, 7] = -np.inf
    sel, _ = O.select_topk(s, O.SelectParams(topk_fixed=4))
    for row in sel:
        assert list(row) == [0, 1, 2, 3]
    sel, _ = O.select_topk(s, O.SelectParams(topk_fixed=9))
    assert list(sel[0]) == [0, 1, 2, 3, 4, 5, 6, 8, 9]


# ---------------------------------------------------------------- whole pipeline

def tiny_inputs(seed=11, T=4, H=16, W=16, NH=2, D=64, t0=0):
    d = synth.make_qkv(seed, NH, D, H, W, t0, t0 + T, dtype="f32")
    return d["q"][1], d["k"][1], d["v"][1]


@pytest.mark.parametrize("border", [O.BORDER_PRESERVED, O.BORDER_TRUNCATED])
@pytest.mark.parametrize("r,shape", [(11, (4, 16, 16)), (3, (4, 32, 24)), (1, (2, 24, 16))])
def test_pipeline_matches_token_space_bruteforce(border, r, shape):
    T, H, W = shape
    q, k, v = tiny_inputs(T=T, H=H, W=W)
    p = O.SelectParams(local_range=r, border=border, topk_fixed=3)
    res = O.lcsa_step(q, k, v, O.KVCache(cap_tb=8), 0, p)
    bf_out, bf_sel, _ = lcsa_bruteforce(q[0], k[0], v[0], 0, 0, r, border,
                                        lambda na, nk: min(3, na))
    for h in range(q.shape[4]):
        for i in range(len(res.sel[0][h])):
            assert list(res.sel[0][h][i]) == bf_sel[(h, i)]
    assert np.abs(res.out[0] - bf_out).max() < 1e-12


def test_streaming_pipeline_matches_bruteforce_on_concatenated_frames():
    """Step n of a stream equals a from-scratch computation over the explicitly
    concatenated frames of the cache window."""
    H, W, NH, D = 16, 24, 2, 32
    p = O.SelectParams(local_range=3, ratio_num=1, ratio_den=4)
    cache = O.KVCache(cap_tb=2)
    seed = 5
    for step in range(4):
        t0 = 2 * step
        d = synth.make_qkv(seed, NH, D, H, W, t0, t0 + 2, dtype="bf16")
        q, k, v = (d[n][1] for n in "qkv")
        res = O.lcsa_step(q, k, v, cache, step, p)
        kt0 = max(0, t0 - 4)
        dk = synth.make_qkv(seed, NH, D, H, W, kt0, t0 + 2, dtype="bf16", which="kv")
        bf_out, bf_sel, _ = lcsa_bruteforce(q[0], dk["k"][1][0], dk["v"][1][0], t0, kt0, 3, 0,
                                            lambda na, nk: O.topk_count(na, nk, p))
        assert np.abs(res.out[0] - bf_out).max() < 1e-12
        for h in range(NH):
            for i in range(len(res.sel[0][h])):
                assert list(res.sel[0][h][i]) == bf_sel[(h, i)]
        assert cache.tbs() == list(range(max(0, step - 1), step + 1))


def test_topk_all_unbounded_is_dense_block_causal_attention():
    """k = every allowed block and a window covering the grid: dense attention
    with a block-causal (temporal block) mask."""
    T, H, W, NH, D = 6, 16, 16, 2, 16
    q, k, v = tiny_inputs(T=T, H=H, W=W, NH=NH, D=D)
    p = O.SelectParams(local_range=99, ratio_num=1, ratio_den=1)
    res = O.lcsa_step(q, k, v, O.KVCache(cap_tb=8), 0, p)
    qf = q[0].reshape(-1, NH, D)
    kf = k[0].reshape(-1, NH, D)
    vf = v[0].reshape(-1, NH, D)
    tb = np.repeat(np.arange(T) // 2, H * W)
    mask = tb[None, :] <= tb[:, None]
    ref = np.empty_like(qf)
    for h in range(NH):
        lg = qf[:, h] @ kf[:, h].T / math.sqrt(D)
        lg = np.where(mask, lg, -np.inf)
        w = np.exp(lg - lg.max(axis=1, keepdims=True))
        ref[:, h] = (w / w.sum(axis=1, keepdims=True)) @ vf[:, h]
    assert np.abs(res.out[0].reshape(-1, NH, D) - ref).max() < 1e-12


def test_single_tb_all_keys_is_torch_sdpa():
    T, H, W, NH, D = 2, 16, 24, 3, 32
    q, k, v = tiny_inputs(T=T, H=H, W=W, NH=NH, D=D)
    p = O.SelectParams(local_range=99, ratio_num=1, ratio_den=1)
    res = O.lcsa_step(q, k, v, O.KVCache(cap_tb=8), 0, p)
    tq = torch.from_numpy(q[0].reshape(-1, NH, D)).permute(1, 0, 2)
    tk = torch.from_numpy(k[0].reshape(-1, NH, D)).permute(1, 0, 2)
    tv = torch.from_numpy(v[0].reshape(-1, NH, D)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    assert np.abs(res.out[0].reshape(-1, NH, D) - ref).max() < 1e-12


def test_constant_v_gives_constant_output():
    q, k, v = tiny_inputs()
    v = np.full_like(v, 0.375)
    res = O.lcsa_step(q, k, v, O.KVCache(cap_tb=8), 0, O.SelectParams(topk_fixed=3))
    assert np.abs(res.out - 0.375).max() < 1e-14


def test_zero_q_gives_mean_of_selected_v():
    q, k, v = tiny_inputs()
    q = np.zeros_like(q)
    res = O.lcsa_step(q, k, v, O.KVCache(cap_tb=8), 0, O.SelectParams(topk_fixed=3))
    vb = O.partition(v)
    ob = O.partition(res.out)
    for h in range(q.shape[4]):
        for i, row in enumerate(res.sel[0][h]):
            want = vb[0, h, row].reshape(-1, vb.shape[-1]).mean(axis=0)
            assert np.abs(ob[0, h, i] - want[None]).max() < 1e-13


def test_k1_is_plain_128x128_attention():
    q, k, v = tiny_inputs()
    res = O.lcsa_step(q, k, v, O.KVCache(cap_tb=8), 0, O.SelectParams(topk_fixed=1))
    qb, kb, vb, ob = (O.partition(a) for a in (q, k, v, res.out))
    D = q.shape[-1]
    for h in range(q.shape[4]):
        for i, row in enumerate(res.sel[0][h]):
            assert len(row) == 1
            tq = torch.from_numpy(qb[0, h, i])[None]
            tk = torch.from_numpy(kb[0, h, row[0]])[None]
            tv = torch.from_numpy(vb[0, h, row[0]])[None]
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0].numpy()
            assert np.abs(ob[0, h, i] - ref).max() < 1e-13


def test_lse_is_log_partition_function():
    q, k, v = tiny_inputs()
    res = O.lcsa_step(q, k, v, O.KVCache(cap_tb=8), 0, O.SelectParams(topk_fixed=2))
    qb, kb = O.partition(q), O.partition(k)
    D = q.shape[-1]
    h, i = 1, 5
    K = kb[0, h, res.sel[0][h][i]].reshape(-1, D)
    lg = qb[0, h, i] @ K.T / math.sqrt(D)
    assert np.allclose(res.lse[0, h, i], scipy.special.logsumexp(lg, axis=1), rtol=0, atol=1e-12)


def test_cold_start_rows_equal_streaming_step():
    """A cold start's last TB rows equal a streaming step with the earlier TBs
    cached: same keys, same allowed count, same k."""
    H, W, NH, D = 24, 32, 2, 32
    p = O.SelectParams(local_range=3, ratio_num=1, ratio_den=3)
    d = synth.make_qkv(9, NH, D, H, W, 0, 6, dtype="bf16")
    q, k, v = (d[n][1] for n in "qkv")
    cold = O.lcsa_step(q, k, v, O.KVCache(cap_tb=3), 0, p)
    cache = O.KVCache(cap_tb=3)
    O.lcsa_step(q[:, :4], k[:, :4], v[:, :4], cache, 0, p, evict=False)
    warm = O.lcsa_step(q[:, 4:], k[:, 4:], v[:, 4:], cache, 2, p)
    assert np.abs(cold.out[:, 4:] - warm.out).max() < 1e-12
    nS = (H // 8) * (W // 8)
    assert np.array_equal(cold.kcount[2 * nS:], warm.kcount)


def test_cache_holds_last_cap_tbs():
    H, W, NH, D = 16, 16, 1, 16
    p = O.SelectParams(local_range=11, topk_fixed=2)
    cache = O.KVCache(cap_tb=3)
    for step in range(7):
        d = synth.make_qkv(3, NH, D, H, W, 2 * step, 2 * step + 2, dtype="f32")
        res = O.lcsa_step(*(d[n][1] for n in "qkv"), cache, step, p)
        assert res.key_tbs == list(range(max(0, step - 3), step + 1))
        assert cache.tbs() == list(range(max(0, step - 2), step + 1))


def test_oracle_is_deterministic_bitwise():
    q, k, v = tiny_inputs()
    p = O.SelectParams(topk_fixed=3)
    a = O.lcsa_step(q, k, v, O.KVCache(cap_tb=8), 0, p)
    b = O.lcsa_step(q, k, v, O.KVCache(cap_tb=8), 0, p)
    assert np.array_equal(a.out, b.out) and np.array_equal(a.probs, b.probs)


# ---------------------------------------------------------------- planted mistakes

def test_planted_window_off_by_one_is_caught(monkeypatch):
    """Positive control: a wrong window must make the independent pin fail."""
    real = O.window_1d

    def wrong(i, n, r, border):
        w = real(i, n, r, border)
        return range(w.start, max(w.start + 1, w.stop - 1))
    monkeypatch.setattr(O, "window_1d", wrong)
    bad = sum(set(O.window_1d(i, 21, 11, 0)) != bp_window(i, 21, 11) for i in range(21))
    assert bad > 0


def test_planted_transposed_scores_are_caught(monkeypatch):
    """Positive control: transposing the draft operands changes selections vs
    the brute force."""
    q, k, v = tiny_inputs(T=4, H=24, W=24)
    p = O.SelectParams(local_range=3, topk_fixed=2)
    monkeypatch.setattr(O, "draft_scores",
                        lambda pq, pk, allowed: np.where(allowed, -(pq @ pk.T), -np.inf))
    res = O.lcsa_step(q, k, v, O.KVCache(cap_tb=8), 0, p)
    _, bf_sel, _ = lcsa_bruteforce(q[0], k[0], v[0], 0, 0, 3, 0, lambda na, nk: min(2, na))
    diff = sum(list(res.sel[0][h][i]) != bf_sel[(h, i)]
               for h in range(2) for i in range(len(res.sel[0][h])))
    assert diff > 0


# ---------------------------------------------------------------- cache priming and row subsets

def _primed_stream(prime, H=16, W=24, NH=2, D=32, seed=13, p=None, n_steps=2):
    """Prime a cap-3 cache with frames 0-5 through ``prime`` (k/v only), then
    step frames 6-7, 8-9, ...: per step the oracle's result and the key
    frames the step attends ([HW] 2.3: the cache keeps the newest temporal
    blocks and drops the oldest)."""
    p = p or O.SelectParams(local_range=3, ratio_num=1, ratio_den=4)
    cache = O.KVCache(cap_tb=3)
    d0 = synth.make_qkv(seed, NH, D, H, W, 0, 6, dtype="bf16", which="kv")
    prime(cache, d0["k"][1], d0["v"][1], 0)
    out = []
    for n in range(n_steps):
        t0 = 6 + 2 * n
        d = synth.make_qkv(seed, NH, D, H, W, t0, t0 + 2, dtype="bf16")
        res = O.lcsa_step(d["q"][1], d["k"][1], d["v"][1], cache, t0 // 2, p)
        out.append((t0, d["q"][1], res, list(cache.tbs())))
    return out, p


def _check_against_bruteforce(steps, p, H=16, W=24, NH=2, D=32, seed=13):
    for t0, q, res, tbs_after in steps:
        kt0 = t0 - 6  # the view: the 3 cached TBs and the new one
        dk = synth.make_qkv(seed, NH, D, H, W, kt0, t0 + 2, dtype="bf16", which="kv")
        bf_out, bf_sel, _ = lcsa_bruteforce(q[0], dk["k"][1][0], dk["v"][1][0], t0, kt0,
                                            p.local_range, p.border,
                                            lambda na, nk: O.topk_count(na, nk, p))
        for h in range(NH):
            for i in range(len(res.sel[0][h])):
                assert list(res.sel[0][h][i]) == bf_sel[(h, i)], (t0, h, i)
        assert np.abs(res.out[0] - bf_out).max() < 1e-12
        assert res.key_tbs == list(range(kt0 // 2, t0 // 2 + 1))
        assert tbs_after == list(range(kt0 // 2 + 1, t0 // 2 + 1))


def test_prime_cache_then_steps_match_bruteforce():
    """prime_cache over frames 0-5 followed by streaming steps equals the
    token-space brute force over the explicitly concatenated key frames."""
    steps, p = _primed_stream(O.prime_cache)
    _check_against_bruteforce(steps, p)


def test_prime_cache_entries_are_the_token_windows():
    """Each primed entry is its temporal block: label first_abs_tb + t, and
    block (by, bx) holds tokens (2t + dt, 8by + dy, 8bx + dx) at position
    (dt*8 + dy)*8 + dx, gathered here straight from token coordinates."""
    H, W, NH, D = 16, 24, 2, 8
    d = synth.make_qkv(4, NH, D, H, W, 0, 6, dtype="f32", which="kv")
    k, v = d["k"][1], d["v"][1]
    cache = O.KVCache(cap_tb=8)
    O.prime_cache(cache, k, v, 5)
    assert cache.tbs() == [5, 6, 7]
    nbx = W // 8
    for t, (tb, kb, vb, kp) in enumerate(cache.entries):
        for s in range(kb.shape[2]):
            by, bx = divmod(s, nbx)
            for tau in range(128):
                dt, dy, dx = tau // 64, (tau // 8) % 8, tau % 8
                tok = (0, 2 * t + dt, 8 * by + dy, 8 * bx + dx)
                assert np.array_equal(kb[0, :, s, tau], k[tok])
                assert np.array_equal(vb[0, :, s, tau], v[tok])
            assert np.allclose(kp[0, :, s], kb[0, :, s].mean(axis=1), rtol=0, atol=1e-15)


def test_planted_prime_cache_mistakes_are_caught(monkeypatch):
    """Positive controls: a primed cache whose temporal-block labels are
    shifted (the newest primed block then counts as later than the query)
    or whose blocks are appended in the wrong order disagrees with the
    brute force."""
    def shifted(cache, k, v, first_abs_tb):
        O.prime_cache(cache, k, v, first_abs_tb + 2)

    def reversed_order(cache, k, v, first_abs_tb):
        tmp = O.KVCache(cap_tb=8)
        O.prime_cache(tmp, k, v, first_abs_tb)
        for e in reversed(tmp.entries):
            cache.append(*e)

    for bad in (shifted, reversed_order):
        steps, p = _primed_stream(bad, n_steps=1)
        with pytest.raises(AssertionError):
            _check_against_bruteforce(steps, p)


def test_lcsa_step_rows_subset_equals_full_run_on_those_rows():
    """rows=R computes exactly the full run's values on the rows in R
    (bitwise: the same per-row arithmetic) and leaves every other row at
    out = 0, lse = -inf; the selections do not depend on R."""
    H, W, NH, D = 16, 24, 2, 32
    p = O.SelectParams(local_range=3, ratio_num=1, ratio_den=3)
    d = synth.make_qkv(21, NH, D, H, W, 0, 4, dtype="bf16")
    q, k, v = (d[n][1] for n in "qkv")
    full = O.lcsa_step(q, k, v, O.KVCache(cap_tb=3), 0, p)
    rows = [(0, 0, 0), (0, 1, 5), (0, 1, 11)]
    part = O.lcsa_step(q, k, v, O.KVCache(cap_tb=3), 0, p, rows=rows)
    ob_full = O.partition(full.out)
    ob_part = O.partition(part.out)
    nq = ob_full.shape[2]
    for h in range(NH):
        assert [list(r) for r in part.sel[0][h]] == [list(r) for r in full.sel[0][h]]
        for i in range(nq):
            if (0, h, i) in rows:
                assert np.array_equal(ob_part[0, h, i], ob_full[0, h, i])
                assert np.array_equal(part.lse[0, h, i], full.lse[0, h, i])
                assert np.abs(ob_full[0, h, i]).max() > 0
            else:
                assert not ob_part[0, h, i].any()
                assert np.all(np.isneginf(part.lse[0, h, i]))


def test_planted_rows_subset_mistake_is_caught(monkeypatch):
    """Positive control: a row-subset branch that computes the wrong row
    (an off-by-one block index) fails the subset pin's comparison."""
    real = O.sparse_attention_row
    calls = {}

    def wrong_row(qb, kb, vb, sel_row, scale):
        calls["n"] = calls.get("n", 0) + 1
        return real(qb[::-1].copy(), kb, vb, sel_row, scale)  # rows of the block reversed
    H, W, NH, D = 16, 16, 1, 16
    p = O.SelectParams(local_range=3, topk_fixed=2)
    d = synth.make_qkv(2, NH, D, H, W, 0, 2, dtype="f32")
    q, k, v = (d[n][1] for n in "qkv")
    full = O.lcsa_step(q, k, v, O.KVCache(cap_tb=3), 0, p)
    monkeypatch.setattr(O, "sparse_attention_row", wrong_row)
    part = O.lcsa_step(q, k, v, O.KVCache(cap_tb=3), 0, p, rows=[(0, 0, 1)])
    assert calls["n"] == 1
    assert not np.array_equal(O.partition(part.out)[0, 0, 1], O.partition(full.out)[0, 0, 1])
