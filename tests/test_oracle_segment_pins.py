"""Pins of the oracle's Stage-1 segment-masked attention.

[FN] Key design 1, Stage 1: attention weights exp(q_i k_j / sqrt(d)) times
the indicator that tokens i and j lie in the same segment, normalised over
the same masked sum. Each check below is a special case that reduces to a
library routine (torch's scaled_dot_product_attention in float64 on the
CPU), a pure-Python brute force of that formula over every key, or an
invariant; planted mistakes in a copy of the oracle must fail them.
"""
from __future__ import annotations

import inspect
import math

import numpy as np
import pytest
import torch

from oracle import lcsa_oracle as O


def inputs(T=4, H=4, W=4, NH=2, D=8, seed=3):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((1, T, H, W, NH, D)) for _ in range(3))


def sdpa(q, k, v):
    """torch SDPA over a [L][NH][D] sequence, float64 on the CPU."""
    t = [torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None] for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(*t)[0].numpy().transpose(1, 0, 2)


def brute(q, k, v, frame_seg):
    """The Stage-1 weight formula, one query token at a time, summing over
    every key token with the indicator written out."""
    _, T, H, W, NH, D = q.shape
    toks = [(t, y, x) for t in range(T) for y in range(H) for x in range(W)]
    out = np.zeros_like(q)
    for (t, y, x) in toks:
        for h in range(NH):
            num = np.zeros(D)
            den = 0.0
            for (t2, y2, x2) in toks:
                same = 1.0 if frame_seg[t] == frame_seg[t2] else 0.0
                wgt = math.exp(float(q[0, t, y, x, h] @ k[0, t2, y2, x2, h]) / math.sqrt(D)) * same
                num += wgt * v[0, t2, y2, x2, h]
                den += wgt
            out[0, t, y, x, h] = num / den
    return out


@pytest.mark.parametrize("seg", [[0, 0, 1, 2], [0, 1, 0, 1], [7, 7, 7, 3], [0, 1, 2, 3]])
def test_segment_attention_matches_brute_force(seg):
    q, k, v = inputs()
    got = O.segment_attention(q, k, v, seg)
    assert np.allclose(got, brute(q, k, v, seg), rtol=0, atol=1e-12)


def test_one_segment_is_plain_sdpa():
    q, k, v = inputs(T=6, H=8, W=8, NH=3, D=16)
    got = O.segment_attention(q, k, v, [5] * 6)
    L = 6 * 64
    exp = sdpa(*(x.reshape(L, 3, 16) for x in (q, k, v))).reshape(q.shape)
    assert np.allclose(got, exp, rtol=0, atol=1e-12)


def test_every_frame_its_own_segment_is_per_frame_sdpa():
    q, k, v = inputs(T=4, H=8, W=8, NH=2, D=16)
    got = O.segment_attention(q, k, v, [0, 1, 2, 3])
    for t in range(4):
        exp = sdpa(*(x[0, t].reshape(64, 2, 16) for x in (q, k, v))).reshape(8, 8, 2, 16)
        assert np.allclose(got[0, t], exp, rtol=0, atol=1e-12)


def test_video_plus_images_splits_into_independent_sdpa():
    """A 5-frame video and three one-frame images: each part equals SDPA
    over its own frames alone."""
    q, k, v = inputs(T=8, H=8, W=8, NH=2, D=16)
    seg = [0, 0, 0, 0, 0, 1, 2, 3]
    got = O.segment_attention(q, k, v, seg)
    for lo, hi in [(0, 5), (5, 6), (6, 7), (7, 8)]:
        n = (hi - lo) * 64
        exp = sdpa(*(x[0, lo:hi].reshape(n, 2, 16) for x in (q, k, v)))
        assert np.allclose(got[0, lo:hi].reshape(n, 2, 16), exp, rtol=0, atol=1e-12)


def test_relabelling_segments_changes_nothing():
    q, k, v = inputs(T=6)
    a = O.segment_attention(q, k, v, [0, 0, 1, 1, 2, 3])
    b = O.segment_attention(q, k, v, [9, 9, -4, -4, 17, 0])
    assert np.array_equal(a, b)


def test_constant_values_give_constant_output():
    q, k, v = inputs(T=4)
    v = np.full_like(v, -0.625)
    got = O.segment_attention(q, k, v, [0, 1, 1, 2])
    assert np.allclose(got, -0.625, rtol=0, atol=1e-14)


def test_query_subset_equals_full_rows():
    q, k, v = inputs(T=4, H=8, W=8)
    seg = [0, 0, 1, 2]
    full = O.segment_attention(q, k, v, seg)
    qs = [(0, 0, 1, 2), (0, 2, 7, 7), (0, 3, 0, 5), (0, 1, 4, 4)]
    sub = O.segment_attention(q, k, v, seg, queries=qs)
    for r, (b, t, y, x) in enumerate(qs):
        assert np.allclose(sub[r], full[b, t, y, x], rtol=0, atol=1e-13)


def test_bad_segment_array_is_refused():
    q, k, v = inputs(T=4)
    with pytest.raises(ValueError):
        O.segment_attention(q, k, v, [0, 0, 1])


# ------------------------------------------------------------ planted mistakes

def planted(old: str, new: str):
    """A copy of the oracle's segment_attention with one textual mistake."""
    src = inspect.getsource(O.segment_attention)
    assert old in src
    ns = dict(vars(O))
    exec(src.replace(old, new), ns)
    return ns["segment_attention"]


@pytest.mark.parametrize("old,new", [
    ("np.repeat(seg, H * W)", "np.tile(seg, H * W)"),                  # wrong token -> frame map
    ("np.nonzero(tok_seg == sg)[0]", "np.arange(L)"),                  # mask dropped
    ("kt[b, keys, h].T) * scale", "kt[b, keys, h].T)"),                # scale dropped
    ("@ vt[b, keys, h]", "@ kt[b, keys, h]"),                          # K in place of V
])
def test_planted_mistakes_are_caught(old, new):
    q, k, v = inputs(T=4, H=4, W=4, D=4)
    seg = [0, 0, 1, 2]
    bad = planted(old, new)(q, k, v, seg)
    assert not np.allclose(bad, brute(q, k, v, seg), rtol=0, atol=1e-6)
