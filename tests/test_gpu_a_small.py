"""GPU parity on small inputs and edge cases (runs first: cheap, every row).

The HIP path through the C-ABI against the float64 oracle.

Every case runs on the GPU and in the oracle from the same seeded inputs.
Selections are compared on every row (exact, or the tie rule for rows whose
k-th and (k+1)-th scores are within 1e-5 relative); outputs element by
element on every row for small cases and on sampled rows at the full
workload sizes (the oracle computes those rows one by one).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import pytest

from block_sparse_attention_03_amd import lcsa as L
from block_sparse_attention_03_amd import synth
from block_sparse_attention_03_amd.workloads import WORKLOADS, Workload
from oracle import lcsa_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_harness import (Stream, compare_step, lib_params, sample_rows, say, to_dev,  # noqa: E402
                         to_host64)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load_library()
    return torch.device("cuda:0")


def small(**kw) -> Workload:
    base = dict(name="small", heads=2, head_dim=128, dtype="bf16", height=40, width=56,
                frames=4, cache_frames=0, cap_tb=3, local_range=3, ratio=(1, 3), seed=77)
    base.update(kw)
    return Workload(**base)


def check_layouts(st: Stream, g, ref):
    """Partition outputs: q blocks (when the step wrote them) and the ring's
    K / V^T blocks, bitwise."""
    if g["q_blk"] is not None:
        assert np.array_equal(to_host64(g["q_blk"]), ref.q_blocks)
    kb, vb = ref.key_blocks
    slots, _ = st.gcache.view()  # after eviction; compare the blocks still held
    nS = st.w.nS
    n_view = kb.shape[2] // nS
    held = len(slots)
    kr = to_host64(st.gcache.k_ring)
    vr = to_host64(st.gcache.v_ring)
    for pos in range(held):
        src = n_view - held + pos  # the newest TBs of the step's view are still held
        for s in range(nS):
            assert np.array_equal(kr[:, :, slots[pos], s], kb[:, :, src * nS + s])
            assert np.array_equal(vr[:, :, slots[pos], s], np.swapaxes(vb[:, :, src * nS + s], -1, -2))


# ------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("case", [
    dict(),                                                   # multi-tile, ragged 5x7 grid
    dict(border=1),                                           # Boundary-Truncated
    dict(ratio=(1, 1), local_range=99),                       # k = all, unbounded window
    dict(topk_fixed=1),                                       # one block per row
    dict(head_dim=64),
    dict(dtype="f32"),
    dict(dtype="f32", head_dim=64, topk_fixed=2),
    dict(batch=2, heads=3),
    dict(height=8, width=8, frames=6, topk_fixed=2),          # 1x1 block grid
    dict(local_range=1, frames=6),                            # window = own column only
    dict(ratio=(2, 7)),
    dict(ratio=(1, 5), ratio_base=1, frames=6),               # ratio of all key blocks
])
def test_small_cases_all_rows(dev, case):
    w = small(**case)
    st = Stream(w, dev)
    g, ref = st.step()
    check_layouts(st, g, ref)
    stats = compare_step(w, g, ref)
    say(f"small {case}: {stats}")


@pytest.mark.parametrize("kw", [dict(), dict(head_dim=64), dict(dtype="f32")],
                         ids=["bf16-d128", "bf16-d64", "f32-d128"])
def test_token_and_block_q_paths_agree(dev, kw):
    """q read in token layout (the partition writes only q's means) and q read
    from q_blk give bitwise the same lists, pooled q, outputs and lse, step
    after step; the block path's q_blk matches the oracle's partition bitwise
    and both match the oracle's attention."""
    w = small(frames=2, cache_frames=6, cap_tb=3, local_range=5, ratio=(1, 4), **kw)
    tok = Stream(w, dev)
    blk = Stream(w, dev, q_blocks=True)
    for n in range(3):
        g1, ref1 = tok.step(want_probs=False)
        g2, ref2 = blk.step(want_probs=False)
        assert g1["q_blk"] is None and g2["q_blk"] is not None
        for key in ("sel_idx", "sel_cnt", "lse", "q_pool"):
            assert np.array_equal(g1[key], g2[key]), key
        assert torch.equal(g1["out"], g2["out"])
        check_layouts(blk, g2, ref2)
        compare_step(w, g1, ref1)
        stats = compare_step(w, g2, ref2)
    say(f"token vs block q: {stats}")


@pytest.mark.parametrize("kw,local", [(dict(), False), (dict(head_dim=64), False),
                                      (dict(dtype="f32"), False), (dict(local_range=3), True)],
                         ids=["bf16-d128", "bf16-d64", "f32-d128", "local-lists"])
def test_pipelined_steps_match_sequential(dev, kw, local):
    """StepPipeline (partition and lists of step n + 1 on a side stream under
    the attention of step n, a ring with one extra slot) gives bitwise the
    lists, outputs and lse of sequential run_step calls, step after step."""
    w = small(**{**dict(frames=2, cache_frames=6, cap_tb=3, local_range=5, ratio=(1, 4)), **kw})
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = L.LCSA_BF16 if w.dtype == "bf16" else L.LCSA_F32
    n_tb = w.frames // 2
    n_steps = 5
    d = synth.make_qkv(w.seed, w.heads, w.head_dim, w.height, w.width, 0,
                       w.cache_frames + n_steps * w.frames, dtype=w.dtype)
    q, k, v = (to_dev(d[n][0], w.dtype, dev) for n in "qkv")
    geom = L.make_geom(1, w.heads, w.head_dim, w.frames, w.height, w.width, code)
    gprime = L.make_geom(1, w.heads, w.head_dim, w.cache_frames, w.height, w.width, code)
    params = lib_params(w)
    caches = []
    for extra in (0, 1):  # the sequential ring, and one slot more for the pipeline
        c = L.KVCache(1, w.heads, w.head_dim, w.height, w.width, tdt,
                      w.cap_tb + n_tb + extra, device=dev)
        first = c.append(w.cache_frames // 2, 0)
        L.lcsa_partition_pool(gprime, None, k[:, :w.cache_frames], v[:, :w.cache_frames],
                              None, None, c.c, first)
        caches.append(c)
    torch.cuda.synchronize()
    seq = []
    for n in range(n_steps):
        f0 = w.cache_frames + n * w.frames
        sl = slice(f0, f0 + w.frames)
        b = L.run_step(geom, q[:, sl], k[:, sl], v[:, sl], caches[0], f0 // 2, params,
                       keep_tb=w.cap_tb, want_lse=True, local=local)
        seq.append({kk: getattr(b, kk).clone() for kk in ("sel_idx", "sel_cnt", "out", "lse")})
    torch.cuda.synchronize()
    kmax = seq[0]["sel_idx"].shape[-1]  # every step's row has the same candidate count
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    pipe = L.StepPipeline(geom, caches[1], params, kmax, main, side, local=local, with_lse=True,
                          device=dev)
    got = []
    for n in range(n_steps):
        f0 = w.cache_frames + n * w.frames
        sl = slice(f0, f0 + w.frames)
        pipe.prep(q[:, sl], k[:, sl], v[:, sl], f0 // 2)
        b = pipe.attend(w.cap_tb)
        got.append({kk: getattr(b, kk).clone() for kk in ("sel_idx", "sel_cnt", "out", "lse")})
    torch.cuda.synchronize()
    for n in range(n_steps):
        for kk in ("sel_idx", "sel_cnt", "out", "lse"):
            assert torch.equal(seq[n][kk], got[n][kk]), (n, kk)
    say(f"pipelined == sequential over {n_steps} steps ({w.dtype}, D {w.head_dim}, local {local})")


def test_small_streaming_with_cache(dev):
    w = small(frames=2, cache_frames=6, cap_tb=3, local_range=5, ratio=(1, 4))
    st = Stream(w, dev)
    for n in range(5):
        g, ref = st.step()
        stats = compare_step(w, g, ref)
    say(f"small stream: {stats}")


@pytest.mark.parametrize("kw", [dict(), dict(head_dim=64), dict(dtype="f32")],
                         ids=["bf16-d128", "bf16-d64", "f32-d128"])
def test_two_stream_partition_matches_one_stream(dev, kw):
    """The transposed-v part of the partition on a second stream (forked after
    the previous step, joined before the attention) gives bitwise the same
    lists, outputs, pooled q and ring contents as the one-stream step, step
    after step while ring slots are reused, and matches the oracle."""
    w = small(frames=2, cache_frames=6, cap_tb=3, local_range=5, ratio=(1, 4), **kw)
    one = Stream(w, dev)
    two = Stream(w, dev, side_stream=torch.cuda.Stream())
    for n in range(4):
        g1, _ = one.step(want_probs=False)
        g2, ref = two.step(want_probs=False)
        for key in ("sel_idx", "sel_cnt", "lse", "q_pool"):
            assert np.array_equal(g1[key], g2[key]), key
        assert torch.equal(g1["out"], g2["out"])
        slots, _ = two.gcache.view()
        assert slots == one.gcache.view()[0]
        for sl in slots:  # the blocks the caches hold (other slots were never written)
            for ring in ("k_ring", "v_ring", "kpool_ring"):
                assert torch.equal(getattr(one.gcache, ring)[:, :, sl],
                                   getattr(two.gcache, ring)[:, :, sl]), (ring, sl)
        check_layouts(two, g2, ref)
        stats = compare_step(w, g2, ref)
    say(f"two-stream partition: {stats}")


@pytest.mark.parametrize("q_scale", [16.0, 64.0])
def test_large_logits(dev, q_scale):
    """q scaled by a power of two (exact in bf16): logits of tens to hundreds,
    so the running row max jumps by far more than the lazy-rescale threshold,
    most probabilities underflow to zero and the softmax is sharply peaked;
    outputs and lse still match the oracle."""
    w = small(frames=2, cache_frames=6, cap_tb=3, local_range=5, ratio=(1, 4))
    st = Stream(w, dev, q_scale=q_scale)
    for n in range(2):
        g, ref = st.step(want_probs=False)
        assert np.isfinite(g["lse"]).all()
        stats = compare_step(w, g, ref)
    say(f"large logits x{q_scale}: {stats}")


def test_equal_scores_take_lowest_ids(dev):
    """q = 0: every draft score is exactly 0, so the selection is the k lowest
    logical ids on both sides (ties broken by index), and the output is the
    mean of V over the selected tokens."""
    w = small(frames=4, ratio=(1, 3))
    st = Stream(w, dev, zero_q=True)
    g, ref = st.step()
    for h in range(w.heads):
        for i in range(w.nq):
            k = int(ref.kcount[i])
            cand = np.nonzero(np.isfinite(ref.scores[0, h, i]))[0][:k]
            assert list(g["sel_idx"][0, h, i, :k]) == list(cand)
    compare_step(w, g, ref)


def test_rows_without_candidates_are_zero(dev):
    """Queries older than every cached block have no candidates: k = 0, an
    empty list, output 0 and lse = -inf."""
    w = small(frames=2)
    code = L.LCSA_BF16
    cache = L.KVCache(1, w.heads, w.head_dim, w.height, w.width, torch.bfloat16, 4, device=dev)
    d = synth.make_qkv(3, w.heads, w.head_dim, w.height, w.width, 6, 10, dtype="bf16")
    first = cache.append(2, 3)
    geom_kv = L.make_geom(1, w.heads, w.head_dim, 4, w.height, w.width, code)
    L.lcsa_partition_pool(geom_kv, None, to_dev(d["k"][0], "bf16", dev), to_dev(d["v"][0], "bf16", dev),
                          None, None, cache.c, first)
    geom = L.make_geom(1, w.heads, w.head_dim, 2, w.height, w.width, code)
    params = L.make_params(local_range=3, ratio=(1, 3))
    bufs = L.StepBuffers(geom, 4, device=dev, with_lse=True, with_q_blk=True)
    qd = synth.make_qkv(3, w.heads, w.head_dim, w.height, w.width, 2, 4, dtype="bf16", which="q")
    q = to_dev(qd["q"][0], "bf16", dev)
    # partition q only through a scratch cache slot is not possible; use a
    # second cache for the query chunk's own k/v, then draft against `cache`
    c2 = L.KVCache(1, w.heads, w.head_dim, w.height, w.width, torch.bfloat16, 1, device=dev)
    s2 = c2.append(1, 1)
    L.lcsa_partition_pool(geom, q, q, q, bufs.q_blk, bufs.q_pool, c2.c, s2)
    L.lcsa_draft_mask(geom, bufs.q_pool, 1, cache.c, params, bufs.kmax, bufs.sel_idx, bufs.sel_cnt)
    L.lcsa_block_sparse_attn(geom, bufs.q_blk, cache.c, bufs.sel_idx, bufs.sel_cnt, bufs.kmax,
                             bufs.out, bufs.lse)
    torch.cuda.synchronize()
    assert int(bufs.sel_cnt.abs().sum()) == 0
    assert bool((bufs.sel_idx == -1).all())
    assert float(bufs.out.float().abs().max()) == 0.0
    assert bool(torch.isinf(bufs.lse).all()) and bool((bufs.lse < 0).all())


def test_empty_chunk_enqueues_nothing(dev):
    geom = L.make_geom(1, 2, 128, 0, 16, 16, L.LCSA_BF16)
    cache = L.KVCache(1, 2, 128, 16, 16, torch.bfloat16, 2, device=dev)
    cache.append(1, 0)
    t = torch.empty(16, device=dev)
    L.lcsa_partition_pool(geom, t, t, t, t, t, cache.c, 0)
    L.lcsa_draft_mask(geom, t, 0, cache.c, L.make_params(), 1, t, t)
    L.lcsa_block_sparse_attn(geom, t, cache.c, t, t, 1, t)
    torch.cuda.synchronize()


def test_bitwise_deterministic_reruns(dev):
    """Negative control: the same step run twice gives identical bits."""
    outs = []
    for _ in range(2):
        st = Stream(small(frames=2, cache_frames=4, cap_tb=2), dev)
        g, _ = st.step(rows=[(0, 0, 0)])
        outs.append((g["out"].view(torch.int16).cpu().numpy(), g["sel_idx"].copy(), g["lse"].copy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_corrupted_index_fails_the_check(dev):
    """Positive control: replacing one selected block by another candidate
    must make the output comparison fail for that row."""
    w = small(frames=2, cache_frames=4, cap_tb=2, ratio=(1, 4))
    st = Stream(w, dev)
    g, ref = st.step()
    b, h, i = 0, 1, 3
    k = int(ref.kcount[i])
    sel = list(g["sel_idx"][b, h, i, :k])
    cand = [j for j in np.nonzero(np.isfinite(ref.scores[b, h, i]))[0] if j not in sel]
    bad = sel.copy()
    bad[0] = int(cand[0])
    kb, vb = ref.key_blocks
    o_good, _ = O.sparse_attention_row(ref.q_blocks[b, h, i], kb[b, h], vb[b, h], np.array(sorted(sel)),
                                       1 / math.sqrt(w.head_dim))
    o_bad, _ = O.sparse_attention_row(ref.q_blocks[b, h, i], kb[b, h], vb[b, h], np.array(sorted(bad)),
                                      1 / math.sqrt(w.head_dim))
    got = O.partition(to_host64(g["out"]))[b, h, i]
    from parity_util import assert_close
    assert_close(got, o_good, w.dtype)
    with pytest.raises(AssertionError):
        assert_close(got, o_bad, w.dtype)
