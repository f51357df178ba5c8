"""GPU parity at the five workload sizes.

The HIP path through the C-ABI against the float64 oracle.

Every case runs on the GPU and in the oracle from the same seeded inputs.
Selections are compared on every row (exact, or the tie rule for rows whose
k-th and (k+1)-th scores are within 1e-5 relative); outputs element by
element on every row of every head for one step of each of the four
full-size workloads, and on sampled rows for the further steps of a stream
(the oracle computes those rows one by one).
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

from gpu_harness import Stream, compare_step, sample_rows, say, to_dev, to_host64  # noqa: E402


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


# ------------------------------------------------------------------ workloads

def test_tiny_fp32_all_rows(dev):
    w = WORKLOADS["tiny"]
    st = Stream(w, dev)
    g, ref = st.step()
    check_layouts(st, g, ref)
    stats = compare_step(w, g, ref)
    say(f"tiny: {stats}")


@pytest.mark.parametrize("want_probs", [True, False], ids=["with-probs", "whole-grid-path"])
def test_cold_start_768x1408_every_row(dev, want_probs):
    """The 11x11 window covers the 6x11 block grid. With the probabilities
    output the draft scores row groups on the vector ALU; without it, the
    whole-grid path (16 rows per workgroup on the fp64 matrix cores)."""
    w = WORKLOADS["cold_768x1408"]
    st = Stream(w, dev)
    g, ref = st.step(want_probs=want_probs)
    assert sorted(set(int(x) for x in ref.kcount)) == [13, 26, 39]
    stats = compare_step(w, g, ref)
    assert stats["rows"] == w.heads * w.nq
    say(f"cold 768x1408 ({'probs' if want_probs else 'no probs'}), every row of 12 heads: {stats}")


def test_streaming_step_768x1408_every_row(dev):
    """The first step every row of all 12 heads, two more on sampled rows."""
    w = WORKLOADS["step_768x1408"]
    st = Stream(w, dev)
    for n in range(3):
        rows = "all" if n == 0 else sample_rows(w, 6, rng_seed=n)
        g, ref = st.step(rows=rows)
        assert set(int(x) for x in ref.kcount) == {52}
        stats = compare_step(w, g, ref, rows=rows)
        say(f"step {n} 768x1408: {stats}")


def test_streaming_100_steps_768x1408_12_heads(dev):
    """100 consecutive steps of the 768x1408 stream at its 12 heads: every
    selection of every step (tie rule), outputs on sampled rows of every
    head, and the ring holding exactly the last 3 TBs after each step."""
    w = dataclasses.replace(WORKLOADS["step_768x1408"], seed=4242)
    st = Stream(w, dev)
    tied = 0
    for n in range(100):
        rows = sample_rows(w, 3, rng_seed=n)
        g, ref = st.step(rows=rows, want_probs=False)
        stats = compare_step(w, g, ref, rows=rows, check_probs=False)
        tied += stats["tied"]
        slots, tbs = st.gcache.view()
        assert tbs == [n + 1, n + 2, n + 3] and st.ocache.tbs() == tbs
    say(f"100 steps x 12 heads ok, tied rows {tied}")


@pytest.mark.parametrize("name", ["step_1536x2688", "step_4k"])
def test_streaming_step_large_every_row(dev, name):
    w = WORKLOADS[name]
    st = Stream(w, dev)
    g, ref = st.step(want_probs=False)
    assert set(int(x) for x in ref.kcount) == {23 if name == "step_1536x2688" else 11}
    stats = compare_step(w, g, ref, check_probs=False)
    assert stats["rows"] == w.heads * w.nq
    say(f"{name}, every row of 12 heads: {stats}")




def test_long_t_parallel_forward_768x1280(dev):
    """The parallel training-shape forward: 24 latent frames (12 TBs) at once,
    every query block over its own and all earlier TBs. Selections on every
    row; outputs on rows from the first, a middle and the last TB of every
    head (list lengths 12 to 144 blocks)."""
    w = WORKLOADS["longT_768x1280"]
    st = Stream(w, dev)
    nS = w.nS
    rows = [(0, h, i) for h in range(w.heads)
            for i in (0, nS + 1, 5 * nS + 7, 11 * nS, 11 * nS + nS - 1)]
    g, ref = st.step(rows=rows, want_probs=False)
    assert sorted(set(int(x) for x in ref.kcount)) == [12 * (t + 1) for t in range(12)]
    stats = compare_step(w, g, ref, rows=rows, check_probs=False)
    say(f"long-T 768x1280: {stats}")
