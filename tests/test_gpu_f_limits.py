"""GPU parity at the interface's declared maxima.

A streaming step whose ring holds LCSA_MAX_SLOTS = 16 temporal blocks (15
cached + the new one) on a 16 x 16 block grid with a window spanning the
grid, so every query row has exactly LCSA_MAX_CANDIDATES = 4096 candidates
(the row-group draft at its largest score buffer). k = 1/64 of them = 64.
Selections on every row, outputs on sampled rows, against the oracle.

The dense draft paths at their largest view: 12 temporal blocks of a 16 x 12
block grid under a window spanning it give 2,304 candidates per row, the
most the fused kernel's LDS rows and the split selection's per-lane registers
(36 scores a lane) take; both forms are compared with the oracle.
"""
from __future__ import annotations

import pytest

from block_sparse_attention_03_amd import lcsa as L
from block_sparse_attention_03_amd.workloads import Workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_harness import Stream, compare_step, sample_rows, say  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load_library()
    return torch.device("cuda:0")


def test_max_slots_and_max_candidates(dev):
    assert L.MAX_SLOTS == 16 and L.MAX_CANDIDATES == 4096
    w = Workload(name="limits: 16-slot ring, 4096 candidates per row", heads=2, head_dim=64,
                 dtype="bf16", height=128, width=128, frames=2, cache_frames=30, cap_tb=15,
                 local_range=17, ratio=(1, 64), seed=4096)
    assert w.n_slots == 16
    st = Stream(w, dev)
    rows = sample_rows(w, 6)
    g, ref = st.step(rows=rows, want_probs=False)
    assert set(int(x) for x in ref.kcount) == {64}
    assert int(ref.allowed.sum(axis=1).max()) == 4096
    stats = compare_step(w, g, ref, rows=rows, check_probs=False)
    slots, tbs = st.gcache.view()
    assert tbs == list(range(1, 16))  # after eviction the newest 15 TBs remain
    say(f"limits: {stats}")


@pytest.mark.parametrize("split", [False, True], ids=["fused", "split"])
def test_dense_draft_at_its_largest_view(dev, split):
    w = Workload(name="dense draft limit: 2,304 candidates per row", heads=2, head_dim=64,
                 dtype="bf16", height=128, width=96, frames=2, cache_frames=22, cap_tb=11,
                 local_range=17, ratio=(1, 16), seed=2304)
    st = Stream(w, dev, draft_ws=split)
    rows = sample_rows(w, 4)
    g, ref = st.step(rows=rows, want_probs=False)
    assert int(ref.allowed.sum(axis=1).max()) == 2304
    assert set(int(x) for x in ref.kcount) == {144}
    stats = compare_step(w, g, ref, rows=rows, check_probs=False)
    say(f"dense draft at 2,304 candidates ({'split' if split else 'fused'}): {stats}")
