"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
and its host-only logic (ring metadata, k rule, argument validation) behaves
as include/lcsa.h states. No device work is enqueued: every call here either
is host-only or fails validation before its first HIP call."""
from __future__ import annotations

import ctypes
import json
import os
import re

import pytest

from block_sparse_attention_03_amd import lcsa as L
from block_sparse_attention_03_amd.workloads import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def lib():
    return L.load_library()


def declared_functions():
    text = open(L.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lcsa_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert lib.lcsa_abi_version() == 5


FAKE = 0x10000  # aligned, never dereferenced: validation fails first


def ring_bytes(nby, nbx, heads, D, dtype, n_slots, batch=1):
    """Bytes of the K (= V) ring and of the pooled-K ring, as include/lcsa.h sizes them."""
    blocks = batch * heads * n_slots * nby * nbx
    return blocks * 128 * D * (2 if dtype == L.LCSA_BF16 else 4), blocks * D * 8


def fake_cache(nby=6, nbx=11, heads=12, D=128, dtype=L.LCSA_BF16, n_slots=4):
    c = L.KvCacheStruct()
    kv, pool = ring_bytes(nby, nbx, heads, D, dtype, n_slots)
    L.lcsa_kv_cache_init(c, 1, heads, D, nby, nbx, dtype, n_slots,
                         type("P", (), {"data_ptr": lambda s: FAKE})(),
                         type("P", (), {"data_ptr": lambda s: FAKE * 2})(),
                         type("P", (), {"data_ptr": lambda s: FAKE * 3})(), kv, kv, pool)
    return c


def test_ring_init_refuses_undersized_buffers(lib):
    """lcsa_kv_cache_init takes the ring buffers' sizes and refuses any
    smaller than n_slots slots need (LCSA_ERR_CAPACITY), before the partition
    could write past them ([HW] "How FlashVSR works" 2.3: the cache of past
    segments the ring holds)."""
    for dtype, D in ((L.LCSA_BF16, 128), (L.LCSA_F32, 64)):
        kv, pool = ring_bytes(6, 11, 3, D, dtype, 4, batch=2)
        P = lambda a: type("P", (), {"data_ptr": lambda s: a})()
        for sizes in ((kv - 1, kv, pool), (kv, kv - 1, pool), (kv, kv, pool - 1), (0, 0, 0)):
            c = L.KvCacheStruct()
            with pytest.raises(L.LcsaError) as e:
                L.lcsa_kv_cache_init(c, 2, 3, D, 6, 11, dtype, 4, P(FAKE), P(FAKE), P(FAKE), *sizes)
            assert e.value.status == 6, sizes
            assert "too small" in str(e.value)
        c = L.KvCacheStruct()
        L.lcsa_kv_cache_init(c, 2, 3, D, 6, 11, dtype, 4, P(FAKE), P(FAKE), P(FAKE), kv, kv, pool)
        assert c.n_slots == 4 and c.count == 0


def test_ring_append_evict_view_wraps(lib):
    c = fake_cache(n_slots=4)
    assert L.lcsa_kv_cache_view(c) == ([], [])
    assert L.lcsa_kv_cache_append(c, 3, 0) == 0
    assert L.lcsa_kv_cache_view(c) == ([0, 1, 2], [0, 1, 2])
    for step in range(3, 12):
        slot = L.lcsa_kv_cache_append(c, 1, step)
        assert slot == step % 4
        slots, tbs = L.lcsa_kv_cache_view(c)
        assert tbs == [step - 3, step - 2, step - 1, step]
        assert slots == [t % 4 for t in tbs]
        L.lcsa_kv_cache_evict(c, 3)
        assert L.lcsa_kv_cache_view(c)[1] == [step - 2, step - 1, step]


def test_ring_capacity_and_order_errors(lib):
    c = fake_cache(n_slots=4)
    L.lcsa_kv_cache_append(c, 4, 10)
    with pytest.raises(L.LcsaError) as e:
        L.lcsa_kv_cache_append(c, 1, 14)
    assert e.value.status == 6
    L.lcsa_kv_cache_evict(c, 2)
    with pytest.raises(L.LcsaError) as e:
        L.lcsa_kv_cache_append(c, 1, 13)          # not newer than TB 13
    assert e.value.status == 4
    with pytest.raises(L.LcsaError):
        L.lcsa_kv_cache_evict(c, -1)
    L.lcsa_kv_cache_evict(c, 0)
    assert L.lcsa_kv_cache_view(c) == ([], [])
    L.lcsa_kv_cache_evict(c, 5)                   # keeping more than held is a no-op
    with pytest.raises(L.LcsaError):
        bad = L.KvCacheStruct()
        L.lcsa_kv_cache_init(bad, 1, 1, 128, 2, 2, L.LCSA_BF16, 17, None, None, None, 0, 0, 0)


def test_topk_count_matches_hand_table(lib):
    g = json.load(open(os.path.join(GOLDEN, "k_table.json")))
    for case in g["k_rows"]:
        if "topk_fixed" in case:
            p = L.make_params(topk_fixed=case["topk_fixed"])
        else:
            p = L.make_params(ratio=tuple(case["ratio"]), scale_by_resolution=case["scale"],
                              out_hw=tuple(case.get("out", (768, 1280))))
        for n, k in zip(case["n_allowed"], case["k"]):
            assert L.lcsa_topk_count(p, n, 10 ** 6) == k, case["name"]
    assert L.lcsa_topk_count(L.make_params(), 0, 10) == 0


@pytest.mark.parametrize("wl,k", [("cold_768x1408", 39), ("step_768x1408", 52),
                                  ("step_1536x2688", 23), ("step_4k", 11), ("tiny", 3)])
def test_max_topk_of_workloads(lib, wl, k):
    w = WORKLOADS[wl]
    c = fake_cache(w.height // 8, w.width // 8, w.heads, w.head_dim,
                   L.LCSA_BF16 if w.dtype == "bf16" else L.LCSA_F32, w.n_slots)
    L.lcsa_kv_cache_append(c, w.n_slots, 0)
    geom = L.make_geom(1, w.heads, w.head_dim, w.frames, w.height, w.width, c.dtype)
    p = L.make_params(local_range=w.local_range, topk_fixed=w.topk_fixed, ratio=w.ratio,
                      scale_by_resolution=w.scale_by_resolution, out_hw=w.out_hw)
    first = w.cache_frames // 2
    assert L.lcsa_max_topk(geom, first, c, p) == k


class _P:
    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def expect(status, fn, *args, **kw):
    with pytest.raises(L.LcsaError) as e:
        fn(*args, **kw)
    assert e.value.status == status, str(e.value)
    return str(e.value)


def test_validation_rejects_bad_input_before_any_device_call(lib):
    c = fake_cache()
    L.lcsa_kv_cache_append(c, 1, 0)
    ok = _P(FAKE)
    geom = L.make_geom(1, 12, 128, 2, 48, 88, L.LCSA_BF16)
    s = 0  # stream handle, never used
    # shapes
    expect(2, L.lcsa_partition_pool, L.make_geom(1, 12, 128, 3, 48, 88, 0), ok, ok, ok, ok, ok, c, 0, s)
    expect(2, L.lcsa_partition_pool, L.make_geom(1, 12, 128, 2, 44, 88, 0), ok, ok, ok, ok, ok, c, 0, s)
    expect(2, L.lcsa_partition_pool, L.make_geom(1, 12, 96, 2, 48, 88, 0), ok, ok, ok, ok, ok, c, 0, s)
    expect(2, L.lcsa_partition_pool, L.make_geom(1, 12, 128, 2, 48, 96, 0), ok, ok, ok, ok, ok, c, 0, s)
    expect(3, L.lcsa_partition_pool, L.make_geom(1, 12, 128, 2, 48, 88, 1), ok, ok, ok, ok, ok, c, 0, s)
    expect(3, L.lcsa_partition_pool, L.make_geom(1, 12, 128, 2, 48, 88, 7), ok, ok, ok, ok, ok, c, 0, s)
    # pointers
    expect(1, L.lcsa_partition_pool, geom, ok, None, ok, ok, ok, c, 0, s)
    expect(1, L.lcsa_partition_pool, geom, ok, ok, ok, ok, None, c, 0, s)   # q_pool missing
    expect(5, L.lcsa_partition_pool, geom, _P(FAKE + 8), ok, ok, ok, ok, c, 0, s)
    # the chunk's TBs must be the newest held, from the slot the last append returned
    expect(4, L.lcsa_partition_pool, geom, ok, ok, ok, ok, ok, c, 2, s)
    expect(4, L.lcsa_partition_pool, geom, ok, ok, ok, ok, ok, c, 9, s)
    # selection parameters
    expect(4, L.lcsa_draft_mask, geom, ok, 0, c, L.make_params(local_range=10), 64, ok, ok, None, s)
    expect(4, L.lcsa_draft_mask, geom, ok, 0, c, L.make_params(local_range=0), 64, ok, ok, None, s)
    expect(4, L.lcsa_draft_mask, geom, ok, 0, c, L.make_params(ratio=(0, 5)), 64, ok, ok, None, s)
    expect(4, L.lcsa_draft_mask, geom, ok, 0, c, L.make_params(ratio=(1, -5)), 64, ok, ok, None, s)
    expect(4, L.lcsa_draft_mask, geom, ok, 0, c, L.make_params(border=2), 64, ok, ok, None, s)
    expect(4, L.lcsa_draft_mask, geom, ok, 0, c,
           L.make_params(scale_by_resolution=True, out_hw=(0, 1280)), 64, ok, ok, None, s)
    # kmax too small (k = 13 for one visible TB of 66 candidates)
    msg = expect(6, L.lcsa_draft_mask, geom, ok, 0, c, L.make_params(), 12, ok, ok, None, s)
    assert "13" in msg
    expect(5, L.lcsa_draft_mask, geom, ok, 0, c, L.make_params(), 64, ok, ok, _P(FAKE + 4), s)
    # probs one double short of [B][NH][nq][n_keys]: 12 heads x 66 rows x 66 keys
    need = 12 * 66 * 66 * 8
    msg = expect(6, L.lcsa_draft_mask, geom, ok, 0, c, L.make_params(), 64, ok, ok, ok, s,
                 probs_bytes=need - 8)
    assert str(need) in msg
    # geometry disagrees with the cache
    expect(2, L.lcsa_draft_mask, L.make_geom(1, 8, 128, 2, 48, 88, 0), ok, 0, c, L.make_params(), 64,
           ok, ok, None, s)
    # attention
    expect(4, L.lcsa_block_sparse_attn, geom, ok, c, ok, ok, 13, ok, None, float("nan"), s)
    expect(4, L.lcsa_block_sparse_attn, geom, ok, c, ok, ok, 13, ok, None, -1.0, s)
    expect(6, L.lcsa_block_sparse_attn, geom, ok, c, ok, ok, 0, ok, None, 0.0, s)
    expect(1, L.lcsa_block_sparse_attn, geom, ok, c, None, ok, 13, ok, None, 0.0, s)
    expect(1, L.lcsa_block_sparse_attn, geom, None, c, ok, ok, 13, ok, None, 0.0, s)
    # the same checks with q in token layout
    A = L.lcsa_block_sparse_attn_tok
    expect(4, A, geom, ok, c, ok, ok, 13, ok, None, float("nan"), s)
    expect(6, A, geom, ok, c, ok, ok, 0, ok, None, 0.0, s)
    msg = expect(1, A, geom, None, c, ok, ok, 13, ok, None, 0.0, s)
    assert "q is NULL" in msg
    expect(5, A, geom, _P(FAKE + 8), c, ok, ok, 13, ok, None, 0.0, s)
    expect(2, A, L.make_geom(1, 8, 128, 2, 48, 88, 0), ok, c, ok, ok, 13, ok, None, 0.0, s)


def test_empty_chunk_is_a_no_op(lib):
    c = fake_cache()
    L.lcsa_kv_cache_append(c, 1, 0)
    ok = _P(FAKE)
    geom = L.make_geom(1, 12, 128, 0, 48, 88, L.LCSA_BF16)
    L.lcsa_partition_pool(geom, ok, ok, ok, ok, ok, c, 0, 0)
    L.lcsa_draft_mask(geom, ok, 0, c, L.make_params(), 1, ok, ok, None, 0)
    L.lcsa_block_sparse_attn(geom, ok, c, ok, ok, 1, ok, None, 0.0, 0)
    L.lcsa_block_sparse_attn_tok(geom, ok, c, ok, ok, 1, ok, None, 0.0, 0)
    L.lcsa_partition_pool(geom, ok, ok, ok, None, ok, c, 0, 0)  # q's means only
    assert L.lcsa_last_error() == ""


def test_draft_workspace_size_and_validation(lib):
    """The draft's workspace: sized for the split path at the cache's fullest
    occupancy (0 where no occupancy takes it), and refused when misaligned
    (LCSA_ERR_ALIGN) or too small (LCSA_ERR_CAPACITY) before any device call."""
    c = fake_cache(17, 30, 2, 128, L.LCSA_BF16, 4)  # the 4K grid: 510 blocks per TB
    geom = L.make_geom(1, 2, 128, 2, 136, 240, L.LCSA_BF16)
    glob = L.make_params(local_range=255, ratio=(1, 5))
    nb = L.lcsa_draft_workspace_size(geom, c, glob)
    assert nb == 2 * 510 * 2048 * 4  # 2 heads x 510 rows x 2,040 candidates padded to 2,048
    assert L.lcsa_draft_workspace_size(geom, c, L.make_params(local_range=11)) == 0
    small = fake_cache(6, 11, 2, 128, L.LCSA_BF16, 4)  # 264 candidates at most: other paths
    assert L.lcsa_draft_workspace_size(L.make_geom(1, 2, 128, 2, 48, 88, L.LCSA_BF16), small,
                                       glob) == 0
    assert lib.lcsa_draft_workspace_size(ctypes.byref(geom), ctypes.byref(c), ctypes.byref(glob),
                                         None) == 1
    L.lcsa_kv_cache_append(c, 4, 0)
    ok = _P(FAKE)
    kmax = L.lcsa_max_topk(geom, 3, c, glob)
    msg = expect(5, L.lcsa_draft_mask, geom, ok, 3, c, glob, kmax, ok, ok, None, 0,
                 workspace=_P(FAKE + 8), workspace_bytes=nb)
    assert "workspace" in msg
    msg = expect(6, L.lcsa_draft_mask, geom, ok, 3, c, glob, kmax, ok, ok, None, 0,
                 workspace=ok, workspace_bytes=nb - 1)
    assert "workspace" in msg


def test_too_many_candidates_is_refused(lib):
    # 16 TBs of a 17x30 grid with an unbounded window: 8160 candidates > 4096
    c = fake_cache(17, 30, 1, 128, L.LCSA_BF16, 16)
    L.lcsa_kv_cache_append(c, 16, 0)
    geom = L.make_geom(1, 1, 128, 2, 136, 240, L.LCSA_BF16)
    expect(6, L.lcsa_draft_mask, geom, _P(FAKE), 15, c, L.make_params(local_range=99, topk_fixed=1),
           4096, _P(FAKE), _P(FAKE), None, 0)


# ------------------------------------------------------------ Stage-1 segments

@pytest.mark.parametrize("seg,T,expect_tbs", [
    ([0] * 23 + [1], 24, 12),              # 23-frame video + one image: the video spans all TBs
    ([0, 0, 0, 0, 0, 1, 2, 3], 8, 3),      # 5-frame video + 3 images: TB 0..2 share the video
    ([0, 1, 2, 3, 4, 5], 6, 1),            # every frame its own segment: a TB lists itself
    ([0, 1, 0, 1], 4, 2),                  # interleaved ids: both TBs share both segments
    ([4] * 8, 8, 4),                       # one segment: every TB
])
def test_segment_max_list(lib, seg, T, expect_tbs):
    g = L.make_geom(1, 2, 128, T, 48, 80, L.LCSA_BF16)
    assert L.lcsa_segment_max_list(g, seg) == expect_tbs * 60


def test_segment_validation_before_any_device_call(lib):
    g = L.make_geom(1, 2, 128, 8, 48, 80, L.LCSA_BF16)
    seg = [0, 0, 0, 0, 0, 1, 2, 3]
    P = type("P", (), {"data_ptr": lambda s: FAKE})()
    c = fake_cache(nby=6, nbx=10, heads=2, n_slots=4)
    # the cache does not yet hold the chunk
    with pytest.raises(L.LcsaError, match="LCSA_ERR_PARAM"):
        L.lcsa_segment_lists(g, 0, c, seg, 180, P, P, stream=0)
    L.lcsa_kv_cache_append(c, 4, 10)
    with pytest.raises(L.LcsaError, match="LCSA_ERR_PARAM"):   # chunk starts at TB 10, not 0
        L.lcsa_segment_lists(g, 0, c, seg, 180, P, P, stream=0)
    with pytest.raises(L.LcsaError, match="LCSA_ERR_CAPACITY"):  # kmax below the longest list
        L.lcsa_segment_lists(g, 10, c, seg, 179, P, P, stream=0)
    with pytest.raises(L.LcsaError, match="LCSA_ERR_PARAM"):
        L.lcsa_segment_attn(g, P, 0, c, seg, P, P, 180, P, stream=0)
    with pytest.raises(L.LcsaError, match="LCSA_ERR_PARAM"):
        L.lcsa_segment_attn_tok(g, P, 0, c, seg, P, P, 180, P, stream=0)
    with pytest.raises(L.LcsaError, match="LCSA_ERR_NULL"):
        L.lcsa_segment_attn_tok(g, None, 10, c, seg, P, P, 180, P, stream=0)
    lib_ = L.load_library()
    assert lib_.lcsa_segment_lists(ctypes.byref(g), 10, ctypes.byref(c), None, 180, FAKE, FAKE,
                                   None) == 1  # LCSA_ERR_NULL
    big = L.make_geom(1, 2, 128, 34, 48, 80, L.LCSA_BF16)
    with pytest.raises(L.LcsaError, match="LCSA_ERR_CAPACITY"):
        L.lcsa_segment_max_list(big, [0] * 34)


# ------------------------------------------------------------------ backward

def test_backward_workspace_size_and_validation(lib):
    g = L.make_geom(1, 2, 128, 4, 16, 24, L.LCSA_BF16)
    nq, rows = 2 * 6, 2 * 2 * 6
    need = L.lcsa_attn_bwd_workspace_size(g)
    up = lambda x: (x + 255) // 256 * 256
    assert need == up(rows * 256 * 4) + up(rows * 4) + up(rows * nq * 4)

    class Buf:  # an aligned fake device buffer: validation fails before any device call
        def __init__(self, addr, n=0):
            self.addr, self.n = addr, n

        def data_ptr(self):
            return self.addr

        def numel(self):
            return self.n

        def element_size(self):
            return 1

    P = Buf(FAKE)

    def call(geom=g, ws=Buf(FAKE, need), kmax=4, scale=0.0):
        L.lcsa_block_sparse_attn_bwd(geom, P, P, P, P, P, P, P, P, kmax, P, P, P, ws, scale=scale,
                                     stream=0)

    with pytest.raises(L.LcsaError, match="LCSA_ERR_CAPACITY"):   # workspace one byte short
        call(ws=Buf(FAKE, need - 1))
    with pytest.raises(L.LcsaError, match="LCSA_ERR_ALIGN"):      # workspace not 256-aligned
        call(ws=Buf(FAKE + 16, need))
    with pytest.raises(L.LcsaError, match="LCSA_ERR_DTYPE"):      # bf16 only
        call(geom=L.make_geom(1, 2, 128, 4, 16, 24, L.LCSA_F32))
    with pytest.raises(L.LcsaError, match="LCSA_ERR_CAPACITY"):
        call(kmax=0)
    with pytest.raises(L.LcsaError, match="LCSA_ERR_PARAM"):
        call(scale=-1.0)
    # a block quarter spans 4 token rows read with 32-bit offsets: (3W + 8) NH D 2 bytes
    # must stay below 2^31 (W = 43688 is the first multiple of 8 past it at NH 64, D 128)
    wide = L.make_geom(1, 64, 128, 4, 16, 43688, L.LCSA_BF16)
    assert (3 * 43688 + 8) * 64 * 128 * 2 >= 2 ** 31 > (3 * 43680 + 8) * 64 * 128 * 2
    with pytest.raises(L.LcsaError, match="LCSA_ERR_CAPACITY.*too wide"):
        call(geom=wide, ws=Buf(FAKE, L.lcsa_attn_bwd_workspace_size(wide)))
    lib_ = L.load_library()
    assert lib_.lcsa_block_sparse_attn_bwd(ctypes.byref(g), None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, 4, ctypes.c_float(0), FAKE, FAKE, FAKE,
                                           FAKE, need, None) == 1  # LCSA_ERR_NULL


def test_partition_requires_the_newest_tbs_in_order(lib):
    """The chunk's temporal blocks go to the slots the last append returned:
    any other first_slot, or a chunk with more TBs than the cache holds, is
    refused before any device call (it would overwrite older cached TBs)."""
    ok = _P(FAKE)
    c = fake_cache(n_slots=4)
    L.lcsa_kv_cache_append(c, 2, 0)              # slots 0, 1
    L.lcsa_kv_cache_evict(c, 1)                   # holds TB 1 in slot 1
    assert L.lcsa_kv_cache_append(c, 2, 2) == 2   # TBs 2, 3 -> slots 2, 3
    two = L.make_geom(1, 12, 128, 4, 48, 88, L.LCSA_BF16)
    three = L.make_geom(1, 12, 128, 6, 48, 88, L.LCSA_BF16)
    one = L.make_geom(1, 12, 128, 2, 48, 88, L.LCSA_BF16)
    for first in (0, 1, 3):                       # not the slot the append returned
        expect(4, L.lcsa_partition_pool, two, ok, ok, ok, ok, ok, c, first, 0)
    expect(6, L.lcsa_partition_pool, L.make_geom(1, 12, 128, 8, 48, 88, 0), ok, ok, ok, ok, ok, c,
           1, 0)                                  # 4 TBs, 3 held
    expect(4, L.lcsa_partition_pool, three, ok, ok, ok, ok, ok, c, 2, 0)  # 3 TBs from slot 2 wrap
    expect(4, L.lcsa_partition_pool, one, ok, ok, ok, ok, ok, c, 2, 0)    # TB 2 is not the newest
    # wrap-around: the newest TB can sit in slot 0
    c2 = fake_cache(n_slots=4)
    L.lcsa_kv_cache_append(c2, 4, 0)
    L.lcsa_kv_cache_evict(c2, 3)
    assert L.lcsa_kv_cache_append(c2, 1, 4) == 0
    expect(4, L.lcsa_partition_pool, one, ok, ok, ok, ok, ok, c2, 3, 0)
    expect(4, L.lcsa_partition_pool, two, ok, ok, ok, ok, ok, c2, 0, 0)


def test_noalloc_backward_validation_before_any_device_call(lib):
    """lcsa_block_sparse_attn_bwd_noalloc refuses a chunk whose workspace
    exceeds the library's fixed scratch, and bad arguments, before any HIP
    call (so these run without a GPU)."""
    P = _P(FAKE)
    big = L.make_geom(1, 12, 128, 24, 96, 160, L.LCSA_BF16)
    assert L.lcsa_attn_bwd_workspace_size(big) > L.NOALLOC_SCRATCH_BYTES
    msg = expect(6, L.lcsa_block_sparse_attn_bwd_noalloc, big, P, P, P, P, P, P, P, P, 4, P, P, P,
                 stream=0)
    assert "scratch" in msg
    g = L.make_geom(1, 2, 128, 4, 16, 24, L.LCSA_BF16)
    expect(1, L.lcsa_block_sparse_attn_bwd_noalloc, g, None, P, P, P, P, P, P, P, 4, P, P, P,
           stream=0)
    expect(3, L.lcsa_block_sparse_attn_bwd_noalloc, L.make_geom(1, 2, 128, 4, 16, 24, L.LCSA_F32),
           P, P, P, P, P, P, P, P, 4, P, P, P, stream=0)
    expect(6, L.lcsa_block_sparse_attn_bwd_noalloc, g, P, P, P, P, P, P, P, P, 0, P, P, P,
           stream=0)
    expect(5, L.lcsa_block_sparse_attn_bwd_noalloc, g, P, P, P, P, P, P, P, _P(FAKE + 4), 4, P, P,
           P, stream=0)
    # an empty chunk is a no-op (no scratch lookup, no device call)
    L.lcsa_block_sparse_attn_bwd_noalloc(L.make_geom(1, 2, 128, 0, 16, 24, L.LCSA_BF16), P, P, P, P,
                                         P, P, P, P, 4, P, P, P, stream=0)


def test_ring_copy_validates_before_any_device_call(lib):
    """lcsa_kv_cache_copy, the checkpoint / resume of a stream's ring ([HW]
    "How FlashVSR works" 2.3: the cache of past segments is the state a
    stream carries between steps), refuses rings of another shape or dtype,
    the same cache, and overlapping rings, and leaves dst's metadata as it
    was. Fake device addresses: every case fails before its first HIP call."""
    P = lambda a: type("P", (), {"data_ptr": lambda s: a})()

    def cache(base, heads=3, D=128, nby=6, nbx=11, dtype=L.LCSA_BF16, n_slots=4):
        kv, pool = ring_bytes(nby, nbx, heads, D, dtype, n_slots)
        c = L.KvCacheStruct()
        L.lcsa_kv_cache_init(c, 1, heads, D, nby, nbx, dtype, n_slots, P(base), P(base + kv),
                             P(base + 2 * kv), kv, kv, pool)
        return c

    span = 1 << 32  # far apart: no ring of one fake cache overlaps the other's
    src = cache(FAKE)
    L.lcsa_kv_cache_append(src, 3, 0)
    bad = {
        2: [cache(span, heads=2), cache(span, D=64), cache(span, nbx=10), cache(span, n_slots=5)],
        3: [cache(span, dtype=L.LCSA_F32)],
        4: [cache(FAKE + 4096), cache(FAKE)],  # overlapping rings
    }
    for status, dsts in bad.items():
        for dst in dsts:
            before = (dst.head, dst.count, list(dst.abs_tb))
            with pytest.raises(L.LcsaError) as e:
                L.lcsa_kv_cache_copy(dst, src, stream=0)
            assert e.value.status == status, (status, str(e.value))
            assert (dst.head, dst.count, list(dst.abs_tb)) == before
    with pytest.raises(L.LcsaError) as e:
        L.lcsa_kv_cache_copy(src, src, stream=0)
    assert e.value.status == 4 and "same cache" in str(e.value)
