"""ctypes binding of liblcsa.so (include/lcsa.h).

Argument marshalling only: every step of LCSA runs in the library's HIP
kernels. PyTorch provides device memory and the stream. The functions carry
the C names; they take torch tensors (or None), check nothing beyond what is
needed to build the call, and raise :class:`LcsaError` with the library's
message when a call returns a non-zero status. If the library is missing,
loading fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblcsa.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lcsa.h")

LCSA_BF16, LCSA_F32 = 0, 1
BORDER_PRESERVED, BORDER_TRUNCATED = 0, 1
MAX_SLOTS = 16
MAX_CANDIDATES = 4096
STATUS = {0: "LCSA_OK", 1: "LCSA_ERR_NULL", 2: "LCSA_ERR_SHAPE", 3: "LCSA_ERR_DTYPE",
          4: "LCSA_ERR_PARAM", 5: "LCSA_ERR_ALIGN", 6: "LCSA_ERR_CAPACITY", 7: "LCSA_ERR_DEVICE"}


class LcsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Geom(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("heads", c_int32), ("head_dim", c_int32),
                ("frames", c_int32), ("height", c_int32), ("width", c_int32),
                ("dtype", c_int32)]


class SelectParams(ctypes.Structure):
    _fields_ = [("local_range", c_int32), ("border", c_int32), ("topk_fixed", c_int32),
                ("ratio_num", c_int32), ("ratio_den", c_int32),
                ("scale_by_resolution", c_int32), ("out_h", c_int32), ("out_w", c_int32),
                ("ref_h", c_int32), ("ref_w", c_int32), ("ratio_base", c_int32)]


class KvCacheStruct(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("heads", c_int32), ("head_dim", c_int32),
                ("nby", c_int32), ("nbx", c_int32), ("dtype", c_int32),
                ("n_slots", c_int32), ("head", c_int32), ("count", c_int32),
                ("reserved", c_int32), ("abs_tb", c_int64 * MAX_SLOTS),
                ("k_ring", c_void_p), ("v_ring", c_void_p), ("kpool_ring", c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load liblcsa.so (built in-tree by build_lib)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is missing: build it with "
                      "`python -m block_sparse_attention_03_amd.build_lib`")
    try:
        # torch first: the library then binds to the HIP runtime torch has
        # loaded, so both see the same devices, streams and allocations
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    G, P, C = POINTER(Geom), POINTER(SelectParams), POINTER(KvCacheStruct)
    sig = {
        "lcsa_kv_cache_init": [C, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                               c_void_p, c_void_p, c_void_p, ctypes.c_size_t, ctypes.c_size_t,
                               ctypes.c_size_t],
        "lcsa_kv_cache_append": [C, c_int32, c_int64, POINTER(c_int32)],
        "lcsa_kv_cache_evict": [C, c_int32],
        "lcsa_kv_cache_copy": [C, C, c_void_p],
        "lcsa_kv_cache_view": [C, POINTER(c_int32), POINTER(c_int32), POINTER(c_int64)],
        "lcsa_topk_count": [P, c_int32, c_int32, POINTER(c_int32)],
        "lcsa_max_topk": [G, c_int64, C, P, POINTER(c_int32)],
        "lcsa_partition_pool": [G, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, C,
                                c_int32, c_void_p],
        "lcsa_draft_mask": [G, c_void_p, c_int64, C, P, c_int32, c_void_p, c_void_p, c_void_p,
                            ctypes.c_size_t, c_void_p, ctypes.c_size_t, c_void_p],
        "lcsa_draft_workspace_size": [G, C, P, POINTER(ctypes.c_size_t)],
        "lcsa_block_sparse_attn": [G, c_void_p, C, c_void_p, c_void_p, c_int32, c_float,
                                   c_void_p, c_void_p, c_void_p],
        "lcsa_block_sparse_attn_tok": [G, c_void_p, C, c_void_p, c_void_p, c_int32, c_float,
                                       c_void_p, c_void_p, c_void_p],
        "lcsa_attn_bwd_workspace_size": [G, POINTER(ctypes.c_size_t)],
        "lcsa_block_sparse_attn_bwd": [G, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_int32, c_float, c_void_p,
                                       c_void_p, c_void_p, c_void_p, ctypes.c_size_t, c_void_p],
        "lcsa_block_sparse_attn_bwd_noalloc": [G, c_void_p, c_void_p, c_void_p, c_void_p,
                                               c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                               c_float, c_void_p, c_void_p, c_void_p, c_void_p],
        "lcsa_max_candidates": [G, c_int64, C, P, POINTER(c_int32)],
        "lcsa_local_lists": [G, c_int64, C, P, c_int32, c_void_p, c_void_p, c_void_p],
        "lcsa_segment_max_list": [G, POINTER(c_int32), POINTER(c_int32)],
        "lcsa_segment_lists": [G, c_int64, C, POINTER(c_int32), c_int32, c_void_p, c_void_p,
                               c_void_p],
        "lcsa_segment_attn": [G, c_void_p, c_int64, C, POINTER(c_int32), c_void_p, c_void_p,
                              c_int32, c_float, c_void_p, c_void_p, c_void_p],
        "lcsa_segment_attn_tok": [G, c_void_p, c_int64, C, POINTER(c_int32), c_void_p,
                                  c_void_p, c_int32, c_float, c_void_p, c_void_p, c_void_p],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = c_int32
    lib.lcsa_last_error.argtypes = []
    lib.lcsa_last_error.restype = c_char_p
    lib.lcsa_abi_version.argtypes = []
    lib.lcsa_abi_version.restype = c_int32
    _lib = lib
    return lib


def _check(st: int):
    if st != 0:
        raise LcsaError(st, _lib.lcsa_last_error().decode())


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return c_void_p(stream)
    return c_void_p(stream.cuda_stream)


def dtype_code(torch_dtype) -> int:
    import torch
    if torch_dtype == torch.bfloat16:
        return LCSA_BF16
    if torch_dtype == torch.float32:
        return LCSA_F32
    raise ValueError(f"unsupported dtype {torch_dtype}")


def make_geom(batch, heads, head_dim, frames, height, width, dtype) -> Geom:
    return Geom(batch, heads, head_dim, frames, height, width, dtype)


def make_params(local_range=11, border=BORDER_PRESERVED, topk_fixed=0, ratio=(1, 5),
                scale_by_resolution=False, out_hw=(768, 1280), ref_hw=(768, 1280),
                ratio_base=0) -> SelectParams:
    return SelectParams(local_range, border, topk_fixed, ratio[0], ratio[1],
                        int(bool(scale_by_resolution)), out_hw[0], out_hw[1], ref_hw[0],
                        ref_hw[1], ratio_base)


# ---------------------------------------------------------------- C names

def _nbytes(t):
    """Size in bytes of a tensor (0 for None or an object without one)."""
    if t is None or not hasattr(t, "numel"):
        return 0
    return t.numel() * t.element_size()


def lcsa_kv_cache_init(cache: KvCacheStruct, batch, heads, head_dim, nby, nbx, dtype, n_slots,
                       k_ring, v_ring, kpool_ring, bytes_k=None, bytes_v=None, bytes_kpool=None):
    """The buffer sizes default to the tensors' own sizes."""
    lib = load_library()
    bk = _nbytes(k_ring) if bytes_k is None else bytes_k
    bv = _nbytes(v_ring) if bytes_v is None else bytes_v
    bp = _nbytes(kpool_ring) if bytes_kpool is None else bytes_kpool
    _check(lib.lcsa_kv_cache_init(ctypes.byref(cache), batch, heads, head_dim, nby, nbx, dtype,
                                  n_slots, _ptr(k_ring), _ptr(v_ring), _ptr(kpool_ring), bk, bv,
                                  bp))


def lcsa_kv_cache_append(cache: KvCacheStruct, n_tb: int, first_abs_tb: int) -> int:
    lib = load_library()
    slot = c_int32(-1)
    _check(lib.lcsa_kv_cache_append(ctypes.byref(cache), n_tb, first_abs_tb, ctypes.byref(slot)))
    return slot.value


def lcsa_kv_cache_evict(cache: KvCacheStruct, keep_tb: int):
    lib = load_library()
    _check(lib.lcsa_kv_cache_evict(ctypes.byref(cache), keep_tb))


def lcsa_kv_cache_view(cache: KvCacheStruct):
    lib = load_library()
    n = c_int32(0)
    slots = (c_int32 * MAX_SLOTS)()
    tbs = (c_int64 * MAX_SLOTS)()
    _check(lib.lcsa_kv_cache_view(ctypes.byref(cache), ctypes.byref(n), slots, tbs))
    return list(slots[:n.value]), list(tbs[:n.value])


def lcsa_kv_cache_copy(dst: KvCacheStruct, src: KvCacheStruct, stream=None):
    lib = load_library()
    _check(lib.lcsa_kv_cache_copy(ctypes.byref(dst), ctypes.byref(src), _stream(stream)))


def lcsa_topk_count(params: SelectParams, n_allowed: int, n_keys: int) -> int:
    lib = load_library()
    k = c_int32(-1)
    _check(lib.lcsa_topk_count(ctypes.byref(params), n_allowed, n_keys, ctypes.byref(k)))
    return k.value


def lcsa_max_topk(geom: Geom, q_first_abs_tb: int, cache: KvCacheStruct,
                  params: SelectParams) -> int:
    lib = load_library()
    k = c_int32(-1)
    _check(lib.lcsa_max_topk(ctypes.byref(geom), q_first_abs_tb, ctypes.byref(cache),
                             ctypes.byref(params), ctypes.byref(k)))
    return k.value


def lcsa_partition_pool(geom: Geom, q, k, v, q_blk, q_pool, cache: KvCacheStruct,
                        first_slot: int, stream=None):
    lib = load_library()
    _check(lib.lcsa_partition_pool(ctypes.byref(geom), _ptr(q), _ptr(k), _ptr(v), _ptr(q_blk),
                                   _ptr(q_pool), ctypes.byref(cache), first_slot,
                                   _stream(stream)))


def lcsa_draft_mask(geom: Geom, q_pool, q_first_abs_tb: int, cache: KvCacheStruct,
                    params: SelectParams, kmax: int, sel_idx, sel_cnt, probs=None, stream=None,
                    probs_bytes=None, workspace=None, workspace_bytes=None):
    """probs_bytes and workspace_bytes default to the tensors' own sizes."""
    lib = load_library()
    pb = _nbytes(probs) if probs_bytes is None else probs_bytes
    wb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(lib.lcsa_draft_mask(ctypes.byref(geom), _ptr(q_pool), q_first_abs_tb,
                               ctypes.byref(cache), ctypes.byref(params), kmax, _ptr(sel_idx),
                               _ptr(sel_cnt), _ptr(probs), pb, _ptr(workspace), wb,
                               _stream(stream)))


def lcsa_draft_workspace_size(geom: Geom, cache: KvCacheStruct, params: SelectParams) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.lcsa_draft_workspace_size(ctypes.byref(geom), ctypes.byref(cache),
                                         ctypes.byref(params), ctypes.byref(n)))
    return n.value


def lcsa_block_sparse_attn(geom: Geom, q_blk, cache: KvCacheStruct, sel_idx, sel_cnt, kmax: int,
                           out, lse=None, scale: float = 0.0, stream=None):
    lib = load_library()
    _check(lib.lcsa_block_sparse_attn(ctypes.byref(geom), _ptr(q_blk), ctypes.byref(cache),
                                      _ptr(sel_idx), _ptr(sel_cnt), kmax, c_float(scale),
                                      _ptr(out), _ptr(lse), _stream(stream)))


def lcsa_block_sparse_attn_tok(geom: Geom, q, cache: KvCacheStruct, sel_idx, sel_cnt, kmax: int,
                               out, lse=None, scale: float = 0.0, stream=None):
    lib = load_library()
    _check(lib.lcsa_block_sparse_attn_tok(ctypes.byref(geom), _ptr(q), ctypes.byref(cache),
                                          _ptr(sel_idx), _ptr(sel_cnt), kmax, c_float(scale),
                                          _ptr(out), _ptr(lse), _stream(stream)))


def lcsa_max_candidates(geom: Geom, q_first_abs_tb: int, cache: KvCacheStruct,
                        params: SelectParams) -> int:
    lib = load_library()
    n = c_int32(-1)
    _check(lib.lcsa_max_candidates(ctypes.byref(geom), q_first_abs_tb, ctypes.byref(cache),
                                   ctypes.byref(params), ctypes.byref(n)))
    return n.value


def lcsa_local_lists(geom: Geom, q_first_abs_tb: int, cache: KvCacheStruct, params: SelectParams,
                     kmax: int, sel_idx, sel_cnt, stream=None):
    lib = load_library()
    _check(lib.lcsa_local_lists(ctypes.byref(geom), q_first_abs_tb, ctypes.byref(cache),
                                ctypes.byref(params), kmax, _ptr(sel_idx), _ptr(sel_cnt),
                                _stream(stream)))


def lcsa_attn_bwd_workspace_size(geom: Geom) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.lcsa_attn_bwd_workspace_size(ctypes.byref(geom), ctypes.byref(n)))
    return n.value


def lcsa_block_sparse_attn_bwd(geom: Geom, q, k, v, out, dout, lse, sel_idx, sel_cnt, kmax: int,
                               dq, dk, dv, workspace, scale: float = 0.0, stream=None):
    lib = load_library()
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.lcsa_block_sparse_attn_bwd(ctypes.byref(geom), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                          _ptr(dout), _ptr(lse), _ptr(sel_idx), _ptr(sel_cnt),
                                          kmax, c_float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                          _ptr(workspace), nbytes, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 48 << 20  # LCSA_NOALLOC_SCRATCH_BYTES


def lcsa_block_sparse_attn_bwd_noalloc(geom: Geom, q, k, v, out, dout, lse, sel_idx, sel_cnt,
                                       kmax: int, dq, dk, dv, scale: float = 0.0, stream=None):
    lib = load_library()
    _check(lib.lcsa_block_sparse_attn_bwd_noalloc(ctypes.byref(geom), _ptr(q), _ptr(k), _ptr(v),
                                                  _ptr(out), _ptr(dout), _ptr(lse), _ptr(sel_idx),
                                                  _ptr(sel_cnt), kmax, c_float(scale), _ptr(dq),
                                                  _ptr(dk), _ptr(dv), _stream(stream)))


def _frame_seg(frame_seg):
    arr = (c_int32 * len(frame_seg))(*[int(x) for x in frame_seg])
    return arr


def lcsa_segment_max_list(geom: Geom, frame_seg) -> int:
    lib = load_library()
    k = c_int32(-1)
    _check(lib.lcsa_segment_max_list(ctypes.byref(geom), _frame_seg(frame_seg), ctypes.byref(k)))
    return k.value


def lcsa_segment_lists(geom: Geom, q_first_abs_tb: int, cache: KvCacheStruct, frame_seg,
                       kmax: int, sel_idx, sel_cnt, stream=None):
    lib = load_library()
    _check(lib.lcsa_segment_lists(ctypes.byref(geom), q_first_abs_tb, ctypes.byref(cache),
                                  _frame_seg(frame_seg), kmax, _ptr(sel_idx), _ptr(sel_cnt),
                                  _stream(stream)))


def lcsa_segment_attn(geom: Geom, q_blk, q_first_abs_tb: int, cache: KvCacheStruct, frame_seg,
                      sel_idx, sel_cnt, kmax: int, out, lse=None, scale: float = 0.0,
                      stream=None):
    lib = load_library()
    _check(lib.lcsa_segment_attn(ctypes.byref(geom), _ptr(q_blk), q_first_abs_tb,
                                 ctypes.byref(cache), _frame_seg(frame_seg), _ptr(sel_idx),
                                 _ptr(sel_cnt), kmax, c_float(scale), _ptr(out), _ptr(lse),
                                 _stream(stream)))


def lcsa_segment_attn_tok(geom: Geom, q, q_first_abs_tb: int, cache: KvCacheStruct, frame_seg,
                          sel_idx, sel_cnt, kmax: int, out, lse=None, scale: float = 0.0,
                          stream=None):
    lib = load_library()
    _check(lib.lcsa_segment_attn_tok(ctypes.byref(geom), _ptr(q), q_first_abs_tb,
                                     ctypes.byref(cache), _frame_seg(frame_seg), _ptr(sel_idx),
                                     _ptr(sel_cnt), kmax, c_float(scale), _ptr(out), _ptr(lse),
                                     _stream(stream)))


def lcsa_last_error() -> str:
    return load_library().lcsa_last_error().decode()


def lcsa_abi_version() -> int:
    return load_library().lcsa_abi_version()


# ---------------------------------------------------------------- buffers

class KVCache:
    """One layer's ring: device buffers (torch) plus the host metadata."""

    def __init__(self, batch, heads, head_dim, height, width, dtype, n_slots, device="cuda"):
        import torch
        self.nby, self.nbx = height // 8, width // 8
        nS = self.nby * self.nbx
        code = dtype_code(dtype)
        self.k_ring = torch.empty((batch, heads, n_slots, nS, 128, head_dim), dtype=dtype,
                                  device=device)
        self.v_ring = torch.empty((batch, heads, n_slots, nS, head_dim, 128), dtype=dtype,
                                  device=device)
        self.kpool_ring = torch.empty((batch, heads, n_slots, head_dim, nS), dtype=torch.float64,
                                      device=device)
        self.c = KvCacheStruct()
        lcsa_kv_cache_init(self.c, batch, heads, head_dim, self.nby, self.nbx, code, n_slots,
                           self.k_ring, self.v_ring, self.kpool_ring)

    def append(self, n_tb, first_abs_tb):
        return lcsa_kv_cache_append(self.c, n_tb, first_abs_tb)

    def evict(self, keep_tb):
        lcsa_kv_cache_evict(self.c, keep_tb)

    def view(self):
        return lcsa_kv_cache_view(self.c)

    def copy_from(self, other: "KVCache", stream=None):
        """Take over other's held blocks and metadata (lcsa_kv_cache_copy)."""
        lcsa_kv_cache_copy(self.c, other.c, stream)


class StepBuffers:
    """Per-chunk outputs of the pipeline for a query geometry."""

    def __init__(self, geom: Geom, kmax: int, device="cuda", with_probs_keys: int = 0,
                 with_lse: bool = False, with_q_blk: bool = False):
        import torch
        nS = (geom.height // 8) * (geom.width // 8)
        nq = (geom.frames // 2) * nS
        dt = torch.bfloat16 if geom.dtype == LCSA_BF16 else torch.float32
        B, NH, D = geom.batch, geom.heads, geom.head_dim
        self.kmax = kmax
        # the query blocks are only materialised for the block-layout path
        self.q_blk = (torch.empty((B, NH, nq, 128, D), dtype=dt, device=device)
                      if with_q_blk else None)
        self.q_pool = torch.empty((B, NH, nq, D), dtype=torch.float64, device=device)
        self.sel_idx = torch.empty((B, NH, nq, max(kmax, 1)), dtype=torch.int32, device=device)
        self.sel_cnt = torch.empty((B, NH, nq), dtype=torch.int32, device=device)
        self.out = torch.empty((B, geom.frames, geom.height, geom.width, NH, D), dtype=dt,
                               device=device)
        self.probs = (torch.empty((B, NH, nq, with_probs_keys), dtype=torch.float64,
                                  device=device) if with_probs_keys else None)
        self.lse = torch.empty((B, NH, nq, 128), dtype=torch.float32,
                               device=device) if with_lse else None


def run_step(geom: Geom, q, k, v, cache: KVCache, first_abs_tb: int, params: SelectParams,
             bufs: StepBuffers | None = None, keep_tb: int | None = None, stream=None,
             want_probs=False, want_lse=False, scale: float = 0.0, local: bool = False,
             q_blocks: bool = False, draft_workspace=None):
    """One LCSA invocation through the C-ABI: append, partition+pool, draft
    (or, with local=True, the FlashVSR+ local lists: every allowed key
    block), attention, evict. The attention reads q in token layout, so the
    partition writes only q's block means; q_blocks=True instead writes the
    query blocks to bufs.q_blk and reads them from there. draft_workspace
    (a device tensor of lcsa_draft_workspace_size bytes, or None) goes to the
    draft. Returns the StepBuffers holding the results."""
    n_tb = geom.frames // 2
    first_slot = cache.append(n_tb, first_abs_tb)
    if local:
        kmax = lcsa_max_candidates(geom, first_abs_tb, cache.c, params)
    else:
        kmax = lcsa_max_topk(geom, first_abs_tb, cache.c, params)
    if bufs is None:
        n_keys = cache.c.count * cache.nby * cache.nbx
        bufs = StepBuffers(geom, kmax, device=q.device,
                           with_probs_keys=n_keys if want_probs and not local else 0,
                           with_lse=want_lse, with_q_blk=q_blocks)
    if q_blocks and bufs.q_blk is None:
        raise ValueError("q_blocks=True needs StepBuffers(with_q_blk=True)")
    q_blk = bufs.q_blk if q_blocks else None
    lcsa_partition_pool(geom, q, k, v, q_blk, bufs.q_pool, cache.c, first_slot, stream)
    if local:
        lcsa_local_lists(geom, first_abs_tb, cache.c, params, bufs.kmax, bufs.sel_idx,
                         bufs.sel_cnt, stream)
    else:
        lcsa_draft_mask(geom, bufs.q_pool, first_abs_tb, cache.c, params, bufs.kmax,
                        bufs.sel_idx, bufs.sel_cnt, bufs.probs, stream,
                        workspace=draft_workspace)
    if q_blocks:
        lcsa_block_sparse_attn(geom, q_blk, cache.c, bufs.sel_idx, bufs.sel_cnt, bufs.kmax,
                               bufs.out, bufs.lse, scale, stream)
    else:
        lcsa_block_sparse_attn_tok(geom, q, cache.c, bufs.sel_idx, bufs.sel_cnt, bufs.kmax,
                                   bufs.out, bufs.lse, scale, stream)
    if keep_tb is not None:
        cache.evict(keep_tb)
    return bufs


def run_segment_step(geom: Geom, q, k, v, cache: KVCache, first_abs_tb: int, frame_seg,
                     bufs: StepBuffers | None = None, stream=None, want_lse=False,
                     scale: float = 0.0, q_blocks: bool = False):
    """Stage-1 segment-masked attention of one chunk through the C-ABI, as a
    cold start: append, partition+pool, segment lists, masked attention,
    then the cache is emptied again. q_blocks as in run_step. Returns the
    StepBuffers."""
    n_tb = geom.frames // 2
    first_slot = cache.append(n_tb, first_abs_tb)
    kmax = lcsa_segment_max_list(geom, frame_seg)
    if bufs is None:
        bufs = StepBuffers(geom, kmax, device=q.device, with_lse=want_lse, with_q_blk=q_blocks)
    if q_blocks and bufs.q_blk is None:
        raise ValueError("q_blocks=True needs StepBuffers(with_q_blk=True)")
    q_blk = bufs.q_blk if q_blocks else None
    lcsa_partition_pool(geom, q, k, v, q_blk, bufs.q_pool, cache.c, first_slot, stream)
    lcsa_segment_lists(geom, first_abs_tb, cache.c, frame_seg, bufs.kmax, bufs.sel_idx,
                       bufs.sel_cnt, stream)
    if q_blocks:
        lcsa_segment_attn(geom, q_blk, first_abs_tb, cache.c, frame_seg, bufs.sel_idx,
                          bufs.sel_cnt, bufs.kmax, bufs.out, bufs.lse, scale, stream)
    else:
        lcsa_segment_attn_tok(geom, q, first_abs_tb, cache.c, frame_seg, bufs.sel_idx,
                              bufs.sel_cnt, bufs.kmax, bufs.out, bufs.lse, scale, stream)
    cache.evict(0)
    return bufs


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
