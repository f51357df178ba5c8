"""LCSA oracle: a plain, slow float64 CPU implementation of locality-constrained
block-sparse causal attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The GPU
library never routes through it, and it shares no code, constant or helper
with the HIP path.

Sources. Two pages describe the method:

* [FN]  "FlashVSR: Towards Real-time Diffusion-Based Streaming Video Super
  Resolution" (papernotes.org CVPR 2026 note), Key design 1 (causal mask of
  Stage 2), Key design 2 (block-sparse causal attention) and Key design 3
  (locality-constrained sparse attention, two border rules).
* [HW]  "How FlashVSR works" (vsr-hover-compare learn page), section 2.2
  (LCSA: step 1 window partition, step 2 local mask, step 3 draft top-k, the
  topk_ratio rule), section 2.3 (streaming with a KV cache) and section 5.3
  (token geometry: one block is 8x8 tokens of 2 latent frames).

The oracle follows those steps in the pages' order. Each step is written out
directly: no blocking, no fusion, no online softmax. Library primitives used
as steps: numpy matmul, exp, lexsort.

Readings of points the pages leave open (each also listed in the design
notes of the repository):

* top-k is taken per query-block row of the block map, over its allowed keys;
* exactly k blocks are kept; equal scores are ordered by lower key index;
* selection ranks draft scores (softmax is monotone, the set is the same);
* the ratio rule multiplies a row's allowed-key count (or, with
  ``ratio_base=1``, the row's whole key count), the result is floored and
  clamped to [1, allowed];
* Boundary-Preserved = a window of fixed size r shifted to stay inside the
  grid; Boundary-Truncated = the centred window clipped at the grid edge;
* causality is at temporal-block granularity: a query block sees every key
  block whose temporal block is not later than its own;
* the cache keeps whole temporal blocks and drops the oldest first;
* Stage-1 segments are runs of whole latent frames (an image is a segment of
  one frame); the mask is applied per token, not per block;
* the backward holds the top-k selection fixed (a discrete choice has no
  gradient) and differentiates the attention over the selected pairs.

All floating point is float64. Inputs are the exact values the GPU receives
(bf16 or fp32), widened.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# [HW] 2.2 step 1: the 3D window is 2 latent frames x 8 x 8 tokens.
WIN_T, WIN_Y, WIN_X = 2, 8, 8
BLOCK_TOKENS = WIN_T * WIN_Y * WIN_X  # 128, [FN] Key design 2

BORDER_PRESERVED = 0
BORDER_TRUNCATED = 1


@dataclass
class SelectParams:
    """Selection knobs: local window and the k rule ([HW] 2.2 steps 2-3)."""

    local_range: int = 11          # window size in blocks per spatial axis (odd)
    border: int = BORDER_PRESERVED
    topk_fixed: int = 0            # > 0: fixed k per row (clamped to allowed)
    ratio_num: int = 1             # base sparse ratio as a fraction
    ratio_den: int = 5
    scale_by_resolution: bool = False
    out_h: int = 768               # output resolution in pixels
    out_w: int = 1280
    ref_h: int = 768               # base resolution of the ratio rule
    ref_w: int = 1280
    ratio_base: int = 0            # 0: ratio of allowed keys, 1: of all keys


# --------------------------------------------------------------------------
# Step 1 -- 3D window partition ([HW] 2.2 step 1; [FN] Key design 2)
# --------------------------------------------------------------------------

def check_grid(frames: int, height: int, width: int) -> None:
    if frames % WIN_T or height % WIN_Y or width % WIN_X:
        raise ValueError("token grid must be a whole number of 2x8x8 windows: "
                         f"got T={frames} H={height} W={width}")


def partition(x: np.ndarray) -> np.ndarray:
    """Token layout [B][T][H][W][NH][D] -> blocks [B][NH][nblk][128][D].

    Block n = (bt*nby + by)*nbx + bx holds tokens (2bt+dt, 8by+dy, 8bx+dx) at
    in-block position (dt*8 + dy)*8 + dx.
    """
    B, T, H, W, NH, D = x.shape
    check_grid(T, H, W)
    nbt, nby, nbx = T // WIN_T, H // WIN_Y, W // WIN_X
    out = np.empty((B, NH, nbt * nby * nbx, BLOCK_TOKENS, D), dtype=x.dtype)
    for bt in range(nbt):
        for by in range(nby):
            for bx in range(nbx):
                n = (bt * nby + by) * nbx + bx
                win = x[:, WIN_T * bt:WIN_T * bt + WIN_T,
                        WIN_Y * by:WIN_Y * by + WIN_Y,
                        WIN_X * bx:WIN_X * bx + WIN_X]          # [B,2,8,8,NH,D]
                out[:, :, n] = win.transpose(0, 4, 1, 2, 3, 5).reshape(B, NH, BLOCK_TOKENS, D)
    return out


def unpartition(xb: np.ndarray, frames: int, height: int, width: int) -> np.ndarray:
    """Inverse of :func:`partition`."""
    B, NH, nblk, _, D = xb.shape
    nbt, nby, nbx = frames // WIN_T, height // WIN_Y, width // WIN_X
    assert nblk == nbt * nby * nbx
    out = np.empty((B, frames, height, width, NH, D), dtype=xb.dtype)
    for bt in range(nbt):
        for by in range(nby):
            for bx in range(nbx):
                n = (bt * nby + by) * nbx + bx
                win = xb[:, :, n].reshape(B, NH, WIN_T, WIN_Y, WIN_X, D).transpose(0, 2, 3, 4, 1, 5)
                out[:, WIN_T * bt:WIN_T * bt + WIN_T,
                    WIN_Y * by:WIN_Y * by + WIN_Y,
                    WIN_X * bx:WIN_X * bx + WIN_X] = win
    return out


# --------------------------------------------------------------------------
# Step 2 -- block-mean pooling ([HW] 2.2 step 3, "each block compressed into
# one vector"; [FN] Key design 2)
# --------------------------------------------------------------------------

def pool(xb: np.ndarray) -> np.ndarray:
    """Mean over the 128 tokens of each block: [B][NH][nblk][D]."""
    return xb.sum(axis=3) / BLOCK_TOKENS


# --------------------------------------------------------------------------
# Step 3 -- local spatial window and temporal causality
# ([HW] 2.2 step 2; [FN] Key design 3 and Key design 1)
# --------------------------------------------------------------------------

def window_1d(i: int, n: int, r: int, border: int) -> range:
    """Block positions along one spatial axis that block i may see."""
    h = r // 2
    if border == BORDER_PRESERVED:
        if n <= r:
            return range(0, n)
        s = min(max(i - h, 0), n - r)
        return range(s, s + r)
    if border == BORDER_TRUNCATED:
        return range(max(i - h, 0), min(i + h, n - 1) + 1)
    raise ValueError(f"unknown border rule {border}")


def block_coords(tbs, nby: int, nbx: int):
    """(absolute temporal block, by, bx) of every block of the listed TBs."""
    return [(tb, by, bx) for tb in tbs for by in range(nby) for bx in range(nbx)]


def allowed_mask(q_tbs, k_tbs, nby: int, nbx: int, p: SelectParams) -> np.ndarray:
    """Boolean [nq][nk]: key block j is a candidate for query block i."""
    qc = block_coords(q_tbs, nby, nbx)
    kc = block_coords(k_tbs, nby, nbx)
    m = np.zeros((len(qc), len(kc)), dtype=bool)
    for i, (tq, yq, xq) in enumerate(qc):
        wy = window_1d(yq, nby, p.local_range, p.border)
        wx = window_1d(xq, nbx, p.local_range, p.border)
        for j, (tk, yk, xk) in enumerate(kc):
            m[i, j] = (tk <= tq) and (yk in wy) and (xk in wx)
    return m


# --------------------------------------------------------------------------
# Step 4 -- draft scores, row softmax, k rule and top-k ([HW] 2.2 step 3 and
# the topk_ratio rule)
# --------------------------------------------------------------------------

def draft_scores(pq: np.ndarray, pk: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """s[i, j] = pq_i . pk_j / sqrt(D) on allowed pairs, -inf elsewhere.

    pq: [nq][D], pk: [nk][D] for one (batch, head).
    """
    D = pq.shape[-1]
    s = (pq @ pk.T) / math.sqrt(D)
    return np.where(allowed, s, -np.inf)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax over the allowed (finite) entries; rows with none are 0."""
    out = np.zeros_like(s)
    for i in range(s.shape[0]):
        fin = np.isfinite(s[i])
        if not fin.any():
            continue
        e = np.exp(s[i, fin] - s[i, fin].max())
        out[i, fin] = e / e.sum()
    return out


def topk_count(n_allowed: int, n_keys: int, p: SelectParams) -> int:
    """Blocks kept in a row with ``n_allowed`` candidates out of ``n_keys``.

    Ratio rule: topk_ratio = sparse_ratio * ref_h*ref_w / (out_h*out_w) when
    scaled by resolution; k = floor(base * topk_ratio) in exact integers,
    clamped to [1, n_allowed]. Fixed rule: min(topk_fixed, n_allowed).
    """
    if n_allowed <= 0:
        return 0
    if p.topk_fixed > 0:
        return min(p.topk_fixed, n_allowed)
    base = n_allowed if p.ratio_base == 0 else n_keys
    num = p.ratio_num * (p.ref_h * p.ref_w if p.scale_by_resolution else 1)
    den = p.ratio_den * (p.out_h * p.out_w if p.scale_by_resolution else 1)
    k = (base * num) // den
    return max(1, min(k, n_allowed))


def select_topk(s: np.ndarray, p: SelectParams):
    """Per row: the k_row allowed keys of largest score, ties to lower index.

    Returns (list of ascending int arrays, int array of k_row).
    """
    sel, ks = [], np.zeros(s.shape[0], dtype=np.int64)
    n_keys = s.shape[1]
    for i in range(s.shape[0]):
        cand = np.nonzero(np.isfinite(s[i]))[0]
        k = topk_count(len(cand), n_keys, p)
        order = cand[np.lexsort((cand, -s[i, cand]))]   # by (-score, index)
        sel.append(np.sort(order[:k]))
        ks[i] = k
    return sel, ks


# --------------------------------------------------------------------------
# Step 5 -- exact attention over the selected block pairs
# ([FN] Key design 2: full 128x128 attention with the original Q, K, V;
#  [HW] 2.2: unselected blocks are skipped)
# --------------------------------------------------------------------------

def sparse_attention_row(qb: np.ndarray, kb: np.ndarray, vb: np.ndarray,
                         sel_row: np.ndarray, scale: float):
    """One query block against the union of its selected key blocks.

    qb: [128][D]; kb, vb: [nk][128][D]. Returns (O [128][D], lse [128]) with
    lse the natural log-sum-exp of the scaled logits. A row with nothing
    selected gives O = 0 and lse = -inf.
    """
    if len(sel_row) == 0:
        return np.zeros_like(qb), np.full(qb.shape[0], -np.inf)
    K = kb[sel_row].reshape(-1, kb.shape[-1])
    V = vb[sel_row].reshape(-1, vb.shape[-1])
    logits = (qb @ K.T) * scale
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    return (e @ V) / z, (m + np.log(z))[:, 0]


# --------------------------------------------------------------------------
# Streaming KV cache ([HW] 2.3)
# --------------------------------------------------------------------------

@dataclass
class KVCache:
    """Per-layer cache of whole temporal blocks, oldest first.

    Entries: (absolute TB index, k blocks [B][NH][nS][128][D],
    v blocks [B][NH][nS][128][D], pooled k [B][NH][nS][D]).
    """

    cap_tb: int = 3
    entries: list = field(default_factory=list)

    def append(self, abs_tb: int, kb, vb, kp) -> None:
        self.entries.append((abs_tb, kb, vb, kp))

    def evict(self) -> None:
        """Keep the newest ``cap_tb`` temporal blocks (drop the oldest)."""
        while len(self.entries) > self.cap_tb:
            self.entries.pop(0)

    def tbs(self):
        return [e[0] for e in self.entries]

    def keys(self):
        """Concatenated view oldest -> newest: kb, vb [B][NH][nk][128][D], kp."""
        kb = np.concatenate([e[1] for e in self.entries], axis=2)
        vb = np.concatenate([e[2] for e in self.entries], axis=2)
        kp = np.concatenate([e[3] for e in self.entries], axis=2)
        return kb, vb, kp


def prime_cache(cache: KVCache, k: np.ndarray, v: np.ndarray, first_abs_tb: int) -> None:
    """Append the k/v blocks of earlier frames (no queries), as a stream's
    earlier steps would have left them ([HW] 2.3)."""
    B, T, H, W, NH, D = k.shape
    check_grid(T, H, W)
    nS = (H // WIN_Y) * (W // WIN_X)
    kb, vb = partition(k), partition(v)
    kp = pool(kb)
    for t in range(T // WIN_T):
        sl = slice(t * nS, (t + 1) * nS)
        cache.append(first_abs_tb + t, kb[:, :, sl], vb[:, :, sl], kp[:, :, sl])


@dataclass
class StepResult:
    out: np.ndarray            # [B][T][H][W][NH][D]
    lse: np.ndarray            # [B][NH][nq][128]
    scores: np.ndarray         # [B][NH][nq][nk]   draft scores (-inf off-window)
    probs: np.ndarray          # [B][NH][nq][nk]   draft softmax
    allowed: np.ndarray        # [nq][nk]
    sel: list                  # [B][NH] -> list over rows of ascending key ids
    kcount: np.ndarray         # [nq] k_row
    q_pool: np.ndarray         # [B][NH][nq][D]
    q_blocks: np.ndarray       # [B][NH][nq][128][D]
    key_tbs: list              # absolute TB of each key TB in the view
    key_blocks: tuple          # (kb, vb) of the view [B][NH][nk][128][D]


def lcsa_step(q: np.ndarray, k: np.ndarray, v: np.ndarray, cache: KVCache,
              first_abs_tb: int, p: SelectParams, scale: float | None = None,
              rows=None, evict: bool = True) -> StepResult:
    """One LCSA invocation on a chunk of new latent frames.

    q, k, v: float64 token layout [B][T][H][W][NH][D] of the new frames; T is
    even and the chunk's first frame is temporal block ``first_abs_tb``. The
    new k/v blocks are appended to ``cache``; queries attend the cache view
    (older blocks plus the new ones) under the causal and local masks; then
    the cache is trimmed to its capacity. A cold start is the same call on an
    empty cache.

    ``rows``: optional list of (b, h, i) query rows for which attention is
    computed (the others are left 0); None computes every row.
    """
    B, T, H, W, NH, D = q.shape
    check_grid(T, H, W)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nby, nbx = H // WIN_Y, W // WIN_X
    nS = nby * nbx
    n_new = T // WIN_T

    qb = partition(q)
    kbn = partition(k)
    vbn = partition(v)
    pq = pool(qb)
    pkn = pool(kbn)
    for t in range(n_new):
        sl = slice(t * nS, (t + 1) * nS)
        cache.append(first_abs_tb + t, kbn[:, :, sl], vbn[:, :, sl], pkn[:, :, sl])

    kb, vb, pk = cache.keys()
    key_tbs = cache.tbs()
    q_tbs = [first_abs_tb + t for t in range(n_new)]
    allowed = allowed_mask(q_tbs, key_tbs, nby, nbx, p)
    nq, nk = allowed.shape

    scores = np.empty((B, NH, nq, nk))
    probs = np.empty((B, NH, nq, nk))
    sel = [[None] * NH for _ in range(B)]
    kcount = None
    ob = np.zeros_like(qb)
    lse = np.full((B, NH, nq, BLOCK_TOKENS), -np.inf)
    want = None if rows is None else set(map(tuple, rows))
    for b in range(B):
        for h in range(NH):
            s = draft_scores(pq[b, h], pk[b, h], allowed)
            scores[b, h] = s
            probs[b, h] = softmax_rows(s)
            sel_bh, kcount = select_topk(s, p)
            sel[b][h] = sel_bh
            for i in range(nq):
                if want is not None and (b, h, i) not in want:
                    continue
                ob[b, h, i], lse[b, h, i] = sparse_attention_row(
                    qb[b, h, i], kb[b, h], vb[b, h], sel_bh[i], scale)
    if evict:
        cache.evict()
    return StepResult(out=unpartition(ob, T, H, W), lse=lse, scores=scores,
                      probs=probs, allowed=allowed, sel=sel, kcount=kcount,
                      q_pool=pq, q_blocks=qb, key_tbs=key_tbs, key_blocks=(kb, vb))


# ------------------------------------------------------------ Stage 1 ------
def segment_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, frame_seg,
                      scale: float | None = None, queries=None) -> np.ndarray:
    """Segment-masked full attention of the Stage-1 teacher.

    [FN] Key design 1, Stage 1: images are treated as one-frame videos inside
    the same 3D attention, and a block-diagonal segment mask keeps attention
    within a segment: the weight of key token j for query token i is
    exp(q_i k_j / sqrt(d)) * [seg(i) = seg(j)], normalised by the same sum
    over all keys. There is no block sparsity and no causality in this stage.

    q, k, v: float64 token layout [B][T][H][W][NH][D]; frame_seg: T segment
    ids, one per latent frame (a token's segment is its frame's). Keys with
    another segment contribute exactly zero to both sums, so each query is
    computed over the keys of its own segment only.

    queries: None for every token (returns [B][T][H][W][NH][D]), or a list
    of (b, t, y, x) query tokens (returns [len(queries)][NH][D]).
    """
    B, T, H, W, NH, D = q.shape
    seg = np.asarray(frame_seg)
    if seg.shape != (T,):
        raise ValueError("frame_seg needs one id per latent frame")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    L = T * H * W
    qt, kt, vt = (x.reshape(B, L, NH, D) for x in (q, k, v))
    tok_seg = np.repeat(seg, H * W)  # token (t, y, x) row-major -> its frame's segment
    if queries is None:
        qidx = [(b, n) for b in range(B) for n in range(L)]
    else:
        qidx = [(b, (t * H + y) * W + x) for (b, t, y, x) in queries]
    out = np.zeros((len(qidx), NH, D))
    by_key = {}
    for r, (b, n) in enumerate(qidx):
        by_key.setdefault((b, tok_seg[n]), []).append(r)
    for (b, sg), rs in by_key.items():
        keys = np.nonzero(tok_seg == sg)[0]
        toks = np.array([qidx[r][1] for r in rs])
        for h in range(NH):
            s = (qt[b, toks, h] @ kt[b, keys, h].T) * scale
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            out[rs, h] = (e / e.sum(axis=1, keepdims=True)) @ vt[b, keys, h]
    if queries is None:
        return out.reshape(B, T, H, W, NH, D)
    return out


# ------------------------------------------------------------ backward -----
def sparse_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                              sel, scale: float | None = None, rows=None):
    """Gradients of the block-sparse attention of a chunk w.r.t. q, k and v.

    The forward is the attention of [FN] Key design 2 on the selected block
    pairs: query block i attends the union of the key blocks in sel[b][h][i]
    (ids into the chunk's own blocks, the training-shape forward where every
    frame is computed at once). The selection is a discrete choice and is
    held fixed; the gradient flows through the attention only. For one query
    block with selected keys K, V (rows of their 128-token blocks):
        P  = softmax(scale * Q K^T)          (row-wise)
        dV += P^T dO        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))       (softmax Jacobian, row-wise)
        dQ = scale * dS K   dK += scale * dS^T Q

    q, k, v, dout: float64 token layout [B][T][H][W][NH][D]; sel: [B][NH]
    lists of per-row ascending key ids. rows: None for every row, or a set of
    (b, h, i) rows whose terms are computed (dq of the other rows stays 0,
    and dk / dv hold only the listed rows' contributions).
    Returns (dq, dk, dv) in block layout [B][NH][nblk][128][D].
    """
    B, T, H, W, NH, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qb, kb, vb, gb = partition(q), partition(k), partition(v), partition(dout)
    nq = qb.shape[2]
    dq, dk, dv = np.zeros_like(qb), np.zeros_like(kb), np.zeros_like(vb)
    want = None if rows is None else set(map(tuple, rows))
    for b in range(B):
        for h in range(NH):
            for i in range(nq):
                ids = list(sel[b][h][i])
                if not ids or (want is not None and (b, h, i) not in want):
                    continue
                K = kb[b, h, ids].reshape(-1, D)
                V = vb[b, h, ids].reshape(-1, D)
                Q, dO = qb[b, h, i], gb[b, h, i]
                logits = (Q @ K.T) * scale
                e = np.exp(logits - logits.max(axis=1, keepdims=True))
                P = e / e.sum(axis=1, keepdims=True)
                dP = dO @ V.T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                dq[b, h, i] = scale * (dS @ K)
                gK = scale * (dS.T @ Q)
                gV = P.T @ dO
                for n, j in enumerate(ids):
                    dk[b, h, j] += gK[n * BLOCK_TOKENS:(n + 1) * BLOCK_TOKENS]
                    dv[b, h, j] += gV[n * BLOCK_TOKENS:(n + 1) * BLOCK_TOKENS]
    return dq, dk, dv
