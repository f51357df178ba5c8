"""Token-space brute force of LCSA, written independently of the oracle.

It never forms blocks as tensors: every quantity is computed from token
coordinates (absolute latent frame, row, column). A token belongs to block
(t//2, y//8, x//8) ([HW] "How FlashVSR works" 2.2 step 1). Windows are found
by a different formulation than the oracle's: Boundary-Preserved picks, among
all length-r runs inside the axis, the one whose centre is nearest the query
(the whole axis if it is not longer than r); Boundary-Truncated is the set
{j : |i - j| <= r//2} clipped to the axis.

Used only on tiny inputs to pin the oracle. Imports nothing from oracle/.
"""
from __future__ import annotations

import math

import numpy as np


def bp_window(i, n, r):
    if n <= r:
        return set(range(n))
    h = r // 2
    best = min(range(0, n - r + 1), key=lambda s: abs(s + h - i))
    return set(range(best, best + r))


def bt_window(i, n, r):
    h = r // 2
    return {j for j in range(n) if abs(i - j) <= h}


def token_coords(t0, T, H, W):
    """Absolute (t, y, x) of every token of frames [t0, t0+T), (t, y, x) order."""
    tt, yy, xx = np.meshgrid(np.arange(t0, t0 + T), np.arange(H), np.arange(W), indexing="ij")
    return tt.ravel(), yy.ravel(), xx.ravel()


def lcsa_bruteforce(q, k_frames, v_frames, q_t0, k_t0, r, border, kfun, scale=None):
    """LCSA for one batch entry, all heads, token space.

    q: [Tq][H][W][NH][D] (new frames starting at absolute frame q_t0);
    k_frames, v_frames: [Tk][H][W][NH][D], every key frame from absolute
    frame k_t0 (the cache view followed by the new frames).
    kfun(n_allowed, n_keys) -> k_row.

    Returns (out [Tq][H][W][NH][D], selections dict (h, qblock) -> sorted list
    of key block ids, scores dict). Key block ids count blocks of the key
    frames in (tb, by, bx) order from the first key frame.
    """
    Tq, H, W, NH, D = q.shape
    Tk = k_frames.shape[0]
    nby, nbx = H // 8, W // 8
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qt, qy, qx = token_coords(q_t0, Tq, H, W)
    kt, ky, kx = token_coords(k_t0, Tk, H, W)
    qflat = q.reshape(-1, NH, D)
    kflat = k_frames.reshape(-1, NH, D)
    vflat = v_frames.reshape(-1, NH, D)

    def qblock_id(t, y, x):
        return (((t - q_t0) // 2) * nby + y // 8) * nbx + x // 8

    def kblock_id(t, y, x):
        return (((t - k_t0) // 2) * nby + y // 8) * nbx + x // 8

    qbid = np.array([qblock_id(*c) for c in zip(qt, qy, qx)])
    kbid = np.array([kblock_id(*c) for c in zip(kt, ky, kx)])
    nq, nk = qbid.max() + 1, kbid.max() + 1
    # block coordinates from any member token
    qcoord = {}
    for idx, b in enumerate(qbid):
        qcoord.setdefault(b, (qt[idx] // 2, qy[idx] // 8, qx[idx] // 8))
    kcoord = {}
    for idx, b in enumerate(kbid):
        kcoord.setdefault(b, (kt[idx] // 2, ky[idx] // 8, kx[idx] // 8))

    win = bp_window if border == 0 else bt_window
    out = np.zeros_like(q).reshape(-1, NH, D)
    sels, scs = {}, {}
    for h in range(NH):
        # pooled means: accumulate token values per block id
        pq = np.zeros((nq, D))
        cq = np.zeros(nq)
        np.add.at(pq, qbid, qflat[:, h])
        np.add.at(cq, qbid, 1.0)
        pq /= cq[:, None]
        pk = np.zeros((nk, D))
        ck = np.zeros(nk)
        np.add.at(pk, kbid, kflat[:, h])
        np.add.at(ck, kbid, 1.0)
        pk /= ck[:, None]
        for i in range(nq):
            ti, yi, xi = qcoord[i]
            wy, wx = win(yi, nby, r), win(xi, nbx, r)
            cand = [j for j in range(nk)
                    if kcoord[j][0] <= ti and kcoord[j][1] in wy and kcoord[j][2] in wx]
            s = {j: float(np.dot(pq[i], pk[j])) / math.sqrt(D) for j in cand}
            kk = kfun(len(cand), nk)
            chosen = sorted(sorted(cand, key=lambda j: (-s[j], j))[:kk])
            sels[(h, i)] = chosen
            scs[(h, i)] = s
            # exact attention of every query token of block i over the chosen blocks
            qa = np.nonzero(qbid == i)[0]
            kb = np.nonzero(np.isin(kbid, chosen))[0]
            if len(kb) == 0:
                continue
            for a in qa:
                logits = (kflat[kb, h] @ qflat[a, h]) * scale
                w = np.exp(logits - logits.max())
                w /= w.sum()
                out[a, h] = w @ vflat[kb, h]
    return out.reshape(q.shape), sels, scs
