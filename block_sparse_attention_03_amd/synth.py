"""Seeded synthetic q/k/v fields for LCSA workloads.

This module only makes input data. It holds none of the attention method's
arithmetic: no partition, pooling, scoring, selection or attention. Both the
GPU path and the CPU oracle receive the arrays it returns.

Recipe (one definition, used by every test and by the bench):

* For a tensor X in {q, k, v} (ids 0, 1, 2), every head h and channel d draw
  frequencies f_t ~ U(-1/16, 1/16) cycles per latent frame and
  f_y, f_x ~ U(-1/48, 1/48) cycles per token, and a phase phi ~ U[0, 2*pi),
  from ``SeedSequence([seed, tensor_id])``.
* X[t, y, x, h, d] = sin(2*pi*(f_t*t + f_y*y + f_x*x) + phi) + eps with
  eps ~ N(0, noise_std**2); the noise of absolute latent frame t comes from
  ``SeedSequence([seed, tensor_id, t])`` so that any window of frames is
  regenerated identically, which makes streams reproducible.
* The field is made in float64, rounded to float32, then (for bf16 inputs)
  to bfloat16 with round-to-nearest-even.

Token layout of the returned arrays: [B][T][H][W][NH][D], tokens ordered
(t, y, x) row-major with the heads split out of the channel axis.

``field_frames_device`` builds the same smooth field on a torch device with
device-side noise (same distribution, different noise values). It exists so
the benchmark can put hundreds of distinct steps into HBM quickly; parity
tests always use the host generator.
"""
from __future__ import annotations

import math
import os

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2}
FIELD_IDS = {**TENSOR_IDS, "dout": 3}  # dout: the upstream gradient of a backward test


def field_params(seed: int, tensor_id: int, heads: int, head_dim: int):
    """Per (head, channel) frequencies and phase of the smooth field."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, tensor_id]))
    ft = rng.uniform(-1.0 / 16.0, 1.0 / 16.0, size=(heads, head_dim))
    fy = rng.uniform(-1.0 / 48.0, 1.0 / 48.0, size=(heads, head_dim))
    fx = rng.uniform(-1.0 / 48.0, 1.0 / 48.0, size=(heads, head_dim))
    phi = rng.uniform(0.0, 2.0 * math.pi, size=(heads, head_dim))
    return ft, fy, fx, phi


def _frame(seed, tensor_id, params, t, y, x, noise_std):
    ft, fy, fx, phi = params
    frame = np.sin(2.0 * math.pi * (ft * t + fy * y + fx * x) + phi)
    if noise_std:
        rng = np.random.default_rng(np.random.SeedSequence([seed, tensor_id, t]))
        frame += noise_std * rng.standard_normal(frame.shape)
    return frame


def field_frames(seed: int, tensor_id: int, heads: int, head_dim: int,
                 height: int, width: int, t0: int, t1: int,
                 batch: int = 1, noise_std: float = 0.5) -> np.ndarray:
    """float64 field for absolute latent frames [t0, t1): [B][T][H][W][NH][D].

    Batch entries b > 0 use seed + 7919*b so that they differ. Frames are
    independent (own noise seed), so they are generated on a thread pool.
    """
    from concurrent.futures import ThreadPoolExecutor

    out = np.empty((batch, t1 - t0, height, width, heads, head_dim), np.float64)
    y = np.arange(height, dtype=np.float64)[:, None, None, None]
    x = np.arange(width, dtype=np.float64)[None, :, None, None]
    jobs = []
    for b in range(batch):
        s = seed + 7919 * b
        params = field_params(s, tensor_id, heads, head_dim)
        for ti, t in enumerate(range(t0, t1)):
            jobs.append((b, ti, s, params, t))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))

    def work(job):
        b, ti, s, params, t = job
        out[b, ti] = _frame(s, tensor_id, params, t, y, x, noise_std)

    if workers == 1:
        for j in jobs:
            work(j)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(work, jobs))
    return out


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bfloat16 (round to nearest even), as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def make_qkv(seed: int, heads: int, head_dim: int, height: int, width: int,
             t0: int, t1: int, dtype: str = "bf16", batch: int = 1,
             which=("q", "k", "v"), noise_std: float = 0.5):
    """Host inputs for frames [t0, t1).

    Returns a dict name -> (storage array, float64 values). Storage is uint16
    bfloat16 bits for dtype "bf16" and float32 for "f32"; the float64 array
    holds exactly the stored values, widened.
    """
    res = {}
    for name in which:
        f = field_frames(seed, FIELD_IDS[name], heads, head_dim, height, width,
                         t0, t1, batch=batch, noise_std=noise_std)
        if dtype == "bf16":
            bits = round_bf16_bits(f)
            res[name] = (bits, bf16_bits_to_f64(bits))
        elif dtype == "f32":
            f32 = f.astype(np.float32)
            res[name] = (f32, f32.astype(np.float64))
        else:
            raise ValueError(f"unknown dtype {dtype!r}")
    return res


def field_frames_device(seed: int, tensor_id: int, heads: int, head_dim: int,
                        height: int, width: int, t0: int, t1: int, device,
                        dtype, batch: int = 1, noise_std: float = 0.5):
    """Same smooth field built on a torch device, device-side noise.

    Returns a tensor [B][T][H][W][NH][D] of ``dtype`` on ``device``.
    """
    import torch

    out = torch.empty((batch, t1 - t0, height, width, heads, head_dim),
                      dtype=dtype, device=device)
    y = torch.arange(height, device=device, dtype=torch.float64)[:, None, None, None]
    x = torch.arange(width, device=device, dtype=torch.float64)[None, :, None, None]
    for b in range(batch):
        s = seed + 7919 * b
        ft, fy, fx, phi = (torch.as_tensor(a, device=device)
                           for a in field_params(s, tensor_id, heads, head_dim))
        for ti, t in enumerate(range(t0, t1)):
            arg = 2.0 * math.pi * (ft * t + fy * y + fx * x) + phi
            frame = torch.sin(arg).float()
            if noise_std:
                g = torch.Generator(device=device)
                g.manual_seed((s * 1000003 + tensor_id * 10007 + t) & 0x7FFFFFFFFFFF)
                frame += noise_std * torch.randn(frame.shape, generator=g,
                                                 device=device, dtype=torch.float32)
            out[b, ti] = frame.to(dtype)
    return out


def random_lists(seed: int, batch: int, heads: int, n_tb: int, n_s: int, k_of_tb, kmax: int):
    """Seeded block index lists for tests of the list consumers.

    Row (b, h, i) of temporal block t = i // n_s holds min(k_of_tb(t),
    (t + 1) * n_s) distinct ids drawn uniformly from [0, (t + 1) * n_s),
    ascending and padded with -1 up to kmax (the shape of causal lists,
    whose length grows with t). Returns (sel_idx int32 [B][NH][nq][kmax],
    sel_cnt int32 [B][NH][nq], nested lists [B][NH][nq])."""
    nq = n_tb * n_s
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x115]))
    idx = np.full((batch, heads, nq, kmax), -1, dtype=np.int32)
    cnt = np.zeros((batch, heads, nq), dtype=np.int32)
    nested = [[[None] * nq for _ in range(heads)] for _ in range(batch)]
    for b in range(batch):
        for h in range(heads):
            for i in range(nq):
                t = i // n_s
                k = min(int(k_of_tb(t)), (t + 1) * n_s, kmax)
                ids = np.sort(rng.choice((t + 1) * n_s, size=k, replace=False)).astype(np.int32)
                idx[b, h, i, :k] = ids
                cnt[b, h, i] = k
                nested[b][h][i] = ids.tolist()
    return idx, cnt, nested
