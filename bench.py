"""LCSA benchmark: one streaming step = partition+pool -> draft mask ->
block-sparse attention -> cache evict, through the C-ABI, on one GPU.

Default workload: the steady-state streaming step at 768x1408 (2 new latent
frames of 48x88 tokens, 12 heads, head_dim 128, bf16, a 6-frame KV cache,
11x11 block window, k = 20 % of each row's candidates), 100 timed steps of a
seeded stream. Every step consumes its own frames, resident in HBM before
the timed region starts.

Prints ONE JSON line (rank 0, N = 1):
  value       whole-step throughput: attention FLOPs of the computed block
              pairs / step time (TFLOP/s)
  ms_per_step mean wall time of one step on the GPU (HIP events)
  roofline    the attention kernel (dominant) against the bf16 MFMA peak,
              its duration measured with HIP events on the launch stream
  cpu_baseline the float64 oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="step_768x1408")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-heads", type=int, default=12)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the warmup, as "
                         "the calibration kernel for rocprofv3 FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per attention launch measured by rocprofv3 counters")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the LCSA path "
              "shards by head with no communication, so one GPU's figure is the per-GPU rate.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_attention_03_amd import lcsa as L
    from block_sparse_attention_03_amd import synth
    from block_sparse_attention_03_amd.workloads import WORKLOADS, attention_flops_per_pair

    w = WORKLOADS[args.workload]
    K = args.steps if args.steps is not None else max(w.steps, 20)
    W = args.warmup
    dev = torch.device("cuda:0")
    L.load_library()
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = L.LCSA_BF16 if w.dtype == "bf16" else L.LCSA_F32

    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- inputs resident in HBM: cache frames + one fresh chunk per step
    n_steps = K + W
    t_first = w.cache_frames
    t_end = t_first + w.frames * n_steps
    qkv = {}
    for name, tid in synth.TENSOR_IDS.items():
        t0 = t_first if name == "q" else 0
        qkv[name] = synth.field_frames_device(w.seed, tid, w.heads, w.head_dim, w.height, w.width,
                                              t0, t_end, dev, tdt, batch=w.batch)
    torch.cuda.synchronize()

    cache = L.KVCache(w.batch, w.heads, w.head_dim, w.height, w.width, tdt, w.n_slots, device=dev)
    params = L.make_params(local_range=w.local_range, border=w.border, topk_fixed=w.topk_fixed,
                           ratio=w.ratio, scale_by_resolution=w.scale_by_resolution,
                           out_hw=w.out_hw, ratio_base=w.ratio_base)
    geom = L.make_geom(w.batch, w.heads, w.head_dim, w.frames, w.height, w.width, code)
    if w.cache_frames:
        first = cache.append(w.cache_frames // 2, 0)
        gp = L.make_geom(w.batch, w.heads, w.head_dim, w.cache_frames, w.height, w.width, code)
        L.lcsa_partition_pool(gp, None, qkv["k"][:, :w.cache_frames], qkv["v"][:, :w.cache_frames],
                              None, None, cache.c, first)

    # buffers sized for the steady state: kmax from a metadata-only copy of
    # the ring with the first chunk appended
    import ctypes
    probe = L.KvCacheStruct()
    ctypes.memmove(ctypes.byref(probe), ctypes.byref(cache.c), ctypes.sizeof(probe))
    tb_first = t_first // 2
    L.lcsa_kv_cache_append(probe, w.frames // 2, tb_first)
    kmax = L.lcsa_max_topk(geom, tb_first, probe, params)
    bufs = L.StepBuffers(geom, kmax, device=dev)

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_steps)]
    keep = w.cap_tb if w.cache_frames else None

    def step(n, timed_attn=None):
        tb = tb_first + n * (w.frames // 2)
        f0 = t_first + n * w.frames
        fq = n * w.frames
        q = qkv["q"][:, fq:fq + w.frames]
        k = qkv["k"][:, f0:f0 + w.frames]
        v = qkv["v"][:, f0:f0 + w.frames]
        slot = cache.append(w.frames // 2, tb)
        L.lcsa_partition_pool(geom, q, k, v, bufs.q_blk, bufs.q_pool, cache.c, slot, stream)
        L.lcsa_draft_mask(geom, bufs.q_pool, tb, cache.c, params, kmax, bufs.sel_idx,
                          bufs.sel_cnt, None, stream)
        if timed_attn is not None:
            timed_attn[0].record(stream)
        L.lcsa_block_sparse_attn(geom, bufs.q_blk, cache.c, bufs.sel_idx, bufs.sel_cnt, kmax,
                                 bufs.out, None, 0.0, stream)
        if timed_attn is not None:
            timed_attn[1].record(stream)
        if keep is not None:
            cache.evict(keep)
        else:  # cold chunks: start each step from an empty cache
            cache.evict(0)

    for n in range(W):
        step(n)
    torch.cuda.synchronize()
    pairs = int(bufs.sel_cnt.to(torch.int64).sum().item())

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for n in range(W, W + K):
        step(n, ev[n])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    attn_ms = [ev[n][0].elapsed_time(ev[n][1]) for n in range(W, W + K)]
    ms_step = total_ms / K
    attn_avg = float(np.mean(attn_ms))
    flops_pair = attention_flops_per_pair(w.head_dim)
    flops_step = pairs * flops_pair
    value = flops_step / (ms_step * 1e-3) / 1e12
    achieved = flops_step / (attn_avg * 1e-3) / 1e12

    traffic = None
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f)
        if tj.get("workload") == args.workload:
            traffic = tj.get("bytes_per_launch")
    except (OSError, ValueError):
        pass

    result = {
        "metric": "block-sparse attn effective TFLOP/s + ms per streaming step at 768x1408",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded smooth field + N(0,0.5^2) noise, device-generated)",
        "config": {"workload": w.name, "heads": w.heads, "head_dim": w.head_dim,
                   "token_grid": [w.frames, w.height, w.width], "cache_frames": w.cache_frames,
                   "local_range": w.local_range, "selected_pairs_per_step": pairs,
                   "kmax": kmax, "parallelism": "single GPU"},
        "attn_ms": round(attn_avg, 4),
        "attn_ms_p10_p90": [round(float(np.percentile(attn_ms, 10)), 4),
                            round(float(np.percentile(attn_ms, 90)), 4)],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_heads, flops_pair)
    print(json.dumps(result), flush=True)


def cpu_baseline(w, sample_heads, flops_pair):
    """The float64 oracle, as it stands, on one streaming step of the same
    workload (the first `sample_heads` heads), timed on the host."""
    import numpy as np

    from block_sparse_attention_03_amd import synth
    from oracle import lcsa_oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    nh = min(sample_heads, w.heads)
    p = O.SelectParams(local_range=w.local_range, border=w.border, topk_fixed=w.topk_fixed,
                       ratio_num=w.ratio[0], ratio_den=w.ratio[1],
                       scale_by_resolution=w.scale_by_resolution, out_h=w.out_hw[0],
                       out_w=w.out_hw[1], ratio_base=w.ratio_base)
    cache = O.KVCache(cap_tb=w.cap_tb)
    if w.cache_frames:
        d0 = synth.make_qkv(w.seed, nh, w.head_dim, w.height, w.width, 0, w.cache_frames,
                            dtype=w.dtype, which="kv")
        O.prime_cache(cache, d0["k"][1], d0["v"][1], 0)
    t0 = w.cache_frames
    d = synth.make_qkv(w.seed, nh, w.head_dim, w.height, w.width, t0, t0 + w.frames, dtype=w.dtype)
    tic = time.perf_counter()
    res = O.lcsa_step(d["q"][1], d["k"][1], d["v"][1], cache, t0 // 2, p)
    sec = time.perf_counter() - tic
    pairs = int(sum(len(r) for bh in res.sel for hh in bh for r in hh))
    return {"value": round(pairs * flops_pair / sec / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(sec, 3),
            "sample": f"one full LCSA step (partition, pool, draft, top-k, attention) of the "
                      f"same workload, heads 0..{nh - 1} of {w.heads}, float64 NumPy"}


if __name__ == "__main__":
    main()
