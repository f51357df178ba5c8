"""LCSA benchmark: one streaming step = partition+pool -> draft mask ->
block-sparse attention -> cache evict, through the C-ABI, on one GPU, one
kernel after the other on one stream.

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
import re
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
    ap.add_argument("--q-blocks", action="store_true",
                    help="have the partition write the query blocks (q_blk) and the attention "
                         "read q from them, instead of reading q in token layout (measured "
                         "slower: q_blk is an extra write and read of the whole of q)")
    ap.add_argument("--no-draft-workspace", action="store_true",
                    help="give the draft no workspace: its whole-grid windows then run the "
                         "fused scoring and selection kernel instead of the split pair")
    ap.add_argument("--cpu-sample-heads", type=int, default=12)
    ap.add_argument("--cpu-sample-steps", type=int, default=4)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the warmup, as "
                         "the calibration kernel for rocprofv3 FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per attention launch measured by rocprofv3 counters")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn the rocprofv3 output of a --kernel-trace --stats run "
                         "and of --pmc FETCH_SIZE / --pmc WRITE_SIZE runs of this script into "
                         "profiles/<kernels>_<workload>.md and the workload's traffic.json entry")
    ap.add_argument("--sq2-dir", default=None,
                    help="with --summarize-profiles: a rocprofv3 --pmc run of SQ_ISSUE_COUNTERS")
    ap.add_argument("--sq-dir", default=None,
                    help="with --summarize-profiles: the output of a rocprofv3 --pmc run of this "
                         "script with the SQ_COUNTERS set (instruction mix, matrix-core busy "
                         "cycles, LDS bank conflicts, GPU clock)")
    ap.add_argument("--bench-log", default=None,
                    help="with --summarize-profiles: a log whose last line is this script's JSON")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the LCSA path "
              "shards by head with no communication, so one GPU's figure is the per-GPU rate.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_attention_03_amd import lcsa as L
    from block_sparse_attention_03_amd import synth
    from block_sparse_attention_03_amd.workloads import (WORKLOADS, attention_flops_per_pair,
                                                         backward_flops_per_pair,
                                                         segment_pair_quarters)

    w = WORKLOADS[args.workload]
    specs = [WORKLOADS[n] for n in w.layers] if w.layers else [w]
    for sp in specs:  # the layers of a stack share the step's token geometry
        assert (sp.heads, sp.head_dim, sp.dtype, sp.height, sp.width, sp.frames, sp.batch) == \
            (w.heads, w.head_dim, w.dtype, w.height, w.width, w.frames, w.batch), sp.name
    K = args.steps if args.steps is not None else max(w.steps, 20)
    W = args.warmup
    dev = torch.device("cuda:0")
    L.load_library()
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = L.LCSA_BF16 if w.dtype == "bf16" else L.LCSA_F32

    if args.copy_probe_mib:
        # the first device-to-device copy of the process: a plain copy kernel
        # of known size that calibrates the FETCH_SIZE / WRITE_SIZE counters
        src = torch.ones(args.copy_probe_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- inputs resident in HBM: cache frames + one fresh chunk per step
    n_steps = K + W
    t_first = max(sp.cache_frames for sp in specs)
    t_end = t_first + w.frames * n_steps
    qkv = {}
    for name, tid in synth.TENSOR_IDS.items():
        t0 = t_first if name == "q" else 0
        qkv[name] = synth.field_frames_device(w.seed, tid, w.heads, w.head_dim, w.height, w.width,
                                              t0, t_end, dev, tdt, batch=w.batch)
    torch.cuda.synchronize()
    geom = L.make_geom(w.batch, w.heads, w.head_dim, w.frames, w.height, w.width, code)
    stream = torch.cuda.current_stream()
    tb_first = t_first // 2

    import ctypes

    class Layer:
        """One attention layer of the step: its own ring cache, list rule
        (draft top-k, local lists or Stage-1 segment lists) and buffers."""

        def __init__(self, sp):
            self.sp = sp
            self.seg = list(sp.frame_seg) if sp.frame_seg else None
            self.cache = L.KVCache(w.batch, w.heads, w.head_dim, w.height, w.width, tdt,
                                   sp.n_slots, device=dev)
            self.params = L.make_params(local_range=sp.local_range, border=sp.border,
                                        topk_fixed=sp.topk_fixed, ratio=sp.ratio,
                                        scale_by_resolution=sp.scale_by_resolution,
                                        out_hw=sp.out_hw, ratio_base=sp.ratio_base)
            if sp.cache_frames:
                t0 = t_first - sp.cache_frames
                first = self.cache.append(sp.cache_frames // 2, t0 // 2)
                gp = L.make_geom(w.batch, w.heads, w.head_dim, sp.cache_frames, w.height,
                                 w.width, code)
                L.lcsa_partition_pool(gp, None, qkv["k"][:, t0:t_first], qkv["v"][:, t0:t_first],
                                      None, None, self.cache.c, first)
            # buffers sized for the steady state: kmax from a metadata-only
            # copy of the ring with the first chunk appended
            probe = L.KvCacheStruct()
            ctypes.memmove(ctypes.byref(probe), ctypes.byref(self.cache.c), ctypes.sizeof(probe))
            L.lcsa_kv_cache_append(probe, w.frames // 2, tb_first)
            if self.seg:
                self.kmax = L.lcsa_segment_max_list(geom, self.seg)
            elif sp.lists == "local":
                self.kmax = L.lcsa_max_candidates(geom, tb_first, probe, self.params)
            else:
                self.kmax = L.lcsa_max_topk(geom, tb_first, probe, self.params)
            self.bufs = L.StepBuffers(geom, self.kmax, device=dev, with_lse=sp.backward,
                                      with_q_blk=args.q_blocks)
            # the draft's workspace (its split path at the whole-grid windows
            # of about a thousand candidates and more; 0 bytes elsewhere)
            nb = 0 if (self.seg or sp.lists == "local" or args.no_draft_workspace) else \
                L.lcsa_draft_workspace_size(geom, self.cache.c, self.params)
            self.dws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
            self.keep = sp.cap_tb if sp.cache_frames else 0  # cold chunks: empty after each step
            if sp.backward:  # training shape: the keys are the chunk's own blocks
                assert sp.cache_frames == 0 and not self.seg
                self.dout = synth.field_frames_device(w.seed, synth.FIELD_IDS["dout"], w.heads,
                                                      w.head_dim, w.height, w.width, 0, w.frames,
                                                      dev, tdt, batch=w.batch)
                self.ws = torch.empty(L.lcsa_attn_bwd_workspace_size(geom), dtype=torch.uint8,
                                      device=dev)
                self.grads = [torch.empty_like(self.dout) for _ in range(3)]

        def run(self, tb, q, k, v, ev=None, evb=None, evk=None):
            c, b = self.cache, self.bufs
            slot = c.append(w.frames // 2, tb)
            if evk is not None:
                evk[0].record(stream)
            L.lcsa_partition_pool(geom, q, k, v, b.q_blk, b.q_pool, c.c, slot, stream)
            if evk is not None:
                evk[1].record(stream)
            if self.seg:
                L.lcsa_segment_lists(geom, tb, c.c, self.seg, self.kmax, b.sel_idx, b.sel_cnt,
                                     stream)
            elif self.sp.lists == "local":
                L.lcsa_local_lists(geom, tb, c.c, self.params, self.kmax, b.sel_idx, b.sel_cnt,
                                   stream)
            else:
                L.lcsa_draft_mask(geom, b.q_pool, tb, c.c, self.params, self.kmax, b.sel_idx,
                                  b.sel_cnt, None, stream, workspace=self.dws)
            if ev is not None:
                ev[0].record(stream)
            if self.seg and b.q_blk is not None:
                L.lcsa_segment_attn(geom, b.q_blk, tb, c.c, self.seg, b.sel_idx, b.sel_cnt,
                                    self.kmax, b.out, None, 0.0, stream)
            elif self.seg:
                L.lcsa_segment_attn_tok(geom, q, tb, c.c, self.seg, b.sel_idx, b.sel_cnt,
                                        self.kmax, b.out, None, 0.0, stream)
            elif b.q_blk is not None:
                L.lcsa_block_sparse_attn(geom, b.q_blk, c.c, b.sel_idx, b.sel_cnt, self.kmax,
                                         b.out, b.lse, 0.0, stream)
            else:
                L.lcsa_block_sparse_attn_tok(geom, q, c.c, b.sel_idx, b.sel_cnt, self.kmax,
                                             b.out, b.lse, 0.0, stream)
            if ev is not None:
                ev[1].record(stream)
            if self.sp.backward:
                if evb is not None:
                    evb[0].record(stream)
                L.lcsa_block_sparse_attn_bwd(geom, q, k, v, b.out, self.dout, b.lse, b.sel_idx,
                                             b.sel_cnt, self.kmax, *self.grads, self.ws,
                                             stream=stream)
                if evb is not None:
                    evb[1].record(stream)
            c.evict(self.keep)

        def flops(self):
            fp = attention_flops_per_pair(w.head_dim)
            if self.seg:  # only the frame pairs of a listed block pair that share a segment
                quarters = sum(segment_pair_quarters(self.seg).values()) * w.nS * w.nS
                return quarters * w.batch * w.heads * fp // 4
            pairs = int(self.bufs.sel_cnt.to(torch.int64).sum().item())
            return pairs * (fp + (backward_flops_per_pair(w.head_dim) if self.sp.backward else 0))

    layers = [Layer(sp) for sp in specs]
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in layers] for _ in range(n_steps)]

    evb = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in layers] for _ in range(n_steps)]
    # partition start, partition end (= list kernel start): the lists end where
    # the attention's start event is recorded
    evk = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in layers] for _ in range(n_steps)]

    def step(n, timed=False):
        tb = tb_first + n * (w.frames // 2)
        f0 = t_first + n * w.frames
        fq = n * w.frames
        q = qkv["q"][:, fq:fq + w.frames]
        k = qkv["k"][:, f0:f0 + w.frames]
        v = qkv["v"][:, f0:f0 + w.frames]
        for li, layer in enumerate(layers):
            layer.run(tb, q, k, v, ev[n][li] if timed else None, evb[n][li] if timed else None,
                      evk[n][li] if timed else None)

    for n in range(W):
        step(n)
    torch.cuda.synchronize()
    pairs = sum(int(la.bufs.sel_cnt.to(torch.int64).sum().item()) for la in layers)
    flops_step = sum(la.flops() for la in layers)

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for n in range(W, W + K):
        step(n, timed=True)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    # attention time of one step: its launches (one per layer), summed
    attn_ms = [sum(e0.elapsed_time(e1) for (e0, e1) in ev[n]) for n in range(W, W + K)]
    has_bwd = any(la.sp.backward for la in layers)
    if has_bwd:  # the attention of a training step: forward and backward launches
        bwd_ms = [sum(e0.elapsed_time(e1) for (e0, e1), la in zip(evb[n], layers)
                      if la.sp.backward) for n in range(W, W + K)]
        attn_ms = [a + b_ for a, b_ in zip(attn_ms, bwd_ms)]
    ms_step = total_ms / K
    attn_avg = float(np.mean(attn_ms))
    flops_pair = attention_flops_per_pair(w.head_dim)
    kmax = max(la.kmax for la in layers)
    seg = layers[0].seg
    value = flops_step / (ms_step * 1e-3) / 1e12
    achieved = flops_step / (attn_avg * 1e-3) / 1e12

    traffic = traffic_for(args.traffic_json, args.workload)

    # ---- the other kernels of the step, against HBM: algorithmic bytes of
    # one launch (what the step must move) over the launch's mean duration
    timed = range(W, W + K)
    part_ms = [sum(a.elapsed_time(b_) for (a, b_) in evk[n]) for n in timed]
    lists_ms = [sum(b_.elapsed_time(e0) for (a, b_), (e0, e1) in zip(evk[n], ev[n])) for n in timed]
    esz = 2 if w.dtype == "bf16" else 4
    blk_heads = w.batch * w.heads * w.nq  # (query block, head) pairs of a chunk
    part_bytes = blk_heads * (5 * 128 * w.head_dim * esz + 2 * w.head_dim * 8
                              + (128 * w.head_dim * esz if args.q_blocks else 0))
    part_bytes *= len(layers)
    lists_bytes = 0
    lists_kind = set()
    for la in layers:
        # the draft's view: the cached TBs (steady state) and the chunk's own
        view_keys = ((la.sp.cap_tb if la.sp.cache_frames else 0) + w.frames // 2) * w.nS
        sel = blk_heads * (la.kmax + 1) * 4
        if la.seg or la.sp.lists == "local":
            lists_bytes += sel
            lists_kind.add("segment lists" if la.seg else "local lists")
        else:  # pooled queries and the pooled keys of the view in, ids out
            lists_bytes += blk_heads * w.head_dim * 8 + w.batch * w.heads * view_keys * \
                w.head_dim * 8 + sel
            lists_kind.add("draft mask")

    def hbm(byts, ms):
        gbs = byts / (ms * 1e-3) / 1e9
        return {"us": round(ms * 1e3, 2), "algorithmic_bytes": int(byts), "gb_s": round(gbs, 1),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}

    kernels = {
        "partition_pool": hbm(part_bytes, float(np.mean(part_ms))),
        "lists": {"kind": " + ".join(sorted(lists_kind)), **hbm(lists_bytes, float(np.mean(lists_ms)))},
        "attention": {"us": round(attn_avg * 1e3, 2), "tflop_s": round(achieved, 1),
                      "mfma_frac": round(achieved / PEAK_BF16_TFLOPS, 4)},
    }

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
                   **({"frame_segments": seg} if seg else {}),
                   **({"layers": list(w.layers)} if w.layers else {}),
                   "kmax": kmax, "q_read_from": "q_blk" if args.q_blocks else "token layout",
                   "streams": 1, "parallelism": "single GPU"},
        "attn_ms": round(attn_avg, 4),
        **({"bwd_ms": round(float(np.mean(bwd_ms)), 4)} if has_bwd else {}),
        "attn_ms_median": round(float(np.median(attn_ms)), 4),
        "attn_ms_p10_p90": [round(float(np.percentile(attn_ms, 10)), 4),
                            round(float(np.percentile(attn_ms, 90)), 4)],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "kernels": kernels,
    }

    if not args.no_cpu_baseline:
        single = (not w.layers and not w.backward and not w.frame_seg and w.lists == "draft")
        if single:  # the oracle on the run's own last steps, compared with the GPU's last step
            la = layers[0]
            last = W + K - 1
            result["cpu_baseline"] = cpu_baseline_run(
                w, qkv, t_first, last, min(args.cpu_sample_steps, last + 1),
                la.bufs, flops_pair)
        else:
            result["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_heads,
                                                  args.cpu_sample_steps, flops_pair)
    print(json.dumps(result), flush=True)


def _cpu_cores():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                        None)
    except OSError:
        return None


def _tied_ok(scores, k, gpu_ids, ref_ids):
    """Selection rule of the parity check: exact, or, where the k-th and
    (k+1)-th draft scores are within 1e-5 relative (+1e-7), any set of k
    holding every score above the tie and none below it. Returns (ok, tied)."""
    import numpy as np
    gpu = sorted(int(x) for x in gpu_ids)
    fin = np.isfinite(scores)
    n = int(fin.sum())
    if len(gpu) != k or len(set(gpu)) != k or not all(fin[j] for j in gpu):
        return False, False
    if k == 0 or k >= n:
        return gpu == sorted(np.nonzero(fin)[0].tolist()), False
    vals = np.sort(scores[fin])[::-1]
    sk, sk1 = vals[k - 1], vals[k]
    tol = 1e-5 * max(abs(sk), abs(sk1)) + 1e-7
    if abs(sk - sk1) > tol:
        return gpu == sorted(int(x) for x in ref_ids), False
    must = set(np.nonzero(fin & (scores > sk + tol))[0].tolist())
    may = set(np.nonzero(fin & (scores >= sk1 - tol))[0].tolist())
    return must <= set(gpu) <= may, True


def cpu_baseline_run(w, qkv, t_first, last, n_steps, bufs, flops_pair):
    """The float64 oracle, as it stands, on the last `n_steps` timed steps of
    this very run (their device-generated q, k, v copied to the host; the
    oracle's cache primed with the frames before them), timed on the host.
    The last of them is then compared with the GPU's results for that step,
    which are still in `bufs`: the selection on every row (exact, or the tie
    rule), and the output and log-sum-exp on every row."""
    import math

    import numpy as np

    from oracle import lcsa_oracle as O

    F = w.frames

    def host(t):
        return t.float().cpu().numpy().astype(np.float64)

    p = O.SelectParams(local_range=w.local_range, border=w.border, topk_fixed=w.topk_fixed,
                       ratio_num=w.ratio[0], ratio_den=w.ratio[1],
                       scale_by_resolution=w.scale_by_resolution, out_h=w.out_hw[0],
                       out_w=w.out_hw[1], ratio_base=w.ratio_base)
    first = last - n_steps + 1
    cache = O.KVCache(cap_tb=w.cap_tb)
    if w.cache_frames:
        c0 = t_first + first * F - w.cache_frames
        O.prime_cache(cache, host(qkv["k"][:, c0:c0 + w.cache_frames]),
                      host(qkv["v"][:, c0:c0 + w.cache_frames]), c0 // 2)
    sec, pairs, res = 0.0, 0, None
    for n in range(first, last + 1):
        f0 = t_first + n * F
        q, k, v = host(qkv["q"][:, n * F:(n + 1) * F]), host(qkv["k"][:, f0:f0 + F]), \
            host(qkv["v"][:, f0:f0 + F])
        tic = time.perf_counter()
        res = O.lcsa_step(q, k, v, cache, f0 // 2, p)
        sec += time.perf_counter() - tic
        pairs += int(sum(len(r) for bh in res.sel for hh in bh for r in hh))
        if not w.cache_frames:
            cache = O.KVCache(cap_tb=w.cap_tb)  # a cold start each step
    # parity of the last step
    sel = bufs.sel_idx.cpu().numpy()
    cnt = bufs.sel_cnt.cpu().numpy()
    out_g = O.partition(host(bufs.out))
    out_r = O.partition(res.out)
    kb, vb = res.key_blocks
    mism, tied, rows = 0, 0, 0
    got, exp = [], []
    for b in range(w.batch):
        for h in range(w.heads):
            for i in range(w.nq):
                rows += 1
                kr = int(res.kcount[i])
                ids = sel[b, h, i, :max(int(cnt[b, h, i]), 0)]
                ok, t = _tied_ok(res.scores[b, h, i], kr, ids, res.sel[b][h][i])
                tied += t
                if not ok or int(cnt[b, h, i]) != kr:
                    mism += 1
                    continue
                got.append(out_g[b, h, i])
                if sorted(int(x) for x in ids) == list(res.sel[b][h][i]):
                    exp.append(out_r[b, h, i])
                else:  # a tied row: the oracle's attention over the GPU's set
                    exp.append(O.sparse_attention_row(res.q_blocks[b, h, i], kb[b, h], vb[b, h],
                                                      np.array(sorted(int(x) for x in ids)),
                                                      1.0 / math.sqrt(w.head_dim))[0])
    got, exp = np.stack(got), np.stack(exp)
    d = got - exp
    max_abs = float(np.abs(d).max())
    rel = float(np.linalg.norm(d) / np.linalg.norm(exp))
    tol = (2e-2, 5e-3) if w.dtype == "bf16" else (1e-4, 1e-5)
    parity = {"step": last, "rows": rows, "selection_mismatches": mism, "tied_rows": tied,
              "max_abs": float(f"{max_abs:.3e}"), "rel_l2": float(f"{rel:.3e}"),
              "tolerance": {"max_abs": tol[0], "rel_l2": tol[1]},
              "pass": mism == 0 and max_abs <= tol[0] and rel <= tol[1]}
    return {"value": round(pairs * flops_pair / sec / 1e12, 6), "unit": "TFLOP/s",
            "cores": _cpu_cores(), "kind": "oracle", "seconds": round(sec, 3),
            "cpu_model": _cpu_model(),
            "sample": f"the last {n_steps} timed steps of this run (steps {first}..{last}), every "
                      f"head and row: full LCSA steps (partition, pool, draft, top-k, attention, "
                      f"cache update) in float64 NumPy on the run's own inputs",
            "parity": parity}


def cpu_baseline(w, sample_heads, sample_steps, flops_pair):
    """The float64 oracle, as it stands, on the first `sample_steps`
    consecutive steps of the same workload's stream (the first
    `sample_heads` heads), timed on the host."""
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
    steps = sample_steps if w.cache_frames else 1
    sec, pairs = 0.0, 0
    for n in range(steps):
        t0 = w.cache_frames + n * w.frames
        d = synth.make_qkv(w.seed, nh, w.head_dim, w.height, w.width, t0, t0 + w.frames,
                           dtype=w.dtype)
        tic = time.perf_counter()
        res = O.lcsa_step(d["q"][1], d["k"][1], d["v"][1], cache, t0 // 2, p)
        sec += time.perf_counter() - tic
        pairs += int(sum(len(r) for bh in res.sel for hh in bh for r in hh))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         None)
    except OSError:
        pass
    return {"value": round(pairs * flops_pair / sec / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(sec, 3), "cpu_model": model,
            "sample": f"{steps} consecutive full LCSA steps (partition, pool, draft, top-k, "
                      f"attention, cache update) of the same workload's stream, heads 0..{nh - 1} "
                      f"of {w.heads}, float64 NumPy"}


ATTN_KERNEL = "attn_bf16"
# The files whose text makes up the attention kernel. traffic.json keeps a
# digest of them and of the kernel's compile flags from when its counters
# were summarized; a run on other sources or flags reports traffic as null
# instead of figures taken on older code.
ATTN_SOURCES = ("block_sparse_attention_03_amd/csrc/sparse_attn.hip",
                "block_sparse_attention_03_amd/csrc/mfma_tiles.h",
                "block_sparse_attention_03_amd/csrc/lcsa_kernels.h")


def attn_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    # the compile flags shape the machine code as much as the sources do
    from block_sparse_attention_03_amd import build_lib
    h.update(" ".join(build_lib.HIP_FLAGS + build_lib.EXTRA.get("sparse_attn.hip", [])).encode())
    return h.hexdigest()[:16]


def traffic_for(path: str, workload: str):
    """Counter-derived HBM bytes per attention launch of `workload`, or None
    when none were taken or they were taken on other kernel sources."""
    try:
        with open(path) as f:
            entry = json.load(f).get(workload) or {}
    except (OSError, ValueError):
        return None
    if entry.get("source_digest") != attn_source_digest():
        return None
    return entry.get("bytes_per_launch")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def _short(name):
    m = re.search(r"lcsa::\(anonymous namespace\)::(\w+)(<[^>]*>)?", name)
    return m.group(1) + (m.group(2) or "") if m else None


def _counter_per_dispatch(d, counter):
    """(calibration copy value, mean value over the attention dispatches, n) in KiB."""
    rows = [r for r in _csv_rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    copy = next((float(r["Counter_Value"]) for r in rows if COPY_KERNEL in r["Kernel_Name"]), None)
    attn = [float(r["Counter_Value"]) for r in rows if ATTN_KERNEL in r["Kernel_Name"]]
    if copy is None or not attn:
        raise SystemExit(f"{d}: calibration copy or attention dispatches missing for {counter}")
    return copy, sum(attn) / len(attn), len(attn)


# The shader-sequencer counters of the instruction-mix run: one rocprofv3
# --pmc pass (at most 8 SQ and 2 GRBM counters).
SQ_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS",
               "SQ_LDS_BANK_CONFLICT", "SQ_WAVES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")
N_SIMDS, N_XCDS = 1024, 8  # MI355X: 256 CUs x 4 SIMDs, 8 XCDs
# The issue-state counters of a second pass: where the waves' cycles go
# (waiting on counters and barriers, waiting to issue, issuing VALU or LDS
# work) and how many of the matrix cores' busy cycles also issued a vector
# instruction (co-execution). The SQ_WAVE_CYCLES / SQ_WAIT_* / SQ_ACTIVE_*
# counters are in units of 4 cycles.
SQ_ISSUE_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                     "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_VALU_MFMA_COEXEC_CYCLES",
                     "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def _per_kernel_counters(d, names):
    """{kernel short name: {counter: mean value per dispatch}} over the LCSA
    kernels of a --pmc run, plus the calibration copy's values."""
    rows = _csv_rows(d, "counter_collection.csv")
    acc, disp, copy = {}, {}, {}
    for r in rows:
        c = r["Counter_Name"]
        if c not in names:
            continue
        v = float(r["Counter_Value"])
        if COPY_KERNEL in r["Kernel_Name"]:
            copy.setdefault(c, v)  # the first copy of the process
            continue
        k = _short(r["Kernel_Name"])
        if not k:
            continue
        acc.setdefault(k, {}).setdefault(c, 0.0)
        acc[k][c] += v
        disp.setdefault(k, {}).setdefault(c, set()).add(r["Dispatch_Id"])
    return {k: {c: v / len(disp[k][c]) for c, v in cs.items()} for k, cs in acc.items()}, copy


def summarize_profiles(args):
    """Host-only: write the kernel-trace summary and the counter-derived HBM
    traffic of the attention kernel for one workload."""
    if not args.copy_probe_mib:
        raise SystemExit("--summarize-profiles needs --copy-probe-mib (the calibration size)")
    trace_dir, fetch_dir, write_dir = args.summarize_profiles
    probe_bytes = args.copy_probe_mib * (1 << 20)
    counters = fetch_dir != "-" and write_dir != "-"  # "-": kernel trace only
    cnt = None
    if counters:
        fc, fa, nf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
        wc, wa, nw = _counter_per_dispatch(write_dir, "WRITE_SIZE")
        f_factor = probe_bytes / (fc * 1024.0)
        w_factor = probe_bytes / (wc * 1024.0)
        fetch_b = fa * 1024.0 * f_factor
        write_b = wa * 1024.0 * w_factor
        cnt = (fetch_b, write_b, fa, wa, fc, wc, f_factor, w_factor, nf, nw)
    stats = [r for r in _csv_rows(trace_dir, "kernel_stats.csv") if _short(r["Name"])]
    bench = None
    if args.bench_log:
        with open(args.bench_log) as f:
            bench = json.loads([ln for ln in f if ln.startswith("{")][-1])
    if cnt:
        _write_traffic(args, *cnt)
    per_kernel = None
    if counters:
        fk, fcopy = _per_kernel_counters(fetch_dir, ("FETCH_SIZE",))
        wk, wcopy = _per_kernel_counters(write_dir, ("WRITE_SIZE",))
        per_kernel = {"fetch": fk, "write": wk,
                      "f_factor": probe_bytes / (fcopy["FETCH_SIZE"] * 1024.0),
                      "w_factor": probe_bytes / (wcopy["WRITE_SIZE"] * 1024.0)}
    sq = _per_kernel_counters(args.sq_dir, SQ_COUNTERS)[0] if args.sq_dir else None
    sq2 = _per_kernel_counters(args.sq2_dir, SQ_ISSUE_COUNTERS)[0] if args.sq2_dir else None
    _write_summary(args, stats, bench, cnt, per_kernel, sq, sq2)


def _write_traffic(args, fetch_b, write_b, fa, wa, fc, wc, f_factor, w_factor, nf, nw):
    probe_bytes = args.copy_probe_mib * (1 << 20)
    entry = {"kernel": ATTN_KERNEL, "bytes_per_launch": round(fetch_b + write_b),
             "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
             "fetch_kib_raw": round(fa, 1), "write_kib_raw": round(wa, 1),
             "calibration": {"copy_bytes": probe_bytes, "fetch_kib": round(fc, 1),
                             "write_kib": round(wc, 1), "fetch_factor": round(f_factor, 4),
                             "write_factor": round(w_factor, 4)},
             "dispatches": [nf, nw], "source_digest": attn_source_digest()}
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f)
    except (OSError, ValueError):
        tj = {}
    tj[args.workload] = entry
    with open(args.traffic_json, "w") as f:
        json.dump(tj, f, indent=1, sort_keys=True)
        f.write("\n")


def _write_summary(args, stats, bench, cnt, per_kernel=None, sq=None, sq2=None):
    sw = (f"--steps {bench['steps']} --warmup {bench['warmup']}" if bench else "--steps S --warmup W")
    kernels = sorted({_short(r["Name"]) for r in stats})
    names = sorted({k.split("<")[0].replace("_kernel", "") for k in kernels})
    tag = "_".join(names) if len(names) <= 3 else "lcsa_kernels"
    out = os.path.join(ROOT, "profiles", f"{tag}_{args.workload}.md")
    cmd_b = (f"python3 bench.py --workload {args.workload} {sw} "
             f"--no-cpu-baseline --copy-probe-mib {args.copy_probe_mib}")
    lines = [f"# Kernel trace and HBM traffic: workload {args.workload}", "",
             "Commands (from the repository root, with `TMPDIR=/tmp` exported for the profiler's "
             "scratch files):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d TRACE_DIR -o tr -- {cmd_b}",
             *([f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d FETCH_DIR -o pmc -- {cmd_b}",
                f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d WRITE_DIR -o pmc -- {cmd_b}"]
               if cnt else []),
             *([f"    rocprofv3 --pmc {' '.join(SQ_COUNTERS)} --output-format csv -d SQ_DIR -o pmc "
                f"-- {cmd_b}"] if sq else []),
             *([f"    rocprofv3 --pmc {' '.join(SQ_ISSUE_COUNTERS)} --output-format csv -d SQ2_DIR "
                f"-o pmc -- {cmd_b}"] if sq2 else []),
             f"    python3 bench.py --workload {args.workload} --copy-probe-mib {args.copy_probe_mib} "
             f"--summarize-profiles TRACE_DIR {'FETCH_DIR WRITE_DIR' if cnt else '- -'} "
             f"{'--sq-dir SQ_DIR ' if sq else ''}{'--sq2-dir SQ2_DIR ' if sq2 else ''}"
             f"--bench-log BENCH_LOG", "",
             "## Kernel durations (rocprofv3 --stats)", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    if bench and "bwd_ms" in bench:
        lines += ["", f"bench.py, same workload, HIP events on the launch stream: attention "
                  f"forward + backward {bench['attn_ms'] * 1e3:.1f} us per step (backward "
                  f"{bench['bwd_ms'] * 1e3:.1f} us), step {bench['ms_per_step'] * 1e3:.1f} us, "
                  f"{bench['config']['selected_pairs_per_step']} block pairs per step "
                  f"(steps={bench['steps']}, warmup={bench['warmup']})."]
    elif bench:
        lines += ["", f"bench.py, same workload, HIP events on the launch stream: attention "
                  f"{bench['attn_ms'] * 1e3:.1f} us per launch, step {bench['ms_per_step'] * 1e3:.1f} us, "
                  f"{bench['config']['selected_pairs_per_step']} block pairs per step "
                  f"(steps={bench['steps']}, warmup={bench['warmup']})."]
    if not cnt:
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(json.dumps({"wrote": out}))
        return
    fetch_b, write_b, fa, wa, fc, wc, f_factor, w_factor, nf, nw = cnt
    lines += ["", "## HBM traffic of the attention kernel (rocprofv3 --pmc)", "",
              f"Calibration: the plain {args.copy_probe_mib} MiB device copy ({COPY_KERNEL}) reads "
              f"FETCH_SIZE {fc:.0f} KiB and WRITE_SIZE {wc:.0f} KiB, so one counted KiB is "
              f"{f_factor:.3f} KiB fetched and {w_factor:.3f} KiB written.", "",
              "| counter | raw KiB per launch | calibrated MB per launch | launches |", "|---|---|---|---|",
              f"| FETCH_SIZE | {fa:.0f} | {fetch_b / 1e6:.1f} | {nf} |",
              f"| WRITE_SIZE | {wa:.0f} | {write_b / 1e6:.1f} | {nw} |", ""]
    avg_us = {_short(r["Name"]): float(r["AverageNs"]) / 1e3 for r in stats}
    if per_kernel:
        ff, wf = per_kernel["f_factor"], per_kernel["w_factor"]
        lines += ["## HBM traffic of every kernel (the same --pmc runs, same calibration)", "",
                  "Bytes the counters saw per launch, and that traffic over the kernel's mean "
                  "duration in the trace run, against the 8 TB/s HBM peak.", "",
                  "| kernel | fetched MB | written MB | average us | counted GB/s | fraction of HBM |",
                  "|---|---|---|---|---|---|"]
        for k in sorted(per_kernel["fetch"], key=lambda k: -avg_us.get(k, 0)):
            fb = per_kernel["fetch"][k].get("FETCH_SIZE", 0) * 1024 * ff
            wb = per_kernel["write"].get(k, {}).get("WRITE_SIZE", 0) * 1024 * wf
            us = avg_us.get(k)
            if not us:
                continue
            gbs = (fb + wb) / (us * 1e-6) / 1e9
            lines.append(f"| {k} | {fb / 1e6:.2f} | {wb / 1e6:.2f} | {us:.1f} | {gbs:.0f} | "
                         f"{gbs / PEAK_HBM_GBS:.3f} |")
        lines.append("")
    if sq:
        lines += ["## Instruction mix and matrix-core use (rocprofv3 --pmc, one pass)", "",
                  "Per launch. GRBM_GUI_ACTIVE sums the 8 XCDs' busy cycles, so the clock is "
                  "GRBM_GUI_ACTIVE / 8 over the trace's mean duration; the matrix cores are busy "
                  "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8) of the time. "
                  "SQ_INSTS_VALU counts the MFMA instructions too.", "",
                  "| kernel | " + " | ".join(SQ_COUNTERS) + " | clock GHz | MFMA busy |",
                  "|---|" + "---|" * (len(SQ_COUNTERS) + 2)]
        for k in sorted(sq, key=lambda k: -avg_us.get(k, 0)):
            c = sq[k]
            us = avg_us.get(k)
            cyc = c.get("GRBM_GUI_ACTIVE", 0) / N_XCDS
            ghz = cyc / (us * 1e3) if us else 0.0
            busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (N_SIMDS * cyc) if cyc else 0.0
            lines.append(f"| {k} | " + " | ".join(f"{c.get(n, 0):.0f}" for n in SQ_COUNTERS) +
                         f" | {ghz:.2f} | {busy:.3f} |")
        lines.append("")
    if sq2:
        lines += ["## Where the wave-cycles go (rocprofv3 --pmc, a second pass)", "",
                  "Per launch, as fractions of the waves' resident cycles (SQ_WAVE_CYCLES; the "
                  "SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_INST_* counters count 4-cycle units): "
                  "waiting on memory counters or a barrier (SQ_WAIT_ANY), waiting to issue an "
                  "instruction that is ready (SQ_WAIT_INST_ANY), and issuing any, VALU or LDS "
                  "instructions (SQ_ACTIVE_INST_*). Co-execution is the share of the matrix cores' "
                  "busy cycles in which a normal vector instruction issued as well "
                  "(SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES). The fractions overlap "
                  "(a wave can wait on a counter while another of its instructions issues).", "",
                  "| kernel | " + " | ".join(SQ_ISSUE_COUNTERS) + " | waiting | waiting to issue | "
                  "issuing | VALU | LDS | MFMA busy | co-execution |",
                  "|---|" + "---|" * (len(SQ_ISSUE_COUNTERS) + 7)]
        for k in sorted(sq2, key=lambda k: -avg_us.get(k, 0)):
            c = sq2[k]
            wc = c.get("SQ_WAVE_CYCLES", 0)
            cyc = c.get("GRBM_GUI_ACTIVE", 0) / N_XCDS
            mb = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0)

            def frac(n):
                return f"{c.get(n, 0) / wc:.3f}" if wc else "-"
            busy = mb / (N_SIMDS * cyc) if cyc else 0.0
            coex = c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0) / mb if mb else 0.0
            lines.append(f"| {k} | " + " | ".join(f"{c.get(n, 0):.0f}" for n in SQ_ISSUE_COUNTERS) +
                         f" | {frac('SQ_WAIT_ANY')} | {frac('SQ_WAIT_INST_ANY')} | "
                         f"{frac('SQ_ACTIVE_INST_ANY')} | {frac('SQ_ACTIVE_INST_VALU')} | "
                         f"{frac('SQ_ACTIVE_INST_LDS')} | {busy:.3f} | {coex:.3f} |")
        lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps({"wrote": out}))


if __name__ == "__main__":
    main()
