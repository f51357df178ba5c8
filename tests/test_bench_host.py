"""Host-side logic of bench.py (no GPU): when the counter-derived HBM
traffic of the attention kernel may be reported."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_source_digest_is_stable_and_covers_the_kernel_files():
    d = bench.attn_source_digest()
    assert d == bench.attn_source_digest() and len(d) == 16
    for rel in bench.ATTN_SOURCES:
        assert os.path.isfile(os.path.join(ROOT, rel)), rel


def test_traffic_only_for_counters_taken_on_the_current_sources(tmp_path):
    p = tmp_path / "traffic.json"
    cur = bench.attn_source_digest()
    p.write_text(json.dumps({
        "now": {"bytes_per_launch": 123, "source_digest": cur},
        "old": {"bytes_per_launch": 456, "source_digest": "0" * 16},
        "legacy": {"bytes_per_launch": 789},
    }))
    assert bench.traffic_for(str(p), "now") == 123
    assert bench.traffic_for(str(p), "old") is None      # kernel changed since
    assert bench.traffic_for(str(p), "legacy") is None   # no record of the sources
    assert bench.traffic_for(str(p), "absent") is None
    assert bench.traffic_for(str(tmp_path / "missing.json"), "now") is None
    (tmp_path / "bad.json").write_text("{")
    assert bench.traffic_for(str(tmp_path / "bad.json"), "now") is None


def _run_oracle_stream(w, qkv, t_first, last):
    """What the GPU would leave in its buffers after step `last`, computed
    here by the oracle itself: the plumbing of the in-run parity check is
    what is under test, not the kernels."""
    import numpy as np
    import torch

    from oracle import lcsa_oracle as O
    F = w.frames
    p = O.SelectParams(local_range=w.local_range, ratio_num=w.ratio[0], ratio_den=w.ratio[1])
    cache = O.KVCache(cap_tb=w.cap_tb)
    host = lambda t: t.float().numpy().astype(np.float64)
    O.prime_cache(cache, host(qkv["k"][:, :t_first]), host(qkv["v"][:, :t_first]), 0)
    for n in range(last + 1):
        f0 = t_first + n * F
        res = O.lcsa_step(host(qkv["q"][:, n * F:(n + 1) * F]), host(qkv["k"][:, f0:f0 + F]),
                          host(qkv["v"][:, f0:f0 + F]), cache, f0 // 2, p)
    kmax = int(res.kcount.max())
    sel = np.full((w.batch, w.heads, w.nq, kmax), -1, dtype=np.int32)
    cnt = np.zeros((w.batch, w.heads, w.nq), dtype=np.int32)
    for h in range(w.heads):
        for i, r in enumerate(res.sel[0][h]):
            sel[0, h, i, :len(r)] = r
            cnt[0, h, i] = len(r)

    class Bufs:
        pass
    b = Bufs()
    b.sel_idx, b.sel_cnt = torch.from_numpy(sel), torch.from_numpy(cnt)
    b.out = torch.from_numpy(res.out).float()
    return b


def test_in_run_parity_check_plumbing():
    """cpu_baseline_run replays the run's last steps on the host from the
    same device-resident frames and checks the last step's selections and
    outputs: identical buffers pass with zero error, and a corrupted
    selection or output is reported."""
    import torch

    from block_sparse_attention_03_amd import synth
    from block_sparse_attention_03_amd.workloads import Workload
    w = Workload("small stream", 2, 32, "f32", 16, 24, 2, 6, 3, local_range=3, ratio=(1, 4))
    t_first, n_steps = w.cache_frames, 3
    qkv = {}
    for name, tid in synth.TENSOR_IDS.items():
        t0 = t_first if name == "q" else 0
        qkv[name] = synth.field_frames_device(w.seed, tid, w.heads, w.head_dim, w.height,
                                              w.width, t0, t_first + w.frames * n_steps,
                                              torch.device("cpu"), torch.float32)
    last = n_steps - 1
    bufs = _run_oracle_stream(w, qkv, t_first, last)
    fp = 4 * 128 * 128 * w.head_dim
    r = bench.cpu_baseline_run(w, qkv, t_first, last, 2, bufs, fp)
    par = r["parity"]
    assert par["pass"] and par["selection_mismatches"] == 0 and par["max_abs"] < 1e-6  # f32 rounding
    assert par["rows"] == w.heads * w.nq and r["kind"] == "oracle" and r["value"] > 0
    # a row whose list names another block fails the check
    i = int(torch.nonzero(bufs.sel_cnt[0, 1] > 0)[0])
    k = int(bufs.sel_cnt[0, 1, i])
    ids = bufs.sel_idx[0, 1, i, :k].tolist()
    cand = [j for j in range(4 * w.nS) if j not in ids]
    ids = sorted(ids[1:] + cand[:1])
    bufs.sel_idx[0, 1, i, :k] = torch.tensor(ids, dtype=torch.int32)
    par = bench.cpu_baseline_run(w, qkv, t_first, last, 1, bufs, fp)["parity"]
    assert par["selection_mismatches"] >= 1 and not par["pass"]
    # an output off by more than the tolerance fails it too
    bufs = _run_oracle_stream(w, qkv, t_first, last)
    bufs.out[0, 0, 0, 0, 0, 0] += 1.0
    par = bench.cpu_baseline_run(w, qkv, t_first, last, 1, bufs, fp)["parity"]
    assert par["selection_mismatches"] == 0 and par["max_abs"] >= 0.99 and not par["pass"]
