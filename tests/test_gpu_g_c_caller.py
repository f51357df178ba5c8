"""One streaming step driven from plain C (tests/host/c_step.c, built by
__graft_entry__.build()): HIP's C API for device memory, the C-ABI for the
ring, partition + pool, draft and attention. The same step through the
Python binding on the same inputs must give bitwise-equal lists, outputs and
log-sum-exp, and the selections must equal the oracle's ("How FlashVSR
works", section 2.2 steps 1-3; the "FlashVSR" note, Key design 2)."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

from block_sparse_attention_03_amd import lcsa as L
from block_sparse_attention_03_amd import synth
from oracle import lcsa_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_harness import say, to_dev  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "host", "c_step")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load_library()
    return torch.device("cuda:0")


def read_c_step(path):
    raw = open(path, "rb").read()
    T, H, W, NH, D, kmax = np.frombuffer(raw, dtype=np.int32, count=6)
    nq = (H // 8) * (W // 8)
    pos = 24
    def take(dtype, shape):
        nonlocal pos
        n = int(np.prod(shape))
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=pos).reshape(shape).copy()
        pos += n * np.dtype(dtype).itemsize
        return a
    qkv = [take(np.uint16, (1, T, H, W, NH, D)) for _ in range(3)]
    cnt = take(np.int32, (1, NH, nq))
    idx = take(np.int32, (1, NH, nq, kmax))
    out = take(np.uint16, (1, 2, H, W, NH, D))
    lse = take(np.float32, (1, NH, nq, 128))
    assert pos == len(raw)
    return (int(T), int(H), int(W), int(NH), int(D), int(kmax)), qkv, cnt, idx, out, lse


def test_step_from_c_equals_the_binding_and_the_oracle(dev, tmp_path):
    if not os.path.exists(EXE):
        pytest.skip("tests/host/c_step is not built (__graft_entry__.build() compiles it)")
    say("c step: 2 heads, d64, 6 x 32 x 48 tokens (4 cached), window 5, k = 1/3")
    path = str(tmp_path / "c_step.bin")
    r = subprocess.run([EXE, path], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    (T, H, W, NH, D, kmax), qkv, cnt, idx, out, lse = read_c_step(path)

    # the same step through the binding, on the same bf16 inputs
    q, k, v = (to_dev(np.ascontiguousarray(x), "bf16", dev) for x in qkv)
    cache = L.KVCache(1, NH, D, H, W, torch.bfloat16, n_slots=4, device=dev)
    gc = L.make_geom(1, NH, D, 4, H, W, L.LCSA_BF16)
    L.lcsa_partition_pool(gc, None, k[:, :4].contiguous(), v[:, :4].contiguous(), None, None,
                          cache.c, cache.append(2, 0))
    g = L.make_geom(1, NH, D, 2, H, W, L.LCSA_BF16)
    params = L.make_params(local_range=5, ratio=(1, 3))
    bufs = L.run_step(g, q[:, 4:].contiguous(), k[:, 4:].contiguous(), v[:, 4:].contiguous(), cache,
                      2, params, want_lse=True)
    torch.cuda.synchronize()
    assert bufs.kmax == kmax
    assert np.array_equal(bufs.sel_cnt.cpu().numpy(), cnt)
    assert np.array_equal(bufs.sel_idx.cpu().numpy(), idx)
    assert np.array_equal(bufs.out.view(torch.int16).cpu().numpy().view(np.uint16), out)
    assert np.array_equal(bufs.lse.cpu().numpy().view(np.uint32), lse.view(np.uint32))

    # the selections against the oracle
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in qkv)
    ocache = O.KVCache(cap_tb=3)
    O.prime_cache(ocache, k64[:, :4], v64[:, :4], 0)
    ref = O.lcsa_step(q64[:, 4:], k64[:, 4:], v64[:, 4:], ocache, 2,
                      O.SelectParams(local_range=5, ratio_num=1, ratio_den=3), rows=[])
    for h in range(NH):
        for i, row in enumerate(ref.sel[0][h]):
            assert cnt[0, h, i] == len(row), (h, i)
            assert list(idx[0, h, i, :len(row)]) == list(row), (h, i)
    say(f"c step: lists, outputs and lse bitwise equal to the binding's; kmax {kmax}")
