"""Checkpoint and resume of a stream's KV ring through lcsa_kv_cache_copy.

[HW] "How FlashVSR works" 2.3: the cache of past segments is the only state a
streaming layer carries from one step to the next. A stream run straight
through, and the same stream saved after three steps into a spare ring,
disturbed by two chunks of other inputs, restored and resumed, give
bitwise-equal lists, outputs and lse on the resumed steps. The ring has one
slot more than the cache keeps, so it wraps during the run.
"""
from __future__ import annotations

import dataclasses

import pytest

from block_sparse_attention_03_amd import lcsa as L
from block_sparse_attention_03_amd import synth
from block_sparse_attention_03_amd.workloads import WORKLOADS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_harness import lib_params, say  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load_library()
    return torch.device("cuda:0")


def frames(w, seed, t0, t1, dev):
    return {n: synth.field_frames_device(seed, tid, w.heads, w.head_dim, w.height, w.width, t0, t1,
                                         dev, torch.bfloat16, batch=w.batch)
            for n, tid in synth.TENSOR_IDS.items()}


@pytest.mark.parametrize("name", ["step_768x1408", "step_1536x2688"])
def test_checkpoint_resume_bitwise(dev, name):
    w = dataclasses.replace(WORKLOADS[name], heads=2)
    n_steps, save_after = 6, 3
    t_first = w.cache_frames
    x = frames(w, w.seed, 0, t_first + w.frames * n_steps, dev)
    other = frames(w, w.seed + 77, t_first, t_first + w.frames * 2, dev)
    geom = L.make_geom(w.batch, w.heads, w.head_dim, w.frames, w.height, w.width, L.LCSA_BF16)
    gp = L.make_geom(w.batch, w.heads, w.head_dim, t_first, w.height, w.width, L.LCSA_BF16)
    params = lib_params(w)

    def new_cache():
        c = L.KVCache(w.batch, w.heads, w.head_dim, w.height, w.width, torch.bfloat16,
                      n_slots=w.n_slots, device=dev)
        first = c.append(t_first // 2, 0)
        L.lcsa_partition_pool(gp, None, x["k"][:, :t_first], x["v"][:, :t_first], None, None,
                              c.c, first)
        return c

    def step(cache, src, n, tb):
        # x holds the stream from frame 0, other holds its two chunks from 0
        f0 = n * w.frames if src is other else t_first + n * w.frames
        sl = slice(f0, f0 + w.frames)
        b = L.run_step(geom, src["q"][:, sl], src["k"][:, sl], src["v"][:, sl], cache, tb, params,
                       keep_tb=w.cap_tb, want_lse=True)
        return {k: getattr(b, k).clone() for k in ("sel_idx", "sel_cnt", "out", "lse")}

    tb0 = t_first // 2
    step_tb = w.frames // 2
    straight = new_cache()
    ref = [step(straight, x, n, tb0 + n * step_tb) for n in range(n_steps)]

    live = new_cache()
    for n in range(save_after):
        step(live, x, n, tb0 + n * step_tb)
    spare = L.KVCache(w.batch, w.heads, w.head_dim, w.height, w.width, torch.bfloat16,
                      n_slots=w.n_slots, device=dev)
    spare.copy_from(live)                      # save
    for n in range(2):                         # disturb the live ring
        step(live, other, n, tb0 + (save_after + n) * step_tb)
    assert live.view() != spare.view()
    live.copy_from(spare)                      # restore
    assert live.view() == spare.view()
    for n in range(save_after, n_steps):
        got = step(live, x, n, tb0 + n * step_tb)
        for k in ref[n]:
            assert torch.equal(got[k], ref[n][k]), (name, n, k)
    torch.cuda.synchronize()
    say(f"{name}: resumed steps {save_after}..{n_steps - 1} bitwise equal to the straight run, "
        f"ring view {live.view()}")
