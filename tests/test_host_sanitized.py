"""The host half of the C-ABI (block_sparse_attention_03_amd/csrc/lcsa_host.cpp,
which uses no HIP API) built with the address and undefined-behaviour
sanitizers into a CPU-only driver (tests/host/host_driver.cpp) that runs
every validation error, ring wrap-around, over- and underflow of the ring,
and the k rule on the hand table of tests/golden/k_table.json ("How FlashVSR
works", section 2.2 step 3: the topk_ratio rule)."""
from __future__ import annotations

import json
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HOST_SRC = os.path.join(ROOT, "block_sparse_attention_03_amd", "csrc", "lcsa_host.cpp")
DRIVER = os.path.join(HERE, "host", "host_driver.cpp")


def k_table_lines():
    g = json.load(open(os.path.join(HERE, "golden", "k_table.json")))
    lines = []
    for case in g["k_rows"]:
        out = case.get("out", (768, 1280))
        num, den = case.get("ratio", (1, 5))
        for n, k in zip(case["n_allowed"], case["k"]):
            lines.append(f"k {num} {den} {int(case.get('scale', False))} {out[0]} {out[1]} "
                         f"{case.get('topk_fixed', 0)} {n} {k}")
    return "\n".join(lines) + "\n"


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_host_logic_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           DRIVER, HOST_SRC, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], input=k_table_lines(), capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
