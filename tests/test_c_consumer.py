"""The C-ABI from plain C: tests/host/c_consumer.c includes include/lcsa.h,
is compiled as strict C11 (-pedantic -Werror) and linked against the built
liblcsa.so. It runs the host-side calls (ring metadata, the k rule on the
hand table of tests/golden/k_table.json, workspace sizes, validation errors)
with aligned device pointers that are never dereferenced."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from block_sparse_attention_03_amd import lcsa as L
from test_host_sanitized import k_table_lines

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_library_is_callable_from_c(tmp_path):
    lib_dir = os.path.dirname(L.LIB_PATH)
    assert os.path.exists(L.LIB_PATH), "liblcsa.so is not built"
    exe = str(tmp_path / "c_consumer")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "host", "c_consumer.c"),
                    "-L", lib_dir, "-llcsa", f"-Wl,-rpath,{lib_dir}", "-o", exe],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], input=k_table_lines(), capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("c consumer ok")
    assert "k table rows 13" in r.stdout
