"""Comparison rules between the GPU path and the float64 oracle.

Selection: exact, except rows whose k-th and (k+1)-th oracle scores differ by
at most 1e-5 relative (plus a 1e-7 absolute floor); such rows are "tied" and
the GPU set G passes if |G| = k and
{j : s_j > s_(k) + tol} <= G <= {j : s_j >= s_(k+1) - tol}.
Outputs: max-abs and relative L2 against the oracle, bf16 bound
max-abs <= 2e-2 and rel-L2 <= 5e-3; fp32 bound max-abs <= 1e-4, rel-L2 <= 1e-5.
"""
from __future__ import annotations

import numpy as np

TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-4, 1e-5)}


def check_row_selection(scores_row: np.ndarray, k: int, gpu_ids, oracle_ids):
    """Returns 'exact' or 'tied'; raises AssertionError on a mismatch."""
    gpu = sorted(int(x) for x in gpu_ids)
    assert len(gpu) == k, f"|G| = {len(gpu)} != k = {k}"
    assert len(set(gpu)) == len(gpu), "duplicate ids"
    fin = np.isfinite(scores_row)
    n = int(fin.sum())
    assert all(fin[j] for j in gpu), "selected a non-candidate"
    if k == 0 or k >= n:
        assert gpu == sorted(np.nonzero(fin)[0].tolist())
        return "exact"
    vals = np.sort(scores_row[fin])[::-1]
    sk, sk1 = vals[k - 1], vals[k]
    tol = 1e-5 * max(abs(sk), abs(sk1)) + 1e-7
    if abs(sk - sk1) > tol:
        assert gpu == sorted(int(x) for x in oracle_ids), "selection differs (untied row)"
        return "exact"
    must = set(np.nonzero(fin & (scores_row > sk + tol))[0].tolist())
    may = set(np.nonzero(fin & (scores_row >= sk1 - tol))[0].tolist())
    g = set(gpu)
    assert must <= g <= may, "tied row: selection outside the tied candidates"
    return "tied"


def errors(gpu: np.ndarray, ref: np.ndarray):
    d = gpu.astype(np.float64) - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def assert_close(gpu, ref, dtype: str, what: str = "output"):
    amax, rel = errors(gpu, ref)
    ta, tr = TOL[dtype]
    assert amax <= ta and rel <= tr, f"{what}: max-abs {amax:.3e} (<= {ta}), rel-L2 {rel:.3e} (<= {tr})"
    return amax, rel
