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
