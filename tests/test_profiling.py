"""Host-side checks of the rocprofv3 summary reader used by bench.py."""
import glob
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from split_kv_paged_amd import profiling  # noqa: E402


def test_code_text_drops_comments_and_layout_only():
    a = "int f(int x) {  // one\n  return x + 1; /* two\n lines */ }\n"
    b = "int f(int x) { return x + 1; }"
    assert profiling.code_text(a) == profiling.code_text(b) == "int f(int x) { return x + 1; }"
    # code changes still show, and string literals keep their text
    assert profiling.code_text("return x + 2;") != profiling.code_text("return x + 1;")
    s = 'const char* u = "a // b /* c */";'
    assert profiling.code_text(s) == s


def test_source_digest_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// header\n__global__ void k() {}\n")
    monkeypatch.setattr(profiling, "CSRC", str(tmp_path))
    d0 = profiling.source_digest()
    src.write_text("// another header\n\n__global__   void k() {}  /* note */\n")
    assert profiling.source_digest() == d0
    src.write_text("__global__ void k() { int x = 0; }\n")
    assert profiling.source_digest() != d0


def test_source_digest_is_stable_and_short():
    a = profiling.source_digest()
    assert a == profiling.source_digest() and len(a) == 16


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "hbm_traffic_*.md"))))
def test_committed_traffic_summaries_parse(path):
    v = profiling.read_traffic(path)
    for key in ("workload", "num_splits", "source_digest", "fetch_bytes_per_launch",
                "write_bytes_per_launch", "traffic_bytes_per_launch"):
        assert key in v, key
    assert os.path.basename(path) == "hbm_traffic_%s.md" % v["workload"]
    total = float(v["fetch_bytes_per_launch"]) + float(v["write_bytes_per_launch"])
    assert abs(total - float(v["traffic_bytes_per_launch"])) <= 1.0


def test_bench_drops_traffic_when_sources_changed(tmp_path, monkeypatch):
    import bench
    name = "example_workload"
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / ("hbm_traffic_%s.md" % name)).write_text(
        "# t\n\n```\nworkload: %s\nnum_splits: 1\nsource_digest: %s\n"
        "fetch_bytes_per_launch: 10\nwrite_bytes_per_launch: 2\n"
        "traffic_bytes_per_launch: 12\n```\n" % (name, profiling.source_digest()))
    monkeypatch.setattr(bench, "__file__", str(tmp_path / "bench.py"))
    assert bench.measured_traffic(name, 1) == 12
    assert bench.measured_traffic(name, 2) is None  # other split count
    monkeypatch.setattr(profiling, "source_digest", lambda: "0" * 16)
    assert bench.measured_traffic(name, 1) is None  # kernel changed since the counters
