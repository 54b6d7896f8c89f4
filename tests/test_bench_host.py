"""Host logic of bench.py (no GPU): which kernel source a workload's timed
step is attributed to, the code-only source digest that keys the recorded
HBM traffic, the traffic-record lookup and the bundle-copy rotation."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_kernel_source_follows_the_dispatch():
    # the decode kernel of the bundle's kind up to batch 7, the matrix-core
    # kernel from batch 8
    for kind in ("q4", "q6"):
        assert [bench.kernel_source(kind, b) for b in (1, 4, 7, 8, 16)] == \
            ["fused_q.hip"] * 3 + ["mfma.hip"] * 2
    assert [bench.kernel_source("bf16", b) for b in (1, 4, 7, 8, 16)] == \
        ["bf16.hip"] * 3 + ["mfma.hip"] * 2


def test_code_text_ignores_comments_and_layout():
    a = "int f(int x) { // one\n  return x + 1; /* two\n three */ }\n"
    b = "int f(int x)\n{\n    return x + 1;   // other words\n}"
    assert bench._code_text(a) == bench._code_text(b)
    assert bench._code_text(a) != bench._code_text(a.replace("x + 1", "x + 2"))


def test_sources_digest_differs_per_kernel_file():
    d = {k: bench.sources_digest(k) for k in ("fused_q.hip", "mfma.hip", "bf16.hip")}
    assert len(set(d.values())) == 3 and all(len(v) == 16 for v in d.values())
    assert bench.sources_digest("fused_q.hip") == d["fused_q.hip"]


def test_recorded_traffic_matches_workload_batch_and_digest(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("# workload batch bytes digest\n"
                 "wl_a 1 1000 abcd\n"
                 "wl_a 4 2000 abcd\n"
                 "wl_b 1 3000 ef01\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("wl_a", 4, "abcd") == 2000
    assert bench.recorded_traffic("wl_b", 1, "ef01") == 3000
    assert bench.recorded_traffic("wl_a", 1, "ffff") is None   # kernel changed since the counters
    assert bench.recorded_traffic("wl_c", 1, "abcd") is None


def test_copies_cover_twice_the_mall():
    # enough copies that one pass over them exceeds twice the MALL, within [2, 96]
    for coded in (23_801_316, 79_562_360, 137_687_908):
        n = bench.copies_for(coded)
        assert n * coded >= 2 * bench.MALL_BYTES > (n - 1) * coded or n == 2
    assert bench.copies_for(120_740) == 96          # a small matrix: capped
    assert bench.copies_for(1 << 30) == 2           # a huge one: at least two
