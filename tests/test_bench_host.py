"""Host-side logic of bench.py that needs no GPU: the digest that ties the committed HBM-traffic
counter summary to the GEMM sources' code."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_layout():
    src = 'int a = 1;  // note\n/* block\n comment */ const char* s = "x // y /* z */";\nchar c = \'"\';\n\tint b;'
    assert bench._code_only(src) == 'int a = 1; const char* s = "x // y /* z */"; char c = \'"\'; int b;'
    # escaped quotes inside a string literal do not end it
    assert bench._code_only('f("a\\"//b"); // c') == 'f("a\\"//b");'


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    names = ("one.cuh", "two.hip")
    for n in names:
        (tmp_path / n).write_text("int f() { return 1; } // first\n")
    monkeypatch.setattr(bench, "GEMM_SOURCES", names)
    monkeypatch.setattr(bench, "__file__", str(tmp_path / "bench.py"))
    d0 = bench.gemm_source_digest()
    (tmp_path / "two.hip").write_text("/* other words */ int f() {\n    return 1;\n}\n")
    assert bench.gemm_source_digest() == d0
    (tmp_path / "two.hip").write_text("int f() { return 2; }\n")
    assert bench.gemm_source_digest() != d0


def test_traffic_summary_is_none_or_positive():
    t = bench.measured_traffic()
    assert t is None or (isinstance(t, int) and t > 0)
