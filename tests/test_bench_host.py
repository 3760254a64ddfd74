"""Host-side logic of bench.py (no GPU): the source fingerprint that decides
whether the committed HBM-traffic counters still describe the kernels."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_code_text_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles\n    return 2 * x; /* plain */\n}\n"
    b = "/* header */\nint f(int x) {\n  return 2 * x;\n}  // end\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text("x = 1; // y") != bench.code_text("x = 2;")


def test_code_text_keeps_literals():
    t = 'const char *s = "a // b /* c */"; char q = \'"\';'
    assert bench.code_text(t) == t


def test_source_hash_follows_code_only(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    f = tmp_path / "k.hip"
    f.write_text("__global__ void k(int *p) { p[0] = 1; }\n")
    h0 = bench.source_hash(["k.hip"])
    f.write_text("// a kernel\n__global__ void k(int *p) {\n    p[0] = 1;  // store\n}\n")
    assert bench.source_hash(["k.hip"]) == h0
    f.write_text("__global__ void k(int *p) { p[0] = 2; }\n")
    assert bench.source_hash(["k.hip"]) != h0
