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


def _csv(path, header, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w") as fh:
        fh.write(",".join(header) + "\n")
        for r in rows:
            fh.write(",".join(str(v) for v in r) + "\n")


def test_profile_summaries_from_synthetic_runs(tmp_path):
    """bench_profiles.py on three tiny synthetic rocprofv3 outputs: the 1 GiB
    calibration copy sets the counter scales, a traced launch gives its
    average duration and GB/s, and kernels absent from the runs get NaN rows
    and null traffic instead of an error."""
    import json
    import bench_profiles
    grid = 16 * (3072 // 16) * (4096 // 512) * 256  # one 16-expert gate_up launch, threads
    name = '"mxq::k_grouped<0, 0, false>(mxq::GroupArgs)"'
    copy = '"__amd_rocclr_copyBuffer"'
    hdr = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Value"]
    alg = 16 * (3072 * 4096 * 3 + 3072 * 128)  # MXFP8 linear gate_up bytes
    _csv(tmp_path / "prof_fetch" / "f_counter_collection.csv", hdr,
         [(1, copy, 1 << 20, 524288.0), (2, name, grid, 3072 * 4096 * 16 * 2 / 2 / 1024)])
    _csv(tmp_path / "prof_write" / "w_counter_collection.csv", hdr,
         [(1, copy, 1 << 20, 1048576.0), (2, name, grid, (alg - 3072 * 4096 * 32) / 1024)])
    _csv(tmp_path / "prof_kt" / "kt_kernel_trace.csv",
         ["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
          "Start_Timestamp", "End_Timestamp"],
         [(2, name, grid, 1, 1, 1_000_000, 1_096_000)])
    out = tmp_path / "out"
    out.mkdir()
    bench_profiles.main([str(tmp_path), "--out", str(out)])
    d = json.loads((out / "hbm_traffic.json").read_text())
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    k = d["kernels"]["k_grouped<MXFP8,LINEAR>"]
    assert k["traffic_bytes_per_launch"] is None  # the down launch is not in the runs
    assert d["kernels"]["k_split<nvfp4,SWIZZLED>"]["traffic_bytes_per_launch"] is None
    md = (out / "k_grouped_qwen3_235b_layer.md").read_text()
    row = [l for l in md.splitlines() if l.startswith("| k_grouped<MXFP8,LINEAR> | gate_up | 1 |")]
    assert row and "| 96.00 |" in row[0] and f"| {alg / 96000:,.0f} |" in row[0]
    assert [l for l in md.splitlines()
            if l.startswith("| k_grouped<MXFP8,LINEAR> | gate_up | 1 | 610,271,232 |")
            and l.endswith("| 1.0000 |")]
