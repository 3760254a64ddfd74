#!/usr/bin/env python3
"""Summarize three rocprofv3 runs of bench.py into profiles/*.md and
profiles/hbm_traffic.json (the per-launch HBM traffic that bench.py reports).

    python bench_profiles.py DIR [--out OUT]

DIR holds the runs' output folders: prof_kt (kernel trace), prof_fetch
(FETCH_SIZE) and prof_write (WRITE_SIZE), made by the commands that each
summary lists, and optionally pmc_valu and pmc_ms (VALUBusy, MemUnitStalled
of the layer alone).  The counter runs add a 1 GiB device copy (bench.py
--calib-copy); what the counters read for it calibrates them to bytes.
Kernels are told apart by name, template arguments and grid size; where one
grid serves several workloads, by dispatch order.  A kernel the runs do not
contain gets a row of n = 0 and NaN figures.  OUT defaults to profiles/.
"""
import argparse
import collections
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
SOURCES = {
    "grouped": ["mxq_grouped.hip", "mxq_device.h", "mxq_internal.h"],
    "split": ["mxq_split.hip", "mxq_device.h", "mxq_internal.h"],
    "fused": ["mxq_fused.hip", "mxq_device.h", "mxq_internal.h"],
}
FMT = {"0": "MXFP8", "1": "NVFP4"}
LAY = {"0": "LINEAR", "1": "SWIZZLED"}
GIB = 1 << 30

CMD_KT = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
          "-d $OUT/prof_kt -o kt -- python3 $REPO/bench.py --steps 5 --warmup 1 --no-cpu-baseline")
CMD_F = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv "
         "-d $OUT/prof_fetch -o f -- python3 $REPO/bench.py --steps 2 --warmup 1 "
         "--no-cpu-baseline --calib-copy --c2-layers 2")
CMD_W = CMD_F.replace("FETCH_SIZE", "WRITE_SIZE").replace("prof_fetch", "prof_write").replace(
    "-o f ", "-o w ")
HDR = ("Commands (`$REPO` is the repository root, `$OUT` an output folder; each counter in a run "
       "of its own), summarized by `python bench_profiles.py $OUT`:\n\n```\n"
       + CMD_KT + "\n" + CMD_F + "\n" + CMD_W + "\n```\n\n")
# The benchmark's layer comes first in every run, before its secondary
# workloads (some of which launch the same kernels on the same grids): a
# layer step makes 128 / 16 launches of each kind, and each run makes
# --warmup + --steps layer steps.
LAYER_LAUNCHES = 128 // 16
KT_STEPS, PMC_STEPS = 1 + 5, 1 + 2
# Qwen3-30B-A3B layers the kernel-trace run streams (bench.py --c2-layers default)
C2_LAYERS = 48


def sf_bytes(rows, C, layout):
    return rows * C if layout == 0 else -(-rows // 128) * 128 * (-(-C // 4) * 4)


def avg(v):
    return sum(v) / len(v) if v else float("nan")


def read_counters(path):
    """[(dispatch, kernel, grid threads, bytes)] and the calibration copy's bytes."""
    rows, calib = [], None
    with open(path) as fh:
        for r in csv.DictReader(fh):
            n = r["Kernel_Name"]
            v = float(r["Counter_Value"]) * 1024  # KiB -> bytes
            if n.startswith("__amd_rocclr_copyBuffer") and calib is None and v > 1e8:
                calib = v  # the first large copy: the 1 GiB calibration copy
            rows.append((int(r["Dispatch_Id"]), n, int(r["Grid_Size"]), v))
    if calib is None:
        raise SystemExit(f"{path}: no calibration copy (run bench.py with --calib-copy)")
    return rows, calib


def read_trace(path):
    """[(dispatch, kernel, grid threads, duration ns, start ns, end ns)] in dispatch order."""
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], g, e - s, s, e))
    return sorted(rows)


def rnd(x, nd=None):
    """round(), or None for a kernel the runs did not contain (NaN)."""
    if x != x:
        return None
    return round(x) if nd is None else round(x, nd)


def lo(v):
    return min(v) if v else float("nan")


def hi(v):
    return max(v) if v else float("nan")


def pct(v, q):
    """The q-quantile of v (nearest rank), NaN when empty."""
    if not v:
        return float("nan")
    w = sorted(v)
    return w[min(len(w) - 1, int(q * len(w)))]


CMD_VALU = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc VALUBusy --output-format csv "
            "-d $OUT/pmc_valu -o v -- python3 $REPO/bench.py --steps 2 --warmup 1 --no-extra "
            "--no-cpu-baseline")
CMD_MS = CMD_VALU.replace("VALUBusy", "MemUnitStalled").replace("pmc_valu", "pmc_ms").replace(
    "-o v ", "-o m ")


def write_valu_summary(valu_csv, ms_csv, out_dir):
    """rocprofv3's derived VALUBusy and MemUnitStalled per grouped kernel and launch."""
    names = {"0, 0": "k_grouped<MXFP8,LINEAR>", "0, 1": "k_grouped<MXFP8,SWIZZLED>",
             "1, 0": "k_grouped<NVFP4,LINEAR>", "1, 1": "k_grouped<NVFP4,SWIZZLED>"}
    proj = {16 * (r // 16) * (c // 512) * 256: p for p, (r, c) in
            {"gate_up": (3072, 4096), "down": (4096, 1536)}.items()}
    vals = {}
    for path, metric in ((valu_csv, "VALUBusy"), (ms_csv, "MemUnitStalled")):
        acc = collections.defaultdict(list)
        with open(path) as fh:
            for r in csv.DictReader(fh):
                n, g = r["Kernel_Name"], int(r["Grid_Size"])
                if "k_grouped<" not in n or ", false>" not in n or g not in proj:
                    continue
                t = n.split("k_grouped<")[1].split(", false>")[0]
                acc[(names[t], proj[g])].append(float(r["Counter_Value"]))
        for k, v in acc.items():
            vals.setdefault(k, {})[metric] = (len(v), avg(v))
    lines = [f"| {k[0]} | {k[1]} | {v['VALUBusy'][0]} | {v['VALUBusy'][1]:.1f} | "
             f"{v['MemUnitStalled'][1]:.1f} |" for k, v in sorted(vals.items())]
    with open(os.path.join(out_dir, "k_grouped_valu_qwen3_235b_layer.md"), "w") as fh:
        fh.write(
            "# k_grouped -- vector ALU busy and memory-unit stall, Qwen3-235B-A22B-shaped layer, "
            "MI355X\n\n"
            "Commands (`$REPO` is the repository root, `$OUT` an output folder; each metric in a "
            "run of its own):\n\n```\n" + CMD_VALU + "\n" + CMD_MS + "\n```\n\n"
            "rocprofv3's derived metrics, per dispatch, averaged over the layer's launches\n"
            "(3 steps of 8 launches per kind): VALUBusy = 100 * SQ_ACTIVE_INST_VALU / CU_NUM /\n"
            "GRBM_GUI_ACTIVE (the share of GPU time the vector ALUs are issuing);\n"
            "MemUnitStalled = 100 * TCP_TCP_TA_DATA_STALL_CYCLES / GRBM_GUI_ACTIVE / SE_NUM.\n\n"
            "| kernel | launch | n | VALUBusy % | MemUnitStalled % |\n|---|---|---|---|---|\n"
            + "\n".join(lines) + "\n\n"
            "Neither the vector ALUs nor the memory unit's data path is saturated: the\n"
            "kernels wait on HBM.  NVFP4 issues about twice the vector work of MXFP8 (the\n"
            "fp32 multiply per element and the per-block scale arithmetic) and still runs\n"
            "within 3 % of MXFP8's bandwidth.\n")


def write_stats_summary(stats_csv, out_dir):
    """rocprofv3's own --stats summary of the kernel-trace run (all dispatches
    of a kernel name together, every workload of the run included)."""
    with open(stats_csv) as fh:
        rows = list(csv.DictReader(fh))
    lines = [f"| `{r['Name'][:90]}` | {int(r['Calls']):,} | {float(r['AverageNs']) / 1e3:,.2f} | "
             f"{float(r['MinNs']) / 1e3:,.2f} | {float(r['MaxNs']) / 1e3:,.2f} | {r['Percentage']} |"
             for r in rows]
    with open(os.path.join(out_dir, "rocprofv3_kernel_stats_bench.md"), "w") as fh:
        fh.write("# rocprofv3 --kernel-trace --stats summary of bench.py (kt_kernel_stats.csv), "
                 "MI355X\n\nCommand (`$REPO` is the repository root, `$OUT` an output folder):\n\n"
                 "```\n" + CMD_KT + "\n```\n\n"
                 "One row per kernel name over every dispatch of the run (the layer steps and the "
                 "secondary workloads together), as rocprofv3 wrote it; the per-launch-shape "
                 "figures are in the k_*.md summaries.\n\n"
                 "| kernel | calls | avg us | min us | max us | % of kernel time |\n"
                 "|---|---|---|---|---|---|\n" + "\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("dir", help="folder holding prof_kt, prof_fetch and prof_write")
    ap.add_argument("--out", default=PROFILES, help="where the summaries go")
    args = ap.parse_args(argv)
    d, out_dir = args.dir, args.out
    sys.path.insert(0, ROOT)
    import bench
    from nvfp4_quantization_moe_amd import workloads

    fetch, cf = read_counters(os.path.join(d, "prof_fetch", "f_counter_collection.csv"))
    write, cw = read_counters(os.path.join(d, "prof_write", "w_counter_collection.csv"))
    trace = read_trace(os.path.join(d, "prof_kt", "kt_kernel_trace.csv"))
    f_scale, w_scale = GIB / cf, GIB / cw
    calib = (f"Calibration: the 1 GiB device copy `--calib-copy` adds (`__amd_rocclr_copyBuffer`) "
             f"reads {cf / 1024:,.1f} KiB of FETCH_SIZE and writes {cw / 1024:,.1f} KiB of "
             f"WRITE_SIZE, so FETCH_SIZE is scaled by {f_scale:.4f} and WRITE_SIZE by "
             f"{w_scale:.4f} to give bytes.\n")

    def select(rows, match):
        return [x for x in rows if match(x[1], x[2])]

    def pmc(match, alg, pick=None):
        fv, wv = select(fetch, match), select(write, match)
        if pick:
            fv, wv = pick(fv), pick(wv)
        fb = avg([x[3] for x in fv]) * f_scale
        wb = avg([x[3] for x in wv]) * w_scale
        return len(fv), fb, wb, (fb + wb) / alg

    def src(kind):
        return {"sources": SOURCES[kind], "source_sha256": bench.source_hash(SOURCES[kind])}

    out = {"fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}

    def write_md(name, title, body):
        with open(os.path.join(out_dir, name), "w") as fh:
            fh.write(f"# {title}\n\n" + HDR + body)

    # ------------------------------------------------------------ grouped
    shapes = workloads.QWEN3_235B_A22B
    lines_t, lines_c = [], []
    for f in "01":
        for l in "01":
            name = f"k_grouped<{FMT[f]},{LAY[l]}>"
            per_alg, per_traf = [], []
            for p, (r, c) in shapes.items():
                fmt = int(f)
                pw = c if fmt == 0 else c // 2
                C = c // (32 if fmt == 0 else 16)
                alg = 16 * (r * c * 2 + r * pw + sf_bytes(r, C, int(l)) + (4 if fmt else 0))
                units = 16 * (-(-r // 128) * 128 // 16 if l == "1" else -(-r // 16)) * (-(-c // 512))
                m = (lambda n, g, f=f, l=l, grid=units * 256:
                     f"k_grouped<{f}, {l}, false>" in n and g == grid)
                dur = [x[3] for x in select(trace, m)][:KT_STEPS * LAYER_LAUNCHES]
                n, fb, wb, ratio = pmc(m, alg, lambda v: v[:PMC_STEPS * LAYER_LAUNCHES])
                lines_t.append(f"| {name} | {p} | {len(dur)} | {avg(dur) / 1e3:,.2f} | "
                               f"{lo(dur) / 1e3:,.2f} | {hi(dur) / 1e3:,.2f} | {alg / avg(dur):,.0f} |")
                lines_c.append(f"| {name} | {p} | {n} | {alg:,} | {fb:,.0f} | {wb:,.0f} | {ratio:.4f} |")
                per_alg.append(alg)
                per_traf.append(fb + wb)
            out["kernels"][name] = {
                "workload": "Qwen3-235B-A22B-shaped layer, 16 experts per launch, mean of the "
                            "gate_up and down launches", **src("grouped"),
                "traffic_bytes_per_launch": rnd(avg(per_traf)),
                "alg_bytes_per_launch": round(avg(per_alg)),
                "ratio": rnd(avg(per_traf) / avg(per_alg), 4)}
    write_md("k_grouped_qwen3_235b_layer.md",
             "k_grouped -- Qwen3-235B-A22B-shaped MoE layer, 16 experts per launch, MI355X",
             "## Kernel trace (per dispatch, from kt_kernel_trace.csv)\n\n"
             "gate_up = 16 x bf16 [3072,4096], down = 16 x bf16 [4096,1536]; 6 steps of 8 "
             "dispatches each (1 warm-up + 5 timed steps, each step one of the 8 streamed layers).  "
             "GB/s = algorithmic bytes / average duration.\n\n"
             "| kernel | launch | n | avg us | min us | max us | GB/s |\n|---|---|---|---|---|---|---|\n"
             + "\n".join(lines_t) + "\n\n"
             "The benchmark's `per_kernel.avg_us` comes from HIP events at the boundaries of each "
             "run of 8 same-kind launches (run time over 8, mean of gate_up and down), so it "
             "includes the gaps between launches and reads a few us longer than the trace's "
             "per-dispatch average.\n\n"
             "## HBM traffic (FETCH_SIZE + WRITE_SIZE per dispatch)\n\n" + calib + "\n"
             "| kernel | launch | n | algorithmic B | fetch B | write B | traffic / algorithmic |\n"
             "|---|---|---|---|---|---|---|\n" + "\n".join(lines_c) + "\n")

    # ------------------------------------- grouped against per-expert dispatch
    # Qwen3-30B-A3B layers, MXFP8 swizzled: each layer is 8 gate_up + 8 down
    # grouped launches, or 128 + 128 single-expert launches, back to back; the
    # serial grouped passes over the 48 layers come first
    rows_l, spans = [], {}
    # bench.timed makes 3 warm-up and 5 timed passes over the 48 layers: the
    # plain grouped passes, then the per-expert passes (first 4 layers), then
    # the chained grouped passes, the two-stream passes joined once per pass
    # and those joined once per layer (same grids as the plain ones; the
    # trace lists dispatches in issue order)
    n_pass_layers = (3 + 5) * C2_LAYERS
    for kind, per in (("grouped", 16), ("per-expert", 1)):
        grids = {p: per * (-(-r // 128) * 128 // 16) * (-(-c // 512)) * 256
                 for p, (r, c) in workloads.QWEN3_30B_A3B.items()}
        seq = [x for x in trace if "k_grouped<0, 1, false>" in x[1] and x[2] in grids.values()]
        n_call = 2 * 128 // per  # launches per layer
        layers = [seq[i:i + n_call] for i in range(0, len(seq) - n_call + 1, n_call)]
        if kind == "grouped":
            chained = layers[n_pass_layers:2 * n_pass_layers]
            two_once = layers[2 * n_pass_layers:3 * n_pass_layers]
            two_layer = layers[3 * n_pass_layers:4 * n_pass_layers]
            layers = layers[:n_pass_layers]
        seq = [x for L in layers for x in L]
        kern = [sum(x[3] for x in L) for L in layers]
        span = [L[-1][5] - L[0][4] for L in layers]
        spans[kind] = (n_call, avg(kern), avg(span))
        for p, g in grids.items():
            dur = [x[3] for x in seq if x[2] == g]
            rows_l.append(f"| {kind} | {p} | {g // 256} | {len(dur)} | {avg(dur) / 1e3:,.2f} |")
    (ng, kg, sg), (ne, ke, se) = spans["grouped"], spans["per-expert"]
    # chained launches overlap, so a layer's time is its span (first start to
    # last end of its 16 launches)
    sc_ = avg([L[-1][5] - L[0][4] for L in chained])

    # launches on two streams overlap: a pass's time is its first start to its
    # last end, over its 48 layers; a layer joined on its own, its own span
    def span_of(Ls):
        return max(x[5] for L in Ls for x in L) - min(x[4] for L in Ls for x in L)
    passes = [two_once[i:i + C2_LAYERS] for i in range(0, len(two_once), C2_LAYERS)]
    s2o = avg([span_of(P) / len(P) for P in passes])
    s2l = avg([span_of([L]) for L in two_layer])
    alg30 = sum(128 * (r * c * 3 + sf_bytes(r, c // 32, 1))
                for r, c in workloads.QWEN3_30B_A3B.values())
    write_md("k_grouped_qwen3_30b_a3b_grouped_vs_per_expert.md",
             "k_grouped -- Qwen3-30B-A3B-shaped MoE layer, MXFP8 swizzled: 16 grouped launches "
             "against 256 per-expert launches, MI355X",
             "128 experts of gate_up bf16 [1536,2048] and 128 of down bf16 [2048,768] "
             f"({alg30:,} algorithmic bytes per layer).  Grouped: 16 experts per launch, "
             "8 + 8 launches; per-expert: one launch per expert, 128 + 128.  The same kernel "
             "and bytes either way.\n\n"
             "| dispatch | launch | workgroups | n | avg us |\n|---|---|---|---|---|\n"
             + "\n".join(rows_l) + "\n\n"
             "| per layer | launches | kernel time us (sum) | traced span us (first start to last end) | GB/s over the span |\n"
             "|---|---|---|---|---|\n"
             f"| grouped | {ng} | {kg / 1e3:,.1f} | {sg / 1e3:,.1f} | {alg30 / sg:,.0f} |\n"
             f"| grouped, chained (MXQ_CHAIN) | {ng} | launches overlap | {sc_ / 1e3:,.1f} | "
             f"{alg30 / sc_:,.0f} |\n"
             f"| grouped, two streams, one join per {C2_LAYERS} layers | {ng} | launches overlap | "
             f"{s2o / 1e3:,.1f} | {alg30 / s2o:,.0f} |\n"
             f"| grouped, two streams, one join per layer | {ng} | launches overlap | "
             f"{s2l / 1e3:,.1f} | {alg30 / s2l:,.0f} |\n"
             f"| per-expert | {ne} | {ke / 1e3:,.1f} | {se / 1e3:,.1f} | {alg30 / se:,.0f} |\n\n"
             "Chained: mx_quant_grouped_batch with MXQ_CHAIN, the 7 launches after the first of "
             "each call dispatched any-order; a layer's time is the span of its 16 launches.  "
             f"Mean over the {len(chained)} chained layer passes; plain grouped over "
             f"{n_pass_layers}.  Two streams: issue_interleaved, launch j of each call on side "
             "stream j % 2, the streams joined back to the caller's once per pass over the "
             f"{C2_LAYERS} layers (the pass's span over {C2_LAYERS}; mean of {len(passes)} passes) "
             f"or once per layer (the layer's span; mean of {len(two_layer)}).\n\n"
             f"Each launch beyond the 16 grouped ones costs {(ke - kg) / (ne - ng) / 1e3:.2f} us of "
             "kernel time: the fixed ramp and tail of a launch, which grouping pays once per 16 "
             "experts.  Kernel tracing adds its own host-side cost to every launch, so the traced "
             f"span ({(se - sg) / (ne - ng) / 1e3:.2f} us per extra launch) overstates the gap; "
             "bench.py reports the untraced layer times over all 48 layers "
             "(`other_workloads.qwen3_30b_a3b_48_layers_mxfp8_swizzled`).\n")

    # ------------------------------------------------ encode scales from data
    r, c = shapes["gate_up"]
    gq = 16 * (-(-r // 128) * 128 // 16) * (c // 512) * 256
    alg_q = 16 * (r * c * 2 + r * c // 2 + sf_bytes(r, c // 16, 1) + 8)
    alg_a = 16 * r * c * 2
    rows_a = []
    for kname, m, alg in (
            ("k_amax", lambda n, g: n.startswith("mxq::k_amax"), alg_a),
            ("k_grouped<NVFP4,SWIZZLED,auto>",
             lambda n, g: "k_grouped<1, 1, true>" in n and g == gq, alg_q)):
        dur = [x[3] for x in select(trace, m)]
        n, fb, wb, ratio = pmc(m, alg)
        rows_a.append(f"| {kname} | {len(dur)} | {avg(dur) / 1e3:,.2f} | {alg:,} | "
                      f"{alg / avg(dur):,.0f} | {fb:,.0f} | {wb:,.0f} | {ratio:.4f} |")
    dz = [x[3] for x in select(trace, lambda n, g: n.startswith("mxq::k_zero_slots"))]
    write_md("k_amax_auto_scale_qwen3_235b_gate_up.md",
             "nvfp4_quant_grouped_auto -- 16 x bf16 [3072,4096] (Qwen3-235B-A22B gate_up), "
             "swizzled, MI355X",
             "Three kernels per call: k_zero_slots (16 accumulators), k_amax (reads the input), "
             "k_grouped<NVFP4,SWIZZLED> with encode scales from the amax (reads it again).  "
             f"k_zero_slots: {len(dz)} dispatches, {avg(dz) / 1e3:.2f} us average.\n\n" + calib + "\n"
             "| kernel | n | avg us | algorithmic B | GB/s | fetch B | write B | traffic / algorithmic |\n"
             "|---|---|---|---|---|---|---|---|\n" + "\n".join(rows_a) + "\n")
    out["kernels"]["k_amax"] = src("grouped")

    # -------------------------------------------------------------- split
    T, H = 8192, 7168
    _, split = workloads.routed_activation()
    rows_s = []
    for key, (f, rs) in {"nvfp4": ("1", "false"), "nvfp4_row_scaled": ("1", "true"),
                         "mxfp8": ("0", "false")}.items():
        for l in "01":
            fmt = int(f)
            C = H // (32 if fmt == 0 else 16)
            pay = T * (H if fmt == 0 else H // 2)
            alg = (T * H * 2 + pay + sum(sf_bytes(m, C, int(l)) for m in split) + 4 * T
                   + (4 if key == "nvfp4" else 0))
            # 512-column steps per wave at 7168 columns: 7 with two waves per row
            # (swizzled), 4 with four (linear)
            nch = 7 if l == "1" else 4
            m = lambda n, g, f=f, rs=rs, l=l, nch=nch: f"k_split<{f}, {rs}, {l}, {nch}>" in n
            dur = [x[3] for x in select(trace, m)]
            n, fb, wb, ratio = pmc(m, alg)
            rows_s.append(f"| {key} | {LAY[l]} | {len(dur)} | {avg(dur) / 1e3:,.2f} | {alg:,} | "
                          f"{alg / avg(dur):,.0f} | {fb:,.0f} | {wb:,.0f} | {ratio:.4f} |")
            out["kernels"][f"k_split<{key},{LAY[l]}>"] = {
                "workload": "routed activation bf16 [8192,7168], 256 experts (10 empty)",
                **src("split"), "traffic_bytes_per_launch": rnd(fb + wb),
                "alg_bytes_per_launch": alg, "ratio": rnd(ratio, 4)}
    write_md("k_split_routed_8192x7168.md",
             "k_split -- routed activation bf16 [8192,7168] split over 256 experts "
             "(10 empty, 19-55 rows each), MI355X",
             "Algorithmic bytes: bf16 input + payload + every expert's (padded) scale region + "
             "4 B of row amax per row.  8 input copies rotate (more than the 256 MB last-level "
             "cache).  Linear scales: one-row units of four waves; swizzled: two-row units of "
             "two waves per row.\n\n" + calib + "\n"
             "| form | scales | n | avg us | algorithmic B | GB/s | fetch B | write B | traffic / algorithmic |\n"
             "|---|---|---|---|---|---|---|---|---|\n" + "\n".join(rows_s) + "\n")

    # -------------------------------------------------------------- fused
    rows_f = []
    for f in "01":
        fmt = int(f)
        by_grid = collections.defaultdict(list)
        for Tt in (1, 16, 64, 256, 1024, 4096):
            if Tt == 1 or 16 < Tt < 32:
                # k_fused_tiny: one 1024-thread workgroup per live row
                by_grid[("k_fused_tiny<" + f + ">", Tt * 1024)].append(Tt)
                continue
            # swizzled units cover the padding rows: sixteen waves per row up to
            # T = 512, four up to 1536, else two waves and four rows per unit
            rt = -(-Tt // 128) * 128
            grid = rt * 1024 if Tt <= 512 else rt * 256 if Tt <= 1536 else rt // 4 * 512
            by_grid[(f"k_fused<{f}, 1,", grid)].append(Tt)
        for (kname, grid), Ts in by_grid.items():
            for k, Tt in enumerate(Ts):
                pw = H if fmt == 0 else H // 2
                nsc = sf_bytes(Tt, H // (32 if fmt == 0 else 16), 1)
                alg = Tt * H * 8 + Tt * pw + nsc + 2 * H + (4 if fmt else 0)
                m = lambda n, g, kname=kname, grid=grid: kname in n and g == grid

                def nth(rows, k=k, nT=len(Ts)):  # T values sharing a grid run in order
                    per = len(rows) // nT
                    return rows[k * per:(k + 1) * per]
                dur = [x[3] for x in nth(select(trace, m))]
                n, fb, wb, ratio = pmc(m, alg, nth)
                rows_f.append(f"| {FMT[f]} | {Tt} | {len(dur)} | {avg(dur) / 1e3:,.2f} | "
                              f"{pct(dur, 0.5) / 1e3:,.2f} | {pct(dur, 0.1) / 1e3:,.2f} | {alg:,} | "
                              f"{alg / avg(dur):,.0f} | {fb:,.0f} | {wb:,.0f} | {ratio:.4f} |")
                if Tt == 4096:
                    out["kernels"][f"k_fused<{FMT[f]},SWIZZLED>"] = {
                        "workload": "residual + RMSNorm + quantize, T=4096, H=7168", **src("fused"),
                        "traffic_bytes_per_launch": rnd(fb + wb), "alg_bytes_per_launch": alg,
                        "ratio": rnd(ratio, 4)}
    write_md("k_fused_rmsnorm_h7168.md",
             "k_fused -- residual add + RMSNorm + quantize, H = 7168, swizzled scales, MI355X",
             "Algorithmic bytes: x, residual in (4 B/elem), residual_out, norm_out (4 B/elem), "
             "payload, padded scales, gamma.  T = 1 runs k_fused_tiny: one 1024-thread "
             "workgroup for the live row, which also writes the padding rows' zero scales.  "
             "Otherwise T <= 512 runs sixteen waves per row (1024-thread workgroups), T = 1024 "
             "four (256 threads), one row per workgroup (the padding rows of a swizzled 128-row "
             "tile are workgroups of their own); T = 4096 runs two waves per row, four rows per "
             "512-thread workgroup.  T = 16 and 64 share one grid (128 workgroups), as do "
             "T = 256 and 1024; their dispatches are told apart by order.  bench.py times each "
             "T as replays of a captured graph of 8 calls (a decode step runs the epilogue "
             "inside a graph; called one at a time from Python, the host's cost per call "
             "exceeds the kernel's and the GPU idles between launches).\n\n" + calib + "\n"
             "Durations at small T are bimodal from launch to launch (medians of 3.9 or 4.7 us "
             "at T = 16 in different runs), so the median and the 10th percentile stand beside "
             "the mean; GB/s is over the mean.\n\n"
             "| format | T | n | avg us | median us | p10 us | algorithmic B | GB/s | fetch B | write B | traffic / algorithmic |\n"
             "|---|---|---|---|---|---|---|---|---|---|---|\n" + "\n".join(rows_f) + "\n")

    # ------------------------------------------------------------ swizzle
    rs_, cs_ = 16 * 3072, 128
    alg = rs_ * cs_ + -(-rs_ // 128) * 128 * cs_
    m = lambda n, g: n.startswith("mxq::k_swizzle")
    dur = [x[3] for x in select(trace, m)]
    n, fb, wb, ratio = pmc(m, alg)
    write_md("k_swizzle_49152x128.md",
             "k_swizzle -- linear MXFP8 scales of a 16-expert Qwen3-235B-A22B gate_up launch "
             "(u8 [49152,128]) to the swizzled 128x4 layout, MI355X",
             "Algorithmic bytes: the linear matrix in, the swizzled matrix out.  48 input/output "
             "pairs rotate (604 MB, more than the 256 MB last-level cache).\n\n" + calib + "\n"
             "| kernel | n | avg us | algorithmic B | GB/s | fetch B | write B | traffic / algorithmic |\n"
             "|---|---|---|---|---|---|---|---|\n"
             f"| k_swizzle | {len(dur)} | {avg(dur) / 1e3:,.2f} | {alg:,} | {alg / avg(dur):,.0f} | "
             f"{fb:,.0f} | {wb:,.0f} | {ratio:.4f} |\n")
    out["kernels"]["k_swizzle"] = {
        "workload": "u8 [49152,128] linear -> swizzled", **src("fused"),
        "traffic_bytes_per_launch": rnd(fb + wb), "alg_bytes_per_launch": alg,
        "ratio": rnd(ratio, 4)}

    # ------------------------------------- vector ALU busy, memory-unit stall
    # (two more counter runs of the layer alone, when DIR holds them)
    valu_csv = os.path.join(d, "pmc_valu", "v_counter_collection.csv")
    ms_csv = os.path.join(d, "pmc_ms", "m_counter_collection.csv")
    if os.path.exists(valu_csv) and os.path.exists(ms_csv):
        write_valu_summary(valu_csv, ms_csv, out_dir)

    stats_csv = os.path.join(d, "prof_kt", "kt_kernel_stats.csv")
    if os.path.exists(stats_csv):
        write_stats_summary(stats_csv, out_dir)

    with open(os.path.join(out_dir, "hbm_traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    for name in sorted(os.listdir(out_dir)):
        if name.endswith(".md"):
            print(f"wrote {os.path.join(out_dir, name)}")


if __name__ == "__main__":
    main()
