#!/usr/bin/env python3
"""Benchmark: grouped block-scaled quantization of a Qwen3-235B-A22B-shaped MoE
layer on one MI355X.

One step quantizes one layer (128 experts of gate_up bf16 [3072,4096] and 128
of down bf16 [4096,1536], N(0, 0.015^2) with 1e-4 of entries x50) held in a
reused stacking buffer: MXFP8 and NVFP4, each with linear and with swizzled
scales, 16 experts per launch (64 launches per step).  Inputs are resident in
HBM before timing starts.  The value is whole-step algorithmic bytes (bf16 in
+ payload + scales + per-expert encode scales) over wall time.

Also reported: per-kernel HIP-event durations and the roofline of the
dominant kernel, the CPU oracle on a bounded sample of the same workload,
and secondary workloads (Qwen3-30B-A3B layer grouped vs per-expert launch,
the [8192,7168] routed-activation split, the residual+RMSNorm+quant sweep,
the small grouped case, a device copy as attainable-bandwidth reference).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "nvfp4_quantization_moe_amd", "csrc")


def code_text(text):
    """C/C++ source with comments removed and whitespace runs collapsed: what
    the compiler sees of it, so that editing a comment changes nothing."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(files):
    """sha256 over the code (not the comments) of the given csrc files."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated on a device copy), or None
    when a source the kernel is built from changed since the counters were
    taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            k = json.load(f)["kernels"][kernel]
        if k["source_sha256"] != source_hash(k["sources"]):
            return None
        return k["traffic_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


class HipTimingEvents:
    """Per-launch timing events created with hipEventDisableSystemFence: a
    plain event record ends with a system-scope fence (cache writeback and
    invalidation) that slows the launches around it; these events only time.
    Uses the HIP runtime torch has loaded (the same one the library uses)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events.append(ev)

    def record(self, k, stream):
        if self.hip.hipEventRecord(self.events[k], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.events[a], self.events[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


def caller_encode_scales(amax):
    """The caller's NVFP4 encode scales for the precomputed-scale calls: the
    usual choice fp32(2688 / amax) (1 for an all-zero tensor), capped at
    FLT_MAX * 2^-9 as the library caps the scales it derives itself.  Input
    preparation, computed untimed; any positive finite fp32 is a valid g."""
    import torch
    a = amax.to(torch.float32)
    g = torch.where(a > 0, torch.full_like(a, 2688.0) / a, torch.ones_like(a))
    return torch.clamp(g, max=float.fromhex("0x1.fffffep+118"))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--cpu-experts", type=int, default=32,
                    help="gate_up experts in the single-thread MXFP8 CPU oracle sample")
    ap.add_argument("--layers", type=int, default=8,
                    help="resident Qwen3-235B-A22B layers the steps cycle through")
    ap.add_argument("--c2-layers", type=int, default=48,
                    help="Qwen3-30B-A3B layers streamed in the secondary workloads")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy first (hardware-counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the grouped quantization shards by expert with no exchange; "
              "run it per GPU with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_quantization_moe_amd as mxq
    from nvfp4_quantization_moe_amd import workloads

    mxq.lib()  # fail loudly without the built library
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    E, G = workloads.N_EXPERTS, workloads.GROUP
    shapes = workloads.QWEN3_235B_A22B
    L = args.layers
    log(f"[bench] generating {L} layers (seeds 5000 + l): {E} x gate_up {shapes['gate_up']} + "
        f"{E} x down {shapes['down']} bf16 each, resident in HBM")
    layers = [workloads.moe_layer(shapes, l, 5000, 0.015, device=dev) for l in range(L)]
    gsc = [{p: caller_encode_scales(lay[p].float().abs().amax(dim=(1, 2))).contiguous()
            for p in lay} for lay in layers]
    torch.cuda.synchronize()

    # outputs, reused by every layer: one payload buffer per format and
    # projection (both layouts write the same payload bytes), one scale
    # buffer per (format, layout, projection)
    outs = {}
    for fmt in (mxq.MXFP8, mxq.NVFP4):
        for proj, (r, c) in shapes.items():
            pw = c if fmt == mxq.MXFP8 else c // 2
            outs[(fmt, proj)] = torch.empty(E, r, pw, dtype=torch.uint8, device=dev)
            for layout in (mxq.LINEAR, mxq.SWIZZLED):
                outs[(fmt, layout, proj)] = torch.empty(E, mxq.scale_bytes(r, c, fmt, layout),
                                                        dtype=torch.uint8, device=dev)
    # calls[l]: layer l's 64 launches, (fmt, layout, proj, GroupedCall, bytes)
    calls = []
    alg_bytes = {}
    for l, lay in enumerate(layers):
        cl = []
        for fmt in (mxq.MXFP8, mxq.NVFP4):
            for proj, (r, c) in shapes.items():
                pw = c if fmt == mxq.MXFP8 else c // 2
                pay = outs[(fmt, proj)]
                for layout in (mxq.LINEAR, mxq.SWIZZLED):
                    sc = outs[(fmt, layout, proj)]
                    nsc = sc.shape[1]
                    for b in range(0, E, G):
                        srcs = [lay[proj][b + i] for i in range(G)]
                        gs = gsc[l][proj][b:b + G] if fmt == mxq.NVFP4 else None
                        call = mxq.GroupedCall(fmt, layout, srcs, [pay[b + i] for i in range(G)],
                                               [sc[b + i] for i in range(G)], gs)
                        nbytes = G * (r * c * 2 + r * pw + nsc + (4 if fmt == mxq.NVFP4 else 0))
                        cl.append((fmt, layout, proj, call, nbytes))
                        if l == 0:
                            alg_bytes[(fmt, layout)] = alg_bytes.get((fmt, layout), 0) + nbytes
        calls.append(cl)
    step_bytes = sum(c[4] for c in calls[0])

    import ctypes
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    # Launches of one kernel kind (format, layout, projection) run back to
    # back in runs of E/G; timing events sit only at run boundaries, so the
    # timed region carries 17 event records per step instead of two per
    # launch.  A launch's duration is its run's time over the run's launches
    # (the gaps between them count against the kernel).  Step s quantizes
    # layer s mod L.
    runs = []  # (first call index, end index)
    c0 = calls[0]
    for k in range(len(c0)):
        if k == 0 or c0[k][:3] != c0[k - 1][:3]:
            runs.append([k, k + 1])
        else:
            runs[-1][1] = k + 1
    n_ev = len(runs) + 1

    def step(s, timer=None, base=0):
        cl = calls[s % L]
        for j, (k0, k1) in enumerate(runs):
            if timer is not None:
                timer.record(base + j, stream)
            for k in range(k0, k1):
                cl[k][3](stream)
        if timer is not None:
            timer.record(base + len(runs), stream)

    if args.calib_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"[bench] warmup {args.warmup} steps ({len(calls[0])} launches/step)")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    timer = HipTimingEvents(n_ev * args.steps)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s, timer, n_ev * s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_bytes * args.steps / elapsed / 1e9

    # per-kernel durations from the events
    names = {(0, 0): "k_grouped<MXFP8,LINEAR>", (0, 1): "k_grouped<MXFP8,SWIZZLED>",
             (1, 0): "k_grouped<NVFP4,LINEAR>", (1, 1): "k_grouped<NVFP4,SWIZZLED>"}
    per = {}
    for s in range(args.steps):
        for j, (k0, k1) in enumerate(runs):
            fmt, layout = c0[k0][0], c0[k0][1]
            ms = timer.elapsed_ms(n_ev * s + j, n_ev * s + j + 1)
            d = per.setdefault((fmt, layout), {"ms": 0.0, "n": 0, "bytes": 0})
            d["ms"] += ms
            d["n"] += k1 - k0
            d["bytes"] += sum(c0[k][4] for k in range(k0, k1))
    # spread of the per-step GPU time (events at each step's ends), and the
    # mean GPU time of each layer's steps
    step_list = [timer.elapsed_ms(n_ev * s, n_ev * s + len(runs)) for s in range(args.steps)]
    step_ms = sorted(step_list)
    per_layer = {}
    for s, ms in enumerate(step_list):
        per_layer.setdefault(s % L, []).append(ms)
    layer_ms = {str(l): round(sum(v) / len(v), 4) for l, v in sorted(per_layer.items())}

    def pct(p):
        return round(step_ms[min(len(step_ms) - 1, int(p * len(step_ms)))], 4)
    timer.close()
    per_kernel = {}
    for key, d in per.items():
        avg_us = d["ms"] * 1e3 / d["n"]
        gbs = d["bytes"] / (d["ms"] * 1e-3) / 1e9
        per_kernel[names[key]] = {"launches": d["n"], "avg_us": round(avg_us, 2),
                                  "alg_bytes_per_launch": d["bytes"] // d["n"],
                                  "GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    dom = max(per, key=lambda k: per[k]["ms"])
    dd = per[dom]
    achieved = dd["bytes"] / (dd["ms"] * 1e-3) / 1e9
    roofline = {"kernel": names[dom], "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(names[dom]),
                "alg_bytes_per_launch": dd["bytes"] // dd["n"],
                "avg_launch_us": round(dd["ms"] * 1e3 / dd["n"], 2)}
    log(f"[bench] step {ms_per_step:.3f} ms, {value:.1f} GB/s; dominant {names[dom]} "
        f"{achieved:.1f} GB/s")

    out = {
        "metric": "effective HBM GB/s (bytes in+out) and % of HBM peak, grouped expert quant",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->mxfp8/nvfp4",
        "data": "synthetic",
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "step_ms_gpu": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)},
        "config": {
            "workload": f"Qwen3-235B-A22B-shaped MoE layers streamed: {L} layers (seeds 5000+l) "
                        "of 128 experts gate_up bf16 [3072,4096] + 128 down bf16 [4096,1536], "
                        "N(0,0.015^2) with 1e-4 outliers x50, resident in HBM; one step = one "
                        "layer (step s quantizes layer s mod L) in MXFP8 and NVFP4, linear and "
                        "swizzled scales, 16 experts per launch",
            "layers": L, "experts": E, "experts_per_launch": G,
            "launches_per_step": len(calls[0]),
            "alg_bytes_per_step": step_bytes,
            "alg_bytes_per_layer": {"mxfp8": alg_bytes[(0, 0)], "nvfp4": alg_bytes[(1, 0)]},
        },
        "layer_ms_gpu": layer_ms,
        "per_kernel": per_kernel,
        "roofline": roofline,
    }

    if not args.no_extra:
        # context, not the headline: the same step with the MXFP8 launches on
        # one stream and the NVFP4 launches on another (default priority), so
        # that one launch's ramp and tail overlap the other stream's work
        side = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
        side_h = [ctypes.c_void_p(q.cuda_stream) for q in side]

        def step_two_streams():
            cur = torch.cuda.current_stream(dev)
            for q in side:
                q.wait_stream(cur)
            for fmt, _, _, call, _ in calls[0]:
                call(side_h[0 if fmt == mxq.MXFP8 else 1])
            for q in side:
                cur.wait_stream(q)
        step_two_streams()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step_two_streams()
        torch.cuda.synchronize()
        t2 = (time.perf_counter() - t0) / args.steps
        out["step_two_streams"] = {"ms_per_step": round(t2 * 1e3, 4),
                                   "GBps": round(step_bytes / t2 / 1e9, 1)}
        out["other_workloads"] = extra_workloads(torch, mxq, workloads, dev, args.c2_layers, side)
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (the oracle)")
        out["cpu_baseline"] = cpu_baseline(torch, layers[0]["gate_up"], gsc[0]["gate_up"],
                                           args.cpu_experts)
    print(json.dumps(out), flush=True)


def timed(torch, fn, iters, warm=3, reps=5):
    """Seconds per call: the median over `reps` blocks of `iters` calls."""
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(iters):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / iters * 1e-3)
    return sorted(per)[len(per) // 2]


def extra_workloads(torch, mxq, workloads, dev, n_layers=48, side=None):
    import ctypes
    res = {}
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    # attainable-bandwidth reference: a 4 GiB device copy (read + write)
    n = 1 << 31
    a = torch.empty(n, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    t = timed(torch, lambda i: b.copy_(a), 10)
    res["d2d_copy_4GiB"] = {"GBps": round(2 * n * 2 / t / 1e9, 1)}
    del a, b

    # Qwen3-30B-A3B model, MXFP8 swizzled: all 48 layers (seeds 2000 + l)
    # resident and streamed, 16 grouped launches per layer; against 256
    # per-expert launches per layer on the first 4 layers
    E, G = workloads.N_EXPERTS, workloads.GROUP
    shapes30 = workloads.QWEN3_30B_A3B
    log(f"[bench] generating {n_layers} Qwen3-30B-A3B layers")
    layers30 = [workloads.moe_layer(shapes30, l, 2000, 0.02, device=dev) for l in range(n_layers)]
    outs30 = {p: (torch.empty(E, r, c, dtype=torch.uint8, device=dev),
                  torch.empty(E, mxq.scale_bytes(r, c, 0, 1), dtype=torch.uint8, device=dev))
              for p, (r, c) in shapes30.items()}
    nbytes = sum(E * (r * c * 3 + outs30[p][1].shape[1]) for p, (r, c) in shapes30.items())
    grouped, chained = [], []  # per layer and projection: one call of 8 launches
    single = []   # per layer (first 4): its 256 launches
    for l, lay in enumerate(layers30):
        sl = []
        for p in shapes30:
            pay, sc = outs30[p]
            srcs = [lay[p][i] for i in range(E)]
            grouped.append(mxq.GroupedCall(0, 1, srcs, [pay[i] for i in range(E)],
                                           [sc[i] for i in range(E)]))
            chained.append(mxq.GroupedCall(0, 1, srcs, [pay[i] for i in range(E)],
                                           [sc[i] for i in range(E)], chain=True))
            if l < min(4, n_layers):
                sl += [mxq.GroupedCall(0, 1, [lay[p][i]], [pay[i]], [sc[i]]) for i in range(E)]
        if sl:
            single.append(sl)
    tg = timed(torch, lambda i: [c() for c in grouped], 1) / n_layers
    ts = timed(torch, lambda i: [c() for sl in single for c in sl], 1) / len(single)
    # the same calls with MXQ_CHAIN: within each call, launches after the
    # first are dispatched any-order and start while the previous one drains
    t2 = timed(torch, lambda i: [c() for c in chained], 1) / n_layers
    # the same calls over two side streams (default priority), launch j of
    # each call on stream j % 2, joined back once per pass over the layers or
    # once per layer; each output slice is written from one stream.  The
    # side streams are the ones the two-stream step used: a process gets 4
    # hardware queues (HIP's default), and streams beyond them share one,
    # which serializes them (measured 359 instead of 289 us per layer)
    if side is None:
        side = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    tw = timed(torch, lambda i: mxq.issue_interleaved(grouped, side), 1) / n_layers
    tl = timed(torch, lambda i: [mxq.issue_interleaved(grouped[2 * l:2 * l + 2], side)
                                 for l in range(n_layers)], 1) / n_layers
    per_launch = len(single[0]) - 2 * E // G
    res["qwen3_30b_a3b_48_layers_mxfp8_swizzled"] = {
        "layers": n_layers, "alg_bytes_per_layer": nbytes,
        "grouped_16_launches_us_per_layer": round(tg * 1e6, 1),
        "grouped_GBps": round(nbytes / tg / 1e9, 1),
        "grouped_chained_us_per_layer": round(t2 * 1e6, 1),
        "chained_GBps": round(nbytes / t2 / 1e9, 1),
        "two_streams_one_join_us_per_layer": round(tw * 1e6, 1),
        "two_streams_one_join_GBps": round(nbytes / tw / 1e9, 1),
        "two_streams_join_per_layer_us_per_layer": round(tl * 1e6, 1),
        "per_expert_256_launches_us_per_layer": round(ts * 1e6, 1),
        "per_expert_GBps": round(nbytes / ts / 1e9, 1),
        "overhead_per_extra_launch_us": round((ts - tg) / per_launch * 1e6, 2)}
    del layers30, outs30, grouped, chained, single
    torch.cuda.empty_cache()

    log("[bench] stacking copy against the descriptor table")
    # the pages' flow for comparison: stack 16 experts into one buffer, then
    # quantize the stack as one tensor (MXFP8, swizzled; Qwen3-235B gate_up)
    r, c = workloads.QWEN3_235B_A22B["gate_up"]
    stack = workloads.expert_stack(G, r, c, std=0.015, seed=5000, device=dev)
    experts = [stack[i].clone() for i in range(G)]  # separate allocations, as in a model
    flat = torch.empty(G * r, c, dtype=torch.bfloat16, device=dev)
    in_place = mxq.GroupedCall(0, 1, experts)
    one_tensor = mxq.GroupedCall(0, 1, [flat])

    def stack_then_quantize(i):
        torch.stack(experts, out=flat.view(G, r, c))
        one_tensor(stream)
    ts = timed(torch, stack_then_quantize, 20)
    tq = timed(torch, lambda i: one_tensor(stream), 20)
    tg = timed(torch, lambda i: in_place(stream), 20)
    nb = G * (r * c * 3 + mxq.scale_bytes(r, c, 0, 1))
    res["stack_vs_descriptor_qwen3_235b_gate_up_mxfp8"] = {
        "alg_bytes": nb, "descriptor_table_us": round(tg * 1e6, 1),
        "stack_then_quantize_us": round(ts * 1e6, 1), "quantize_stacked_only_us": round(tq * 1e6, 1)}
    del stack, experts, flat, in_place, one_tensor

    log("[bench] encode scales from the data")
    # NVFP4 with encode scales from the data, same call (amax pass + quantize):
    # one Qwen3-235B-A22B gate_up launch of 16 experts, swizzled
    r, c = workloads.QWEN3_235B_A22B["gate_up"]
    stack = workloads.expert_stack(G, r, c, std=0.015, seed=5000, device=dev)
    auto = mxq.GroupedAutoCall(1, [stack[i] for i in range(G)])
    gs = caller_encode_scales(stack.float().abs().amax(dim=(1, 2))).contiguous()
    plain = mxq.GroupedCall(1, 1, [stack[i] for i in range(G)], auto.payloads, auto.scales, gs)

    def torch_amax_then_grouped(i):
        a = torch.linalg.vector_norm(stack, ord=float("inf"), dim=(1, 2)).float()
        gs.copy_(torch.where(a > 0, 2688.0 / a, torch.ones_like(a)))
        plain()
    ta = timed(torch, lambda i: auto(), 20)
    tp = timed(torch, lambda i: plain(), 20)
    tt = timed(torch, torch_amax_then_grouped, 20)
    nb = G * (r * c * 2 + r * c // 2 + mxq.scale_bytes(r, c, 1, 1) + 8)
    res["nvfp4_auto_scale_qwen3_235b_gate_up_16x3072x4096"] = {
        "alg_bytes": nb, "hbm_bytes_two_pass": nb + G * r * c * 2,
        "auto_us": round(ta * 1e6, 1), "auto_GBps_alg": round(nb / ta / 1e9, 1),
        "auto_GBps_two_pass": round((nb + G * r * c * 2) / ta / 1e9, 1),
        "precomputed_g_us": round(tp * 1e6, 1),
        "torch_amax_then_grouped_us": round(tt * 1e6, 1)}
    del stack, auto, plain

    log("[bench] routed activation split")
    # routed activation split, 8 rotating input copies (> MALL): NVFP4 with one
    # encode scale, row-scaled NVFP4, MXFP8; linear and swizzled scales
    x, split = workloads.routed_activation()
    xs = [x.to(dev) for _ in range(8)]
    g = caller_encode_scales(xs[0].float().abs().amax()).reshape(1)
    T, H = x.shape
    am = torch.empty(T, dtype=torch.float32, device=dev)
    splits = {}
    for mode, fmt in (("nvfp4", 1), ("nvfp4_row_scaled", 1), ("mxfp8", 0)):
        pay = torch.empty(T, H if fmt == 0 else H // 2, dtype=torch.uint8, device=dev)
        for layout, lname in ((0, "linear"), (1, "swizzled")):
            total = mxq.split_scale_offset(split, len(split), H, fmt, layout)
            sc = torch.empty(total, dtype=torch.uint8, device=dev)
            scs = [mxq.SplitCall(mode, xs[k], split, layout, g if mode == "nvfp4" else None,
                                 pay, sc, am) for k in range(8)]
            t = timed(torch, lambda i: scs[i % 8](stream), 20)
            nb = T * H * 2 + pay.numel() + total + 4 * T + (4 if mode == "nvfp4" else 0)
            splits[f"{mode}_{lname}"] = {"us": round(t * 1e6, 1), "alg_bytes": nb,
                                         "GBps": round(nb / t / 1e9, 1)}
    res["split_8192x7168_256experts"] = splits
    del xs

    log("[bench] fused epilogue sweep")
    # fused residual + RMSNorm + quantize (swizzled), MXFP8 and NVFP4, with the
    # same-run e4m3 cast reference.  Each is timed as replays of a captured
    # graph of 8 calls over 4 rotating inputs: a decode step runs the
    # epilogue inside a graph, and called one at a time from Python the
    # host's cost per call (about 5 us) exceeds the kernel's
    def graph_of(fns):
        for fn in fns:
            fn()  # warm, eager
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for k in range(8):
                fns[k % len(fns)]()
        return gr
    for fmt, fname in ((0, "mxfp8"), (1, "nvfp4")):
        sweep = {}
        for T in (1, 16, 64, 256, 1024, 4096):
            H = 7168
            ins = [workloads.epilogue_inputs(T, H, seed=4000 + T + k, device=dev) for k in range(4)]
            nsc = mxq.scale_bytes(T, H, fmt, 1)
            pw = H if fmt == 0 else H // 2
            outs = (torch.empty(T, H, dtype=torch.bfloat16, device=dev),
                    torch.empty(T, H, dtype=torch.bfloat16, device=dev),
                    torch.empty(T, pw, dtype=torch.uint8, device=dev),
                    torch.empty(nsc, dtype=torch.uint8, device=dev))
            gf = torch.ones(1, dtype=torch.float32, device=dev)
            fcs = [mxq.FusedCall(*ins[k], 1e-6, fmt, 1, gf, outs) for k in range(4)]
            gr = graph_of(fcs)
            t = timed(torch, lambda i: gr.replay(), 10) / 8
            nb = T * H * 8 + T * pw + nsc + 2 * H + (4 if fmt == 1 else 0)
            entry = {"us": round(t * 1e6, 2), "GBps": round(nb / t / 1e9, 1)}
            if fmt == 0:
                gc = graph_of([lambda k=k: ins[k][0].to(torch.float8_e4m3fn) for k in range(4)])
                tc = timed(torch, lambda i: gc.replay(), 10) / 8
                entry["e4m3_cast_us"] = round(tc * 1e6, 2)
                del gc
            sweep[str(T)] = entry
            del gr
        res[f"fused_rmsnorm_{fname}_H7168"] = sweep

    log("[bench] small grouped case, scale swizzle")
    # small grouped case: 8 x [256,512] MXFP8 linear (launch-bound)
    xs8 = [x.to(dev) for x in workloads.small_grouped_experts(seed=0)]
    call = mxq.GroupedCall(0, 0, xs8)
    t = timed(torch, lambda i: call(), 100)
    res["small_grouped_8x256x512_mxfp8"] = {"us": round(t * 1e6, 2),
                                            "GBps": round(3178496 / t / 1e9, 1)}

    # receiver-side scale conversion: the linear MXFP8 scales of one 16-expert
    # gate_up launch (16 x [3072, 128] stacked) to the swizzled layout, 48
    # rotating inputs and outputs (604 MB, more than the 256 MB last-level
    # cache holds), so each call reads and writes HBM
    nrot = 48
    lin = [torch.randint(0, 255, (16 * 3072, 128), dtype=torch.uint8, device=dev)
           for _ in range(nrot)]
    outs = [torch.empty(16 * 3072 * 128, dtype=torch.uint8, device=dev) for _ in range(nrot)]
    t = timed(torch, lambda i: mxq.scale_swizzle(lin[i % nrot], outs[i % nrot]), 2 * nrot)
    nb = 2 * 16 * 3072 * 128
    res["scale_swizzle_49152x128"] = {"us": round(t * 1e6, 2), "GBps": round(nb / t / 1e9, 1),
                                      "rotating_buffers": nrot}
    del lin, outs
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(torch, gate_up, g_gate_up, n_experts):
    """The oracle as it stands on the same input bytes the GPU quantized: the
    first n_experts gate_up experts of layer 0, MXFP8 with swizzled scales,
    single-threaded (the reported value); an NVFP4 sample (16 experts, their
    per-expert encode scales); and MXFP8 on 64 experts with one oracle call
    per expert on the host threads of the machine's CPU share for one GPU (the C
    call releases the GIL)."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    oracle.lib()
    n_experts = min(n_experts, gate_up.shape[0])
    n_all = min(64, gate_up.shape[0])
    host = gate_up[:n_all].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    g = g_gate_up.cpu().numpy()
    rows, cols = host.shape[1], host.shape[2]
    mx_bytes = rows * cols * 3 + rows * cols // 32             # per expert, swizzled = linear here
    nv_bytes = rows * cols * 2 + rows * cols // 2 + rows * cols // 16 + 4
    t0 = time.perf_counter()
    for i in range(n_experts):
        oracle.quantize(oracle.MXFP8, oracle.SWIZZLED, host[i])
    dt = time.perf_counter() - t0
    nb = n_experts * mx_bytes
    out = {"value": round(nb / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{n_experts} gate_up experts bf16 [{rows},{cols}] of layer 0, MXFP8 with "
                     f"swizzled scales ({nb} algorithmic bytes, {dt:.1f} s, one thread)",
           "cpu_model": cpu_model(), "nproc": os.cpu_count()}
    n_nv = min(16, n_all)
    t0 = time.perf_counter()
    for i in range(n_nv):
        oracle.quantize(oracle.NVFP4, oracle.SWIZZLED, host[i], g=float(g[i]))
    dt = time.perf_counter() - t0
    out["nvfp4"] = {"value": round(n_nv * nv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                    "sample": f"{n_nv} gate_up experts, NVFP4 swizzled, per-expert g "
                              f"({n_nv * nv_bytes} algorithmic bytes, {dt:.1f} s)"}
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    n_threads = max(1, min(16, avail))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(n_threads) as pool:
        list(pool.map(lambda i: oracle.quantize(oracle.MXFP8, oracle.SWIZZLED, host[i]),
                      range(n_all)))
    dt = time.perf_counter() - t0
    out["threaded"] = {"value": round(n_all * mx_bytes / dt / 1e9, 4), "unit": "GB/s",
                       "cores": n_threads, "cpus_available": avail, "seconds": round(dt, 2),
                       "sample": f"{n_all} gate_up experts MXFP8 swizzled, one oracle call per "
                                 f"expert on {n_threads} host threads (the CPU share of one GPU "
                                 f"on the GPU box is 16 threads)"}
    return out


if __name__ == "__main__":
    main()
