#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

One step = one pass of the whole path (route -> permute -> FC1+SwiGLU -> FC2 ->
finalize) over one batch of the synthetic workload, inputs already resident in
HBM.  Prints ONE JSON line on stdout (details go to stderr):

  value      whole-job tokens/s of the headline workload (DeepSeek-V3-shaped
             prefill, T=8192, H=7168, 256 routed experts + 1 shared, top-8)
  roofline   the dominant kernel (FC1 grouped GEMM): algorithmic bytes/FLOPs
             per launch / its mean launch duration from HIP events recorded on
             the launch stream, over as many steps again as were timed (the
             timed steps themselves run without the events)
  workloads  every configuration (tiny fp32, Mixtral-shaped bf16, DeepSeek-V3
             decode and prefill, Qwen3-shaped fp8 weights): tokens/s, ms per
             step, FC1 and FC2 rooflines, the grouped-GEMM summary and a
             cpu_baseline of its own
  fp8_activations  the fp8 x fp8 path (quantise x in 1x128 blocks, fp8 MFMA
             grouped GEMMs, h quantised in FC1's epilogue) on the two
             DeepSeek-V3 shapes with fp8 e4m3 weights; rooflines use the fp8 peak
  routing    moe_route alone for each of the seven routing methods at the
             prefill and decode T, E and k, against its HBM roofline
  cpu_baseline  the CPU oracle timed on a bounded token sample of the headline
             workload on this host's cores (a reported baseline, not a target)
  calibration  attainable peaks measured in the same run: an HBM read stream
             (the repository's own kernel, non-temporal 16-byte loads over
             4 GiB), a 1 GiB device copy, and 8192^3 bf16 / fp8 GEMMs of
             torch/hipBLASLt on random data; each roofline also reports its
             fraction of these

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads ...]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"hbm": 8000.0, "bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}  # GB/s, TFLOP/s
DOMINANT = "fc1"
# sources of the grouped GEMM kernels (the tile engine's helpers live in dma.h)
KERNEL_SOURCES = [os.path.join(ROOT, "mixture_experts_layer_07_amd", "csrc", f)
                  for f in ("ffn.hip", "dma.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha(text=None):
    """Hash of the GEMM sources with comments and whitespace removed, so that the
    traffic summaries stay valid across comment-only edits."""
    import re
    if text is None:
        text = ""
        for p in KERNEL_SOURCES:
            with open(p) as f:
                text += f.read() + "\n"
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def fc_work(w, touched_groups, which, fp8_act=False):
    """Algorithmic FLOPs and HBM bytes of one FC1 or FC2 launch.

    FC1: 2*R*H*(2I) FLOPs; reads every touched group's w13 (2I*H weights, +
    fp8 scales), each token's activation row once, writes h (R*I).
    FC2: 2*R*I*H FLOPs; reads touched w2 (H*I) and h, writes fc2_out (R*H).
    With fp8 activations x and h are e4m3 codes plus one fp32 scale per 128
    values; fc2_out stays bf16.
    """
    wsz = {"f32": 4, "bf16": 2, "fp8": 1}[w.wdt]
    asz = 4 if w.act == "f32" else 2
    qsz = 1 + 4.0 / 128 if fp8_act else asz   # x and h
    R, H, I, T = w.R, w.H, w.I, w.T
    sc = 4.0 / (128 * 128) if w.wdt == "fp8" else 0.0
    if which == "fc1":
        flops = 2.0 * R * H * 2 * I
        nbytes = touched_groups * 2 * I * H * (wsz + sc) + T * H * qsz + R * I * qsz
    else:
        flops = 2.0 * R * I * H
        nbytes = touched_groups * H * I * (wsz + sc) + R * I * qsz + R * H * asz
    return flops, nbytes


def fc_min_bytes(w, touched_groups, which, fp8_act=False):
    """The method's minimum traffic attributed to one GEMM: the touched groups'
    weights plus x read once (FC1) or y written once (FC2); h and fc2_out,
    which this two-kernel design also moves, are not counted."""
    wsz = {"f32": 4, "bf16": 2, "fp8": 1}[w.wdt]
    asz = 4 if w.act == "f32" else 2
    sc = 4.0 / (128 * 128) if w.wdt == "fp8" else 0.0
    if which == "fc1":
        qsz = 1 + 4.0 / 128 if fp8_act else asz
        return touched_groups * 2 * w.I * w.H * (wsz + sc) + w.T * w.H * qsz
    return touched_groups * w.H * w.I * (wsz + sc) + w.T * w.H * asz


def mfma_peak(w, fp8_act=False):
    return PEAK["fp8" if fp8_act else ("f32" if w.act == "f32" else "bf16")]


def roofline(w, touched, ms_per_step, which=DOMINANT, traffic=None, launches=None, fp8_act=False):
    """Roofline of one grouped GEMM per step.  A grouped GEMM is issued as one
    launch per row class of groups (tile shape); its time per step is the sum
    of those launches, and the algorithmic work is that of the whole GEMM."""
    flops, nbytes = fc_work(w, touched, which, fp8_act)
    peak_f = mfma_peak(w, fp8_act)
    t_f = flops / (peak_f * 1e12)
    t_b = nbytes / (PEAK["hbm"] * 1e9)
    s = ms_per_step * 1e-3
    if t_f >= t_b:
        ach, peak, unit, bound = flops / s / 1e12, peak_f, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = nbytes / s / 1e9, PEAK["hbm"], "GB/s", "hbm"
    nmin = fc_min_bytes(w, touched, which, fp8_act)
    return {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": traffic,
            "kernel": f"grouped GEMM {which.upper()} (row-class launches per step: {launches})",
            "ms_per_step": round(ms_per_step, 4),
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "mfma_frac": round(flops / s / 1e12 / peak_f, 4),
            "hbm_frac": round(nbytes / s / 1e9 / PEAK["hbm"], 4),
            "algorithmic_bytes_min": nmin,
            "hbm_frac_min": round(nmin / s / 1e9 / PEAK["hbm"], 4),
            "bytes_note": ("algorithmic_bytes: touched weights + the GEMM's activation input "
                           "(x or h) + its output (h or fc2_out); algorithmic_bytes_min: touched "
                           "weights + x (FC1) or y (FC2) only, the method's minimum")}


def fused_summary(w, touched, res, two_call_kernels, fp8_act=False):
    """The fused FC1+FC2 kernel (h kept on chip) on the same inputs: its time
    per step beside FC1 + FC2 of the two-call path, and its roofline.  Its
    algorithmic bytes are those of both GEMMs minus the h round trip."""
    f1, b1 = fc_work(w, touched, "fc1", fp8_act)
    f2, b2 = fc_work(w, touched, "fc2", fp8_act)
    qsz = 1 + 4.0 / 128 if fp8_act else 2
    flops, nbytes = f1 + f2, b1 + b2 - 2 * w.R * w.I * qsz
    ms = res["per_kernel"]["ffn_fused"]
    s = ms * 1e-3
    peak_f = mfma_peak(w, fp8_act)
    if flops / (peak_f * 1e12) >= nbytes / (PEAK["hbm"] * 1e9):
        ach, peak, unit, bound = flops / s / 1e12, peak_f, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = nbytes / s / 1e9, PEAK["hbm"], "GB/s", "hbm"
    two = two_call_kernels["fc1"] + two_call_kernels["fc2"]
    return {"kernel": "fused FC1+SwiGLU+FC2, h in LDS (one launch per step)",
            "layer_ms_per_step": round(res["ms"], 4), "ffn_ms_per_step": round(ms, 4),
            "two_call_ffn_ms_per_step": round(two, 4), "ffn_speedup_vs_two_call": round(two / ms, 3),
            "split": res["split"],
            "roofline": {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                         "frac": round(ach / peak, 4), "traffic": None,
                         "algorithmic_bytes": nbytes, "algorithmic_flops": flops}}


def grouped_gemm_summary(w, touched, per_kernel, fp8_act=False):
    """FC1 + FC2 together: the layer's expert-FFN FLOPs (real rows, not padded
    tiles) and algorithmic bytes over the two GEMMs' time per step."""
    f1, b1 = fc_work(w, touched, "fc1", fp8_act)
    f2, b2 = fc_work(w, touched, "fc2", fp8_act)
    ms = per_kernel["fc1"] + per_kernel["fc2"]
    s = ms * 1e-3
    peak_f = mfma_peak(w, fp8_act)
    routed = (f1 + f2) * w.P / w.R  # FLOPs of the routed rows only (shared rows excluded)
    return {"ms_per_step": round(ms, 4), "algorithmic_flops": f1 + f2,
            "algorithmic_bytes": b1 + b2, "tflops": round((f1 + f2) / s / 1e12, 2),
            "routed_only_tflops": round(routed / s / 1e12, 2),
            "gbps": round((b1 + b2) / s / 1e9, 1),
            "mfma_frac": round((f1 + f2) / s / 1e12 / peak_f, 4),
            "hbm_frac": round((b1 + b2) / s / 1e9 / PEAK["hbm"], 4)}


def load_traffic(workload, which="fc1"):
    """HBM bytes per step of one grouped GEMM (all its row-class launches) from
    the committed rocprofv3 counter summary, or None when the summary is
    missing or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{which}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != kernel_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def calibrate(device, reps=5):
    """Measured attainable peaks on this GPU: HBM GB/s of a 1 GiB copy (read +
    write), bf16 and fp8 dense GEMM TFLOP/s of the vendor library at 8192^3 on
    N(0,1) data (fp8 through torch._scaled_mm with unit scales; None when the
    build has no fp8 GEMM)."""
    import torch
    out = {}
    src = torch.empty(1 << 30, dtype=torch.uint8, device=device).random_()
    dst = torch.empty_like(src)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)

    out["hbm_copy_gbps"] = round(2 * src.numel() / best(lambda: dst.copy_(src)) / 1e9, 1)
    del src, dst
    out["hbm_read_gbps"] = hbm_read_stream(device, best)
    n = 8192
    a = torch.randn(n, n, device=device, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=device, dtype=torch.bfloat16)
    out["bf16_gemm_tflops"] = round(2.0 * n ** 3 / best(lambda: torch.matmul(a, b)) / 1e12, 1)
    try:
        a8 = a.to(torch.float8_e4m3fn)
        b8 = b.t().contiguous().to(torch.float8_e4m3fn).t()
        one = torch.ones((), device=device, dtype=torch.float32)
        out["fp8_gemm_tflops"] = round(2.0 * n ** 3 / best(
            lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)) / 1e12, 1)
    except Exception as e:  # noqa: BLE001 - report what the build lacks
        out["fp8_gemm_tflops"] = None
        log(f"[bench] fp8 calibration GEMM unavailable: {type(e).__name__}: {e}")
    del a, b
    torch.cuda.empty_cache()
    out["method"] = ("best of 5: HBM read stream of 4 GiB (libmoe_calib: non-temporal 16-byte "
                     "loads, 1-4 workgroups of 1024 threads per CU, best), torch copy_ of 1 GiB "
                     "(2 GiB moved), torch.matmul bf16 8192^3, torch._scaled_mm e4m3 8192^3 "
                     "(unit scales), N(0,1) operands")
    return out


def hbm_read_stream(device, best):
    """GB/s of reading a 4 GiB device buffer once (the repository's stream
    kernel, libmoe_calib.so), best over 1, 2 and 4 workgroups per CU."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "mixture_experts_layer_07_amd", "libmoe_calib.so")
    L = ctypes.CDLL(path)
    L.moe_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p]
    L.moe_calib_stream_read.restype = ctypes.c_int
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device).random_()
    ncu = torch.cuda.get_device_properties(device).multi_processor_count
    out = torch.empty(4 * ncu * 1024, dtype=torch.int32, device=device)
    stream = torch.cuda.current_stream(device).cuda_stream
    rate = 0.0
    for per_cu in (1, 2, 4):
        def run(g=per_cu * ncu):
            rc = L.moe_calib_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), g, stream)
            if rc != 0:
                raise RuntimeError(f"moe_calib_stream_read failed: hipError {rc}")
        rate = max(rate, nbytes / best(run) / 1e9)
    del buf, out
    return round(rate, 1)


def add_calibrated(rl, cal, fp8_act=False):
    """Fraction of the measured peak next to the published one."""
    if cal is None:
        return rl
    if rl["bound"] == "hbm":
        peak = cal.get("hbm_read_gbps")
    else:
        peak = cal.get("fp8_gemm_tflops" if fp8_act else "bf16_gemm_tflops")
    rl["calibrated_peak"] = peak
    rl["frac_of_calibrated"] = round(rl["achieved"] / peak, 4) if peak else None
    return rl


def calibration_copy(mib, device):
    """A plain streaming kernel of known traffic (reads and writes `mib` MiB once),
    run before the workload so rocprofv3 FETCH_SIZE / WRITE_SIZE can be scaled."""
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def summarize_traffic(fetch_dir, write_dir, workload, copy_mib, commands):
    """Write profiles/fc1_<workload>_traffic.json and fc2_<workload>_traffic.json
    from two rocprofv3 --pmc runs of `bench.py --workloads <workload>
    --calibrate-copy-mib N ...` (FETCH_SIZE, then WRITE_SIZE; counter values are
    KiB per dispatch).  A GEMM's HBM bytes per step are its counters summed over
    its row-class launches, divided by the number of layer calls, each scaled by
    true/counted bytes of the copy."""
    import csv

    def rows_of(d, counter):
        path = os.path.join(d, "run_counter_collection.csv")
        if not os.path.exists(path):
            for root, _, files in os.walk(d):
                for f in files:
                    if f.endswith("counter_collection.csv"):
                        path = os.path.join(root, f)
        return path, [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]

    def is_gemm(name, mode):
        return (f"dma_gemm_kernel<{mode}," in name
                or ("grouped_gemm_kernel<" in name and f", {mode}, moe::" in name))

    def load(d, counter, mode):
        path, rows = rows_of(d, counter)
        calib = [float(r["Counter_Value"]) for r in rows if "bitwise_not" in r["Kernel_Name"]]
        vals = [float(r["Counter_Value"]) for r in rows if is_gemm(r["Kernel_Name"], mode)]
        calls = sum(1 for r in rows if "route_kernel" in r["Kernel_Name"])
        if not calib or not vals or not calls:
            raise SystemExit(f"{path}: calibration copy, GEMM or route dispatches missing")
        scale = (copy_mib * 1024.0) / max(calib)
        return sum(vals) * 1024.0 * scale / calls, scale, calls

    for mode, which in ((0, "fc1"), (1, "fc2")):
        fetch, sf, n1 = load(fetch_dir, "FETCH_SIZE", mode)
        write, sw, n2 = load(write_dir, "WRITE_SIZE", mode)
        out = {"workload": workload,
               "kernel": f"grouped GEMM {which.upper()} (all row-class launches of a step)",
               "kernel_source_sha": kernel_sha(), "fetch_bytes_per_launch": fetch,
               "write_bytes_per_launch": write, "hbm_bytes_per_launch": fetch + write,
               "copy_calibration": {"mib": copy_mib, "fetch_scale": sf, "write_scale": sw},
               "layer_calls_seen": [n1, n2], "commands": commands}
        path = os.path.join(ROOT, "profiles", f"{which}_{workload}_traffic.json")
        with open(path, "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out, indent=1))


LIB_KERNELS = {"route_kernel", "permute_one_kernel", "permute_count_kernel", "permute_scan_kernel",
               "permute_scatter_kernel",
               "finalize_kernel", "quantize_fp8_kernel", "grouped_gemm_kernel", "fused_ffn_kernel"}


def class_summary(pmc_dirs, trace_dir):
    """Markdown table per kernel (grouped-GEMM row classes separately) from
    rocprofv3 --pmc runs (GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_BUSY_CU_CYCLES, SQ_WAVE_CYCLES, SQ_WAIT_INST_ANY, TCC_HIT_sum,
    TCC_MISS_sum; per dispatch) and a --kernel-trace run of the same command
    (median duration): MFMA-busy fraction of the CU-busy cycles, the fraction
    of wave cycles spent waiting on a counter, the L2 hit rate and the mean
    clock (GPU-busy cycles per XCD over the kernel's duration)."""
    import csv
    import glob
    import re
    from collections import defaultdict

    def cls(n):
        m = re.search(r"dma_gemm_kernel<(\d), moe::\(anonymous namespace\)::DmaCfg<(\d+), (\d+), (\d+), "
                      r"(\d+), (\d+), (\d+)", n)
        if m:
            kind = " fp8 x fp8" if "true, true" in n else (" fp8 weights" if "true, false" in n else "")
            return (f"FC{int(m.group(1)) + 1} {m.group(2)}x{m.group(3)} tiles, "
                    f"{int(m.group(4)) * int(m.group(5))} waves, group-M {m.group(6)}, "
                    f"ring {m.group(7)}{kind}")
        m = re.search(r"(\w+_kernel)(<[^(]*>)?", n)
        return m.group(0) if m else n[:40]
    agg, disp, dur = defaultdict(lambda: defaultdict(float)), defaultdict(set), defaultdict(list)
    for d in pmc_dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                c = cls(r["Kernel_Name"])
                agg[c][r["Counter_Name"]] += float(r["Counter_Value"])
                disp[(c, r["Counter_Name"])].add(r["Dispatch_Id"])
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            dur[cls(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    n_xcd = 8
    lines = ["| kernel | median us | dispatches | MFMA busy / CU busy | waves waiting | L2 hit | clock GHz |",
             "|---|---|---|---|---|---|---|"]
    for c in sorted(dur, key=lambda c: -sorted(dur[c])[len(dur[c]) // 2]):
        ds = sorted(dur[c])
        med = ds[len(ds) // 2]
        if med < 10 or not (c.startswith("FC") or c.split("<")[0] in LIB_KERNELS):
            continue
        a = agg.get(c, {})
        per = lambda k: a.get(k, 0.0) / max(1, len(disp.get((c, k), ())))  # noqa: E731
        busy = a.get("SQ_BUSY_CU_CYCLES", 0.0)
        mf = a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4 * busy) if busy else float("nan")
        wt = a.get("SQ_WAIT_INST_ANY", 0.0) / a["SQ_WAVE_CYCLES"] if a.get("SQ_WAVE_CYCLES") else float("nan")
        h, m = a.get("TCC_HIT_sum", 0.0), a.get("TCC_MISS_sum", 0.0)
        l2 = h / (h + m) if h + m else float("nan")
        clk = per("GRBM_GUI_ACTIVE") / n_xcd / (med * 1e3) if per("GRBM_GUI_ACTIVE") else float("nan")
        lines.append(f"| {c} | {med:.1f} | {len(ds)} | {mf:.3f} | {wt:.3f} | {l2:.3f} | {clk:.2f} |")
    print("\n".join(lines))


def time_layer(layer, inp, steps, warmup):
    """ms per step of layer(inp) and its per-kernel ms per step (HIP-event hooks
    on, in a second pass of as many steps)."""
    import torch
    import mixture_experts_layer_07_amd as moe

    def step():
        return layer(inp["x"], inp["logits"], inp["w13"], inp["w2"], inp["bias"],
                     inp["w13_scale"], inp["w2_scale"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    moe.timing_enable(True)
    moe.kernel_times(reset=True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kt = moe.kernel_times(reset=True)
    moe.timing_enable(False)
    return ms, {k: round(v[0] / steps, 4) for k, v in kt.items()}


ROUTE_METHODS = [(0, "default"), (1, "renormalize"), (2, "deepseek_v3"), (3, "llama4"),
                 (4, "renormalize_naive"), (5, "minimax2"), (6, "sigmoid_renorm")]


def routing_summary(names, device, reps=100):
    """moe_route alone, every method, at each named workload's T, E and k
    (DeepSeek-V3's groups and scaling for method 2, a correction bias for 2 and
    5), against the HBM roofline of one launch: logits (and bias) read once,
    ids and scales written once.  Logits are N(0, 1) drawn directly."""
    import torch
    import mixture_experts_layer_07_amd as moe
    from mixture_experts_layer_07_amd import workloads as wl

    out = {"kernel": "route_kernel (one launch per call)", "peak_gbps": 8000.0,
           "logits": "seeded N(0, 1), drawn directly", "reps": reps}
    for name in names:
        w = wl.get(name)
        logits = wl.make_logits_direct(w).to(device)
        bias = wl.make_bias(w.with_(bias=True)).to(device)
        ids = torch.empty((w.T, w.k), dtype=torch.int32, device=device)
        sc = torch.empty((w.T, w.k), dtype=torch.float32, device=device)
        per = {}
        for m, mname in ROUTE_METHODS:
            grouped = m == 2
            b = bias if m in (2, 5) else None

            def call(m=m, b=b, grouped=grouped):
                moe.route(logits, w.k, m, w.n_group if grouped else 1,
                          w.topk_group if grouped else 1, b, w.scaling if grouped else 1.0,
                          out=(ids, sc))

            for _ in range(5):
                call()
            torch.cuda.synchronize()
            moe.timing_enable(True)
            moe.kernel_times(reset=True)
            for _ in range(reps):
                call()
            torch.cuda.synchronize()
            ms, n = moe.kernel_times(reset=True)["route"]
            moe.timing_enable(False)
            us = ms * 1e3 / n
            nbytes = w.T * w.E * 4 + (w.E * 4 if b is not None else 0) + w.T * w.k * 8
            per[mname] = {"us": round(us, 2), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "hbm_frac": round(nbytes / (us * 1e-6) / 8e12, 4)}
        out[name] = {"T": w.T, "E": w.E, "k": w.k, "bytes_per_call": w.T * w.E * 4 + w.T * w.k * 8,
                     "methods": per}
        log(f"[bench] routing {name}: " + ", ".join(f"{k} {v['us']} us" for k, v in per.items()))
    return out


def run_workload(name, steps, warmup, device, fp8_act=False, fused=False):
    import torch
    import mixture_experts_layer_07_amd as moe
    from mixture_experts_layer_07_amd import workloads as wl

    w = wl.get(name)
    t0 = time.time()
    inp = wl.make_inputs(w, 0, device)
    layer = moe.layer_for_workload(w, device, fp8_act=fp8_act)
    torch.cuda.synchronize()
    if fp8_act:
        name = name + " (fp8 activations)"
    log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s")

    def step():
        return layer(inp["x"], inp["logits"], inp["w13"], inp["w2"], inp["bias"],
                     inp["w13_scale"], inp["w2_scale"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps run without per-launch events (they cost ~0.1 ms a step);
    # the per-kernel breakdown comes from the same number of steps run after
    # them with the library's HIP-event hooks on
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    moe.timing_enable(True)
    moe.kernel_times(reset=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    kt = moe.kernel_times(reset=True)
    moe.timing_enable(False)
    step_ms = sorted(a.elapsed_time(b) for a, b in ev)
    cnt = torch.bincount(layer.ids.flatten().long(), minlength=w.E).cpu()
    touched = int((cnt > 0).sum()) + w.n_shared
    ms = elapsed * 1e3 / steps
    # per step: a grouped GEMM is one launch per row class of groups (tile shape)
    per_kernel = {k: round(v[0] / steps, 4) for k, v in kt.items()}
    launches = {k: v[1] // steps for k, v in kt.items()}
    log(f"[bench] {name}: {ms:.3f} ms/step, per-kernel ms per step {per_kernel}, launches per step {launches}")
    log(f"[bench] {name}: rows per expert min {int(cnt.min())} median "
        f"{int(cnt.median())} max {int(cnt.max())}, empty experts {int((cnt == 0).sum())}")
    fres = None
    if fused and w.act == "bf16" and w.I <= moe.binding.FUSED_MAX_I:
        lf = moe.layer_for_workload(w, device, fp8_act=fp8_act, fused=True)
        fms, fk = time_layer(lf, inp, steps, warmup)
        fres = dict(ms=fms, per_kernel=fk, split="automatic")
        log(f"[bench] {name} fused FFN: {fms:.3f} ms/step, per-kernel ms per step {fk}")
        del lf
    return dict(w=w, inp=inp, layer=layer, ms=ms, per_kernel=per_kernel, touched=touched, fused=fres,
                counts=cnt, launches=launches,
                step_stats={"median_ms": round(step_ms[len(step_ms) // 2], 4),
                            "min_ms": round(step_ms[0], 4),
                            "note": "per-step HIP events in the pass with kernel hooks on"},
                histogram={"rows_per_expert_min": int(cnt.min()),
                           "rows_per_expert_median": int(cnt.median()),
                           "rows_per_expert_max": int(cnt.max()),
                           "empty_experts": int((cnt == 0).sum())})


def cpu_baseline(res, seconds):
    """Time the CPU oracle on a bounded token sample of the same workload."""
    import numpy as np
    import oracle

    w, inp, layer = res["w"], res["inp"], res["layer"]
    host = lambda t: None if t is None else t.detach().cpu()  # noqa: E731
    x, logits, bias = host(inp["x"]), host(inp["logits"]), host(inp["bias"])
    t0 = time.perf_counter()
    ids, sc, _ = oracle.route(logits, w.k, w.method, w.n_group, w.topk_group, bias, w.scaling,
                              bool(w.flags & 1))
    oracle.permute(ids, w.E, w.n_shared)
    t_route = time.perf_counter() - t0
    W = oracle.Weights(host(inp["w13"]), host(inp["w2"]), w.wdt, host(inp["w13_scale"]),
                       host(inp["w2_scale"]))
    threads = oracle.num_threads()
    rng = np.random.default_rng(0)
    order = rng.permutation(w.T).astype(np.int32)
    done, t_ffn, batch = 0, 0.0, threads
    while done < w.T and t_ffn < seconds:
        toks = order[done:done + batch]
        t0 = time.perf_counter()
        oracle.layer_tokens(W, x, w.act, w.T, w.k, w.E, w.n_shared, ids, sc, toks)
        t_ffn += time.perf_counter() - t0
        done += len(toks)
        batch = threads * 2
    est = t_route + t_ffn * w.T / done
    return {"value": round(w.T / est, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{w.name}: routing + permute of all {w.T} tokens ({t_route:.2f}s), "
                       f"expert FFN + weighted sum of {done} random tokens ({t_ffn:.1f}s), "
                       f"scaled to {w.T} tokens; fp64, OpenMP over tokens")}


WORKLOAD_ORDER = ["dsv3_prefill", "dsv3_decode", "tiny_fp32", "mixtral_bf16", "qwen3_fp8"]


def describe(w):
    return (f"{w.name}: T={w.T} H={w.H} E={w.E}+{w.n_shared} shared I={w.I} top-{w.k}, "
            f"route method {w.method}, {w.act} activations, {w.wdt} weights")


def workload_summary(res, cal, fp8_act=False, traffic=True):
    """tokens/s, ms per step, FC1 / FC2 rooflines and the grouped-GEMM summary of
    one run_workload result."""
    w = res["w"]
    pk, la = res["per_kernel"], res["launches"]
    tr = (lambda fc: load_traffic(w.name, fc)) if traffic and not fp8_act else (lambda fc: None)
    out = {"workload": describe(w),
           "value": round(w.T / (res["ms"] * 1e-3), 1), "unit": "tokens/s",
           "ms_per_step": round(res["ms"], 4),
           "roofline": add_calibrated(roofline(w, res["touched"], pk["fc1"], "fc1", tr("fc1"),
                                               la["fc1"], fp8_act), cal, fp8_act),
           "roofline_fc2": add_calibrated(roofline(w, res["touched"], pk["fc2"], "fc2", tr("fc2"),
                                                   la["fc2"], fp8_act), cal, fp8_act),
           "grouped_gemm": grouped_gemm_summary(w, res["touched"], pk, fp8_act),
           "per_kernel_ms": pk,
           "step_stats": res["step_stats"],
           "rows_per_expert": res["histogram"]}
    if res["fused"]:
        out["fused_ffn"] = fused_summary(w, res["touched"], res["fused"], pk, fp8_act)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill", help="the headline workload")
    ap.add_argument("--workloads", nargs="*", default=None,
                    help="workloads to run (default: all five; the headline is always run)")
    ap.add_argument("--fp8act-workloads", nargs="*", default=["dsv3_prefill_fp8", "dsv3_decode_fp8"],
                    help="workloads also run on the fp8-activation path (none: skip)")
    ap.add_argument("--fused", action="store_true",
                    help="also time the fused FC1+FC2 kernel beside each workload")
    ap.add_argument("--no-routing", action="store_true",
                    help="skip timing moe_route alone for every routing method")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="CPU oracle time budget per workload (token sample)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the measured-peak calibration (streams and library GEMMs)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run a plain copy of this many MiB first (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 --pmc runs into profiles/ and exit")
    ap.add_argument("--traffic-command", action="append", default=[],
                    help="command lines recorded in the traffic summary")
    ap.add_argument("--class-summary", nargs="+", metavar="DIR",
                    help="print per-kernel counter table: rocprofv3 --pmc output dirs, then the "
                         "--kernel-trace dir of the same command (last argument), and exit")
    args = ap.parse_args()
    if args.class_summary:
        class_summary(args.class_summary[:-1], args.class_summary[-1])
        return
    if args.traffic_from:
        summarize_traffic(args.traffic_from[0], args.traffic_from[1], args.workload,
                          args.calibrate_copy_mib, args.traffic_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the layer keeps all experts on one device "
              f"and has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy_mib:
        calibration_copy(args.calibrate_copy_mib, dev)
    cal = None if args.no_calibration else calibrate(dev)
    if cal:
        log(f"[bench] calibration {cal}")
    names = WORKLOAD_ORDER if args.workloads is None else list(args.workloads)
    names = [args.workload] + [n for n in names if n != args.workload]
    summaries = {}
    head = None
    for name in names:
        res = run_workload(name, args.steps, args.warmup, dev, fused=args.fused)
        summaries[name] = workload_summary(res, cal)
        if not args.no_cpu_baseline:
            summaries[name]["cpu_baseline"] = cpu_baseline(res, args.cpu_seconds)
            log(f"[bench] {name} cpu baseline {summaries[name]['cpu_baseline']}")
        if name == args.workload:
            head = res["w"]
        # the freed blocks stay in torch's cache for the next workload's
        # buffers: returning them to the driver and allocating again placed
        # the DeepSeek-V3 decode weights so that the layer ran 3% slower
        # (3.63 vs 3.50 ms) than in a fresh process or on reused blocks
        del res
    hs = summaries[args.workload]
    out = {
        "metric": "MoE layer tokens/s + grouped-GEMM %MFMA / %HBM peak, DSV3 shapes T=512/8192",
        "value": hs["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": hs["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if head.act == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": describe(head), "global_batch": head.T,
                   "parallelism": "single GPU, all experts local"},
        "roofline": hs["roofline"],
        "roofline_fc2": hs["roofline_fc2"],
        "grouped_gemm": hs["grouped_gemm"],
        "per_kernel_ms": hs["per_kernel_ms"],
        "step_stats": hs["step_stats"],
        "rows_per_expert": hs["rows_per_expert"],
        "calibration": cal,
    }
    if "cpu_baseline" in hs:
        out["cpu_baseline"] = hs["cpu_baseline"]
    if "fused_ffn" in hs:
        out["fused_ffn"] = hs["fused_ffn"]
    out["workloads"] = summaries
    if args.fp8act_workloads:
        out["fp8_activations"] = {}
        for name in args.fp8act_workloads:
            r = run_workload(name, args.steps, args.warmup, dev, fp8_act=True, fused=args.fused)
            o = workload_summary(r, cal, fp8_act=True)
            o["workload"] = (f"{r['w'].name}: T={r['w'].T} H={r['w'].H} E={r['w'].E}+{r['w'].n_shared} "
                             f"shared I={r['w'].I} top-{r['w'].k}; x and h quantised to e4m3 in 1x128 "
                             f"blocks, fp8 weights (128x128 block scales), fp8 MFMA, bf16 output")
            o["dtype"] = "fp8 e4m3 x e4m3, fp32 accumulate"
            out["fp8_activations"][name] = o
            del r
    if not args.no_routing:
        out["routing"] = routing_summary(["dsv3_prefill", "dsv3_decode"], dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
