"""Benchmark of the W4A4 MXFP4 linear layer (dynamic activation quantization + block-scaled GEMM
+ bias, BF16 output) at the Wan2.2-A14B attention-projection shape M=75600, K=N=5120.

One step = one call of the library's ``mx_linear``: the activation quantizer kernel followed by
the GEMM kernel, on inputs already resident in HBM.  ``value`` is whole-step throughput in
TFLOP/s (2*M*N*K per step).  The roofline object describes the dominant kernel (the GEMM),
timed alone with HIP events on the stream it is launched on; the quantizer is timed the same
way and reported beside it.  The CPU baseline times the oracle on a bounded row sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Other workloads (``--workload``) bench the variant paths: the FFN pair, W4A8 SVDQuant, the MXFP8
W8A8 reference layer, NVFP4, the fused LayerNorm + quantizer and microscaled attention.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 MXFP4 linear TFLOPS (quant+GEMM) at Wan-A14B shapes; % MXFP4 MFMA peak"
PEAK_TFLOPS = {"mxfp4": 10100.0, "mxfp8": 5000.0, "bf16": 2500.0}
HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "fp4_block_scaled_amd", "csrc")


def kernel_sources(kernel: str):
    """The source files a kernel is built from (its own file and the shared headers)."""
    own = ("mx_gemm.hip" if "gemm_" in kernel else
           "mx_attn.hip" if ("attn_" in kernel or "quant_vt" in kernel) else "mx_quant.hip")
    return [os.path.join(CSRC, f) for f in (own, "mx_common.h", "mx_internal.h")]


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed: edits to comments or layout
    leave the hash alone (string literals in these files hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in kernel_sources(kernel):
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the kernel whose name contains `kernel`, from the committed
    rocprofv3 counter runs, if they were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    hits = [(name, e) for name, e in t.get(workload, {}).items() if kernel in name]
    if len(hits) != 1 or hits[0][1].get("source_hash") != kernel_source_hash(hits[0][0]):
        return None
    return hits[0][1].get("bytes_per_launch")


def cpu_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def time_events(fn, iters: int, torch, warmup: int = 3):
    """Average milliseconds of fn() over iters launches, HIP events on the current stream, after
    `warmup` untimed launches."""
    s = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(s)
    for _ in range(iters):
        fn()
    end.record(s)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def launch_stats(fn, iters: int, torch, warmup: int = 3):
    """Per-launch milliseconds of fn(): one HIP event pair around each of `iters` launches on the
    current stream (after `warmup` untimed ones); median, min, mean and max."""
    import statistics
    s = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(s)
        fn()
        e1.record(s)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    return {"median": statistics.median(ms), "min": min(ms), "mean": sum(ms) / len(ms), "max": max(ms),
            "launches": iters}


GEMM_KERNEL = "gemm_mx_ring_kernel<256,256,ping-pong> (MXFP4 x MXFP4, tiled operands, bias, BF16 out)"


def sample_sclk(fn, launches: int, torch):
    """Shader clock (MHz) that rocm-smi reports while `launches` calls of fn run back to back (the
    calls are queued first, the reading is taken while they execute); None if it cannot be read."""
    import json
    import re
    import shutil
    import subprocess
    # under a profiler (a preloaded rocprofiler library) the rocm-smi child would inherit the
    # preload and initialise the GPU before its interpreter starts: skip the reading there
    if not shutil.which("rocm-smi") or "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    torch.cuda.synchronize()
    for _ in range(launches):
        fn()
    time.sleep(0.5)
    sclk = None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        for card in json.loads(r.stdout).values():
            for key, val in (card.items() if isinstance(card, dict) else ()):
                m = re.search(r"(\d+)\s*mhz", str(val), re.IGNORECASE)
                if sclk is None and key.lower().startswith("sclk clock speed") and m:
                    sclk = float(m.group(1))
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    torch.cuda.synchronize()
    return sclk


def cpu_baseline_mx(wl, a_bits, w_codes, w_scales, b_bits, rows: int):
    """The oracle (as it stands) on a sample of rows: quantize + dequantize + fp64 GEMM."""
    import numpy as np
    import oracle as O
    idx = np.concatenate([np.arange(rows // 2), np.arange(wl.M - rows // 2, wl.M)])
    sample = np.ascontiguousarray(a_bits[idx])
    wdeq = O.dequantize_mx(w_codes, w_scales, wl.K)     # weight preparation: not timed
    bias = O.f16_values(b_bits) if b_bits is not None else None
    t0 = time.perf_counter()
    ac, as_ = O.quantize_mx_bf16(sample, O.E2M1)
    adeq = O.dequantize_mx(ac, as_, wl.K, O.E2M1)
    O.gemm(adeq, wdeq, bias)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * wl.K * wl.N
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{rows} rows (first and last {rows // 2}) of the {wl.M}x{wl.K}x{wl.N} linear: "
                     f"oracle MXFP4 quantization + dequantization + fp64 GEMM, {dt:.2f} s; "
                     f"CPU: {cpu_info()}"}
    # the same on one thread (OpenMP of the oracle and the BLAS under numpy), on 1024 rows
    try:
        from threadpoolctl import threadpool_limits
        r1 = min(rows, 1024)
        s1 = np.ascontiguousarray(sample[np.r_[0:r1 // 2, rows - r1 // 2:rows]])
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            ac, as_ = O.quantize_mx_bf16(s1, O.E2M1)
            O.gemm(O.dequantize_mx(ac, as_, wl.K, O.E2M1), wdeq, bias)
            d1 = time.perf_counter() - t0
        res["single_thread"] = {"value": 2.0 * r1 * wl.K * wl.N / d1 / 1e12, "unit": "TFLOP/s",
                                "rows": r1, "seconds": d1}
    except ImportError:
        pass
    # the oracle's quantizer alone on the full activation (all threads), as GB/s of the same
    # algorithmic bytes the GPU quantizer is measured on
    t0 = time.perf_counter()
    O.quantize_mx_bf16(a_bits, O.E2M1)
    dq = time.perf_counter() - t0
    qbytes = wl.M * wl.K * 2 + wl.M * wl.K // 2 + wl.M * wl.K // 32
    res["quantizer"] = {"value": qbytes / dq / 1e9, "unit": "GB/s", "seconds": dq,
                        "sample": f"the full {wl.M}x{wl.K} activation"}
    return res


def smallest_instance_latency(torch, mx, synth, iters: int = 200, warmup: int = 50):
    """The smallest MXFP4 instance (256x512x512, bias, BF16 out): per-launch latency of the whole
    linear (quantizer + GEMM) and of each kernel, in microseconds.  Launch-bound: no roofline
    fraction applies."""
    import numpy as np
    wl = synth.WORKLOADS["mxfp4_256x512x512"]
    to_dev = lambda bits, dt: torch.from_numpy(bits.view(np.int16)).view(dt).cuda()
    a = to_dev(synth.bits16(synth.to_bf16(wl.activation())), torch.bfloat16)
    wq = mx.quantize(to_dev(synth.bits16(synth.to_bf16(wl.weight())), torch.bfloat16), "mxfp4", layout="tiled")
    bias = to_dev(synth.bits16(synth.to_f16(wl.bias())), torch.float16)
    out = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.linear_workspace_bytes(wl.M, wl.K, "mxfp4"), dtype=torch.uint8, device="cuda")
    aq = mx.empty_qmatrix(wl.M, wl.K, "mxfp4", layout="tiled")
    res = {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N}
    linear = lambda: mx.linear(a, wq, bias, out=out, workspace=ws)
    for name, fn in (("linear", linear),
                     ("quantizer", lambda: mx.quantize(a, "mxfp4", out=aq)),
                     ("gemm", lambda: mx.linear_q(aq, wq, bias, out=out))):
        st = launch_stats(fn, iters, torch, warmup)
        res[name + "_us"] = {k: (v * 1e3 if k != "launches" else v) for k, v in st.items()}
    # the same call replayed from a captured HIP graph (the path allocates nothing when out and
    # workspace are given), alone and as 16 calls in one graph
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            linear()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g1, g16 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        linear()
    with torch.cuda.graph(g16):
        for _ in range(16):
            linear()
    st = launch_stats(g1.replay, iters, torch, warmup)
    res["linear_graph_us"] = {k: (v * 1e3 if k != "launches" else v) for k, v in st.items()}
    st = launch_stats(g16.replay, max(1, iters // 16), torch, max(1, warmup // 16))
    res["linear_graph16_us_per_call"] = {k: (v * 1e3 / 16 if k != "launches" else v) for k, v in st.items()}
    return res


def bench_mx_linear(args, torch, mx, synth):
    import numpy as np
    wl = synth.WORKLOADS[args.workload]
    M, K, N = wl.M, wl.K, wl.N
    t0 = time.perf_counter()
    a_bits = synth.bits16(synth.to_bf16(wl.activation()))
    w_bf = synth.to_bf16(wl.weight())
    b = wl.bias()
    b_bits = synth.bits16(synth.to_f16(b)) if b is not None else None
    a = torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).cuda()
    bias = torch.from_numpy(b_bits.view(np.int16)).view(torch.float16).cuda() if b is not None else None
    wq = mx.quantize(w_bf.cuda(), "mxfp4", layout="tiled")  # offline weight preparation
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.linear_workspace_bytes(M, K, "mxfp4"), dtype=torch.uint8, device="cuda")
    aq = mx.empty_qmatrix(M, K, "mxfp4", layout="tiled")  # what mx_linear stages internally
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0

    step = lambda: mx.linear(a, wq, bias, out=out, workspace=ws)
    quant = lambda: mx.quantize(a, "mxfp4", out=aq)
    gemm = lambda: mx.linear_q(aq, wq, bias, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ms_step = time_events(step, args.steps, torch)
    wall_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    quant()
    ms_quant = time_events(quant, args.steps, torch)
    ms_gemm = time_events(gemm, args.steps, torch)
    # per-launch distributions (one event pair per launch, outside the timed region above)
    dist = {"step": launch_stats(step, args.steps, torch, 1), "quantizer": launch_stats(quant, args.steps, torch, 1),
            "gemm": launch_stats(gemm, args.steps, torch, 1)}

    # the shader clock during about 1.5 s of back-to-back GEMMs (the published peak assumes 2.4 GHz)
    sclk = sample_sclk(gemm, max(100, int(1500.0 / ms_gemm)), torch)

    flops = 2.0 * M * N * K
    quant_bytes = M * K * 2 + M * K // 2 + M * K // 32
    gemm_bytes = M * K // 2 + M * K // 32 + N * K // 2 + N * K // 32 + M * N * 2 + (N * 2 if b is not None else 0)
    achieved = flops / (ms_gemm * 1e-3) / 1e12
    traffic = measured_traffic(args.workload, "gemm_mx_ring_kernel<256, 256")
    res = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": M, "K": K, "N": N,
                   "activation": f"N(0,1), {int(round(wl.outlier_frac * K))} outlier channels x{wl.outlier_factor:g}",
                   "weight": f"N(0,{wl.w_sigma}) MXFP4", "bias": "fp16", "output": "bf16"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS["mxfp4"],
                     "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS["mxfp4"],
                     "traffic": traffic,
                     "kernel": GEMM_KERNEL,
                     "algorithmic_flops_per_launch": flops, "ms_per_launch": ms_gemm,
                     "ms_per_launch_median": dist["gemm"]["median"], "ms_per_launch_min": dist["gemm"]["min"],
                     "sclk_mhz_sampled": sclk,
                     # context only: the achieved rate against the peak scaled to that clock
                     "frac_at_sampled_clock": (achieved / (PEAK_TFLOPS["mxfp4"] * sclk / 2400.0)) if sclk else None},
        "kernels": {
            "quantizer": {"ms": ms_quant, "GB/s": quant_bytes / (ms_quant * 1e-3) / 1e9,
                          "frac_hbm": quant_bytes / (ms_quant * 1e-3) / 1e9 / HBM_GBPS,
                          "algorithmic_bytes": quant_bytes,
                          "traffic": measured_traffic(args.workload, "quant_mx_tiled_kernel<0>")},
            "gemm": {"ms": ms_gemm, "TFLOP/s": achieved, "algorithmic_bytes": gemm_bytes},
            "step_frac_of_mxfp4_peak": flops / (ms_step * 1e-3) / 1e12 / PEAK_TFLOPS["mxfp4"],
            "wall_ms_per_step": wall_ms,
            "per_launch_ms": dist,
            "step_tflops_at_median": flops / (dist["step"]["median"] * 1e-3) / 1e12,
        },
        "setup_s": setup_s,
    }
    if wl.name == "wan_a14b_attn_75600x5120x5120":
        res["smallest_instance"] = smallest_instance_latency(torch, mx, synth)
    if not args.no_cpu:
        wrm = mx.relayout(wq)  # the oracle reads the canonical layout
        res["cpu_baseline"] = cpu_baseline_mx(wl, a_bits, wrm.codes.cpu().numpy(),
                                              wrm.scales.cpu().numpy(), b_bits, args.cpu_rows)
    else:
        res["cpu_baseline"] = None
    return res


def bench_variant(args, torch, mx, synth):
    """Variant workloads (not the headline metric): FFN pair, W4A8 SVDQuant, MXFP8 W8A8, NVFP4,
    and the producer-fused quantizer."""
    import numpy as np
    wl = synth.WORKLOADS[args.workload]
    M, K, N = wl.M, wl.K, wl.N
    to_dev = lambda bits, dt: torch.from_numpy(bits.view(np.int16)).view(dt).cuda()
    a = to_dev(synth.bits16(synth.to_bf16(wl.activation())), torch.bfloat16)
    w_dev = to_dev(synth.bits16(synth.to_bf16(wl.weight())), torch.bfloat16)
    b = wl.bias()
    bias = to_dev(synth.bits16(synth.to_f16(b)), torch.float16) if b is not None else None
    kernels = {}
    if wl.N2:  # FFN pair
        wq = mx.quantize(w_dev, "mxfp4", layout="tiled")
        w2q = mx.quantize(to_dev(synth.bits16(synth.to_bf16(wl.weight2())), torch.bfloat16), "mxfp4",
                          layout="tiled")
        b2 = to_dev(synth.bits16(synth.to_f16(wl.bias2())), torch.float16)
        h = mx.empty_qmatrix(M, N, "mxfp4", layout="tiled")  # FFN0 writes H in the GEMM layout
        out = torch.empty((M, wl.N2), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mx.linear_workspace_bytes(M, K, "mxfp4"), dtype=torch.uint8, device="cuda")
        step = lambda: (mx.linear(a, wq, bias, epilogue="bias_gelu_quant_mxfp4_tiled", out=h, workspace=ws),
                        mx.linear_q(h, w2q, b2, out=out))
        flops = 2.0 * M * K * N + 2.0 * M * N * wl.N2
        dtype, peak = "mxfp4", PEAK_TFLOPS["mxfp4"]
        aq = mx.quantize(a, "mxfp4", layout="tiled")
        kernels["ffn0_gemm_gelu_requant_ms"] = time_events(
            lambda: mx.linear_q(aq, wq, bias, epilogue="bias_gelu_quant_mxfp4_tiled", out=h), args.steps, torch)
        kernels["ffn2_gemm_ms"] = time_events(lambda: mx.linear_q(h, w2q, b2, out=out), args.steps, torch)
    elif wl.fmt == "w4a8":
        wq = mx.quantize(w_dev, "mxfp4", layout="tiled")
        down = to_dev(synth.bits16(synth.to_bf16(np.ascontiguousarray(wl.lora_down().T))), torch.bfloat16)
        up = to_dev(synth.bits16(synth.to_bf16(np.ascontiguousarray(wl.lora_up().T))), torch.bfloat16)
        lr = mx.LowRank(down, up)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mx.linear_workspace_bytes(M, K, "mxfp8", wl.rank), dtype=torch.uint8, device="cuda")
        step = lambda: mx.linear(a, wq, bias, act_fmt="mxfp8", lowrank=lr, out=out, workspace=ws)
        flops = 2.0 * M * N * K
        dtype, peak = "mxfp8xmxfp4", PEAK_TFLOPS["mxfp8"]
        aq = mx.quantize(a, "mxfp8", layout="tiled")
        kernels["gemm_no_lowrank_ms"] = time_events(lambda: mx.linear_q(aq, wq, bias, out=out), args.steps, torch)
        kernels["quant_mxfp8_ms"] = time_events(lambda: mx.quantize(a, "mxfp8", out=aq), args.steps, torch)
    elif wl.fmt == "w8a8":
        wq = mx.quantize(w_dev, "mxfp8", layout="tiled")
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mx.linear_workspace_bytes(M, K, "mxfp8"), dtype=torch.uint8, device="cuda")
        step = lambda: mx.linear(a, wq, bias, act_fmt="mxfp8", out=out, workspace=ws)
        flops = 2.0 * M * N * K
        dtype, peak = "mxfp8", PEAK_TFLOPS["mxfp8"]
        aq = mx.quantize(a, "mxfp8", layout="tiled")
        kernels["gemm_ms"] = time_events(lambda: mx.linear_q(aq, wq, bias, out=out), args.steps, torch)
        kernels["gemm_tflops"] = flops / (kernels["gemm_ms"] * 1e-3) / 1e12
        kernels["quant_mxfp8_ms"] = time_events(lambda: mx.quantize(a, "mxfp8", out=aq), args.steps, torch)
    elif wl.fmt == "nvfp4":
        wq = mx.quantize_weight_nvfp4(w_dev)
        sg_a = mx.nvfp4_global_scale(wl.act_amax_static)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mx.linear_workspace_bytes(M, K, "nvfp4"), dtype=torch.uint8, device="cuda")
        step = lambda: mx.linear(a, wq, bias, act_fmt="nvfp4", act_global_scale=sg_a, out=out, workspace=ws)
        flops = 2.0 * M * N * K
        dtype, peak = "nvfp4->f16", PEAK_TFLOPS["bf16"]  # FP16 and BF16 MFMA share the 2.5 PF peak
        aq = mx.quantize(a, "nvfp4", sg_a)
        kernels["gemm_ms"] = time_events(lambda: mx.linear_q(aq, wq, bias, out=out), args.steps, torch)
        kernels["quant_nvfp4_ms"] = time_events(lambda: mx.quantize(a, "nvfp4", sg_a, out=aq), args.steps, torch)
    elif wl.fmt == "norm":
        # the producer in front of the linear, fused with its quantizer, against the unfused pair
        sc, sh = wl.modulation()
        mod = {"scale": torch.from_numpy(sc).cuda(), "shift": torch.from_numpy(sh).cuda()}
        q = mx.norm_quantize(a, 1e-6, fmt="mxfp4", layout="tiled", **mod)
        h = mx.norm(a, 1e-6, **mod)
        aq = mx.empty_qmatrix(M, K, "mxfp4", layout="tiled")
        step = lambda: mx.norm_quantize(a, 1e-6, fmt="mxfp4", layout="tiled", out=q, **mod)
        kernels["norm_bf16_ms"] = time_events(lambda: mx.norm(a, 1e-6, out=h, **mod), args.steps, torch)
        kernels["quantize_ms"] = time_events(lambda: mx.quantize(h, "mxfp4", out=aq), args.steps, torch)
        kernels["unfused_ms"] = kernels["norm_bf16_ms"] + kernels["quantize_ms"]
        for _ in range(args.warmup):
            step()
        ms = time_events(step, args.steps, torch)
        kernels["step_per_launch_ms"] = launch_stats(step, args.steps, torch, 1)
        byts = M * K * 2 + M * K // 2 + M * K // 32 + 2 * K * 4
        v = byts / (ms * 1e-3) / 1e9
        kernels["speedup_vs_unfused"] = kernels["unfused_ms"] / ms
        return {"metric": f"{wl.name} GB/s (LayerNorm + modulation + MXFP4 quantization, fused)",
                "value": v, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "bf16->mxfp4", "data": "synthetic",
                "config": {"workload": wl.name, "M": M, "K": K, "algorithmic_bytes": byts},
                "frac_of_peak": v / HBM_GBPS, "peak_gbps": HBM_GBPS, "kernels": kernels}
    else:
        raise SystemExit(f"unknown variant workload {args.workload}")
    for _ in range(args.warmup):
        step()
    ms = time_events(step, args.steps, torch)
    kernels["step_per_launch_ms"] = launch_stats(step, args.steps, torch, 1)
    v = flops / (ms * 1e-3) / 1e12
    return {"metric": f"{wl.name} TFLOPS (quant+GEMM)", "value": v, "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
            "config": {"workload": wl.name, "M": M, "K": K, "N": N},
            "frac_of_peak": v / peak, "peak_tflops": peak, "kernels": kernels}


def bench_attention(args, torch, mx, synth):
    """Microscaled attention at the Wan2.2-A14B 720p self-attention shape, in the projections'
    layout: one step quantizes Q and K to MXFP4 and V^T to MXFP8, then runs the attention kernel.
    FLOPs 4 S^2 D H (half on FP4 x FP4 MFMA, half on FP8 x FP8); the peak quoted is that mix's,
    1 / (0.5 / 10.1 + 0.5 / 5.0) PFLOP/s."""
    import numpy as np
    wl = synth.WORKLOADS[args.workload]
    S, H, D = wl.M, wl.extra["heads"], mx.ATTN_HEAD_DIM
    to_dev = lambda x: torch.from_numpy(synth.bits16(synth.to_bf16(x)).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = (to_dev(x) for x in wl.qkv())
    vv = v.view(S, H, D).transpose(0, 1)
    qg, kg = mx.quantize(q, "mxfp4"), mx.quantize(k, "mxfp4")
    vt = mx.quantize_vt(vv)
    o = torch.empty((S, H * D), dtype=torch.bfloat16, device="cuda")
    attn = lambda: mx.attention(qg, kg, vt, H, layout="shd", out=o)
    step = lambda: (mx.quantize(q, "mxfp4", out=qg), mx.quantize(k, "mxfp4", out=kg),
                    mx.quantize_vt(vv, out=vt), attn())
    flops = 4.0 * S * S * D * H
    peak = 1.0 / (0.5 / PEAK_TFLOPS["mxfp4"] + 0.5 / PEAK_TFLOPS["mxfp8"])
    kernels = {}
    for _ in range(args.warmup):
        step()
    ms = time_events(step, args.steps, torch)
    kernels["attention_ms"] = time_events(attn, args.steps, torch)
    kernels["attention_per_launch_ms"] = launch_stats(attn, min(args.steps, 10), torch, 1)
    kernels["attention_tflops"] = flops / (kernels["attention_ms"] * 1e-3) / 1e12
    kernels["quant_qk_ms"] = time_events(lambda: (mx.quantize(q, "mxfp4", out=qg), mx.quantize(k, "mxfp4", out=kg)),
                                         args.steps, torch)
    kernels["quant_vt_ms"] = time_events(lambda: mx.quantize_vt(vv, out=vt), args.steps, torch)
    val = flops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu:
        # the oracle on 64 query rows of head 0 against all S keys (its quantization of that
        # head's Q, K and V^T included), as TFLOP/s of the same 4 S D work per query row
        import oracle as O
        hb = [synth.bits16(x[:, :D].contiguous().cpu()) for x in (q, k, v)]  # head 0's columns
        rows = np.concatenate([np.arange(32), np.arange(S - 32, S)])
        t0 = time.perf_counter()
        qc, qs = O.quantize_mx_bf16(hb[0])
        kc, ks = O.quantize_mx_bf16(hb[1])
        vtc, vts = O.quantize_vt_mx8(hb[2], 1, S, D, mx.ATTN_KVB)
        O.attention_mx(qc, qs, kc, ks, vtc, vts, 1, S, D, mx.ATTN_KVB, D ** -0.5, qrows=rows)
        dt = time.perf_counter() - t0
        cpu = {"value": 4.0 * S * D * rows.size / dt / 1e12, "unit": "TFLOP/s",
               "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), "kind": "oracle",
               "sample": f"64 query rows (first and last 32) of head 0 against all {S} keys, with that "
                         f"head's quantization: {dt:.2f} s; CPU: {cpu_info()}"}
    return {"metric": f"{wl.name} TFLOPS (Q/K/V quantization + attention)", "value": val,
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "mxfp4 QK, mxfp8 PV", "data": "synthetic",
            "config": {"workload": wl.name, "S": S, "heads": H, "head_dim": D},
            "frac_of_peak": val / peak, "peak_tflops": peak, "kernels": kernels, "cpu_baseline": cpu}


COPY_BYTES = 1 << 30
COPY_KERNEL_HINT = "copy"  # substring of the device copy kernel's name in the counter CSV


def copy_calibration(torch):
    """A plain copy of COPY_BYTES (read once, written once): the counters' bytes for it give the
    scale factor from FETCH_SIZE / WRITE_SIZE to HBM bytes."""
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES}), flush=True)


def _counter_means(csv_path: str, counter: str):
    """Counter value per dispatch (KiB), by kernel name, from a rocprofv3 counter CSV: the mean
    over the dispatches within a factor 2 of the kernel's largest (the full-size launches; the
    same kernel also runs on the small weight matrix at set-up)."""
    import csv
    vals = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    out = {}
    for k, v in vals.items():
        big = [x for x in v if x >= 0.5 * max(v)]
        out[k] = (sum(big) / len(big), len(big))
    return out


def ingest_counters(args, fetch_csv: str, write_csv: str, out_md: str):
    """Every kernel of the counter runs except the calibration copy: HBM bytes per launch (the
    counters scaled by the copy calibration) into profiles/traffic.json under the workload, keyed
    by kernel name, and a table appended to out_md."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")

    def find(d, *subs):
        hits = [k for k in d if all(s in k for s in subs)]
        if not hits:
            raise SystemExit(f"no kernel matching {subs} in counters")
        return max(hits, key=lambda k: d[k][0])

    kc_f, kc_w = find(fetch, COPY_KERNEL_HINT), find(write, COPY_KERNEL_HINT)
    f_scale = COPY_BYTES / (fetch[kc_f][0] * 1024.0)
    w_scale = COPY_BYTES / (write[kc_w][0] * 1024.0)
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    wl = table[args.workload] = {}
    lines = [f"# HBM traffic per launch, workload {args.workload}", "",
             f"Copy calibration: {kc_f}: FETCH_SIZE {fetch[kc_f][0]:.0f} KiB, "
             f"WRITE_SIZE {write[kc_w][0]:.0f} KiB per launch for a {COPY_BYTES} B copy; "
             f"scale factors {f_scale:.4f} (fetch), {w_scale:.4f} (write).", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read B | HBM write B |",
             "|---|---|---|---|---|---|"]
    for kf in sorted(fetch):
        if COPY_KERNEL_HINT in kf or kf not in write or kf.startswith("void at::"):
            continue  # the calibration copy and torch's own fill kernel
        rd, wr = fetch[kf][0] * 1024.0 * f_scale, write[kf][0] * 1024.0 * w_scale
        wl[kf] = {"bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
                  "source_hash": kernel_source_hash(kf)}
        lines.append(f"| {kf[:110]} | {fetch[kf][1]} | {fetch[kf][0]:.0f} | {write[kf][0]:.0f} | "
                     f"{rd:.4g} | {wr:.4g} |")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    with open(out_md, "a") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan_a14b_attn_75600x5120x5120")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=16384,
                    help="rows of the CPU oracle sample (about 10-30 s on 8-16 cores)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain device copy of COPY_BYTES, for HBM counter calibration")
    ap.add_argument("--ingest-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; each holding the "
                         "copy calibration and a bench run) into profiles/traffic.json and a summary")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(args, *args.ingest_counters)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only: the linear shards along M "
                                   "(tokens) with no exchange between GPUs, so one GPU's share is the "
                                   "measured unit; run --gpus 1"}), flush=True)
        raise SystemExit(2)

    import torch
    import fp4_block_scaled_amd as mx
    from fp4_block_scaled_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    mx.lib()
    if args.copy_calibration:
        copy_calibration(torch)
    if args.workload == "wan_a14b_attn_75600x5120x5120" or synth.WORKLOADS[args.workload].fmt == "mxfp4" \
            and not synth.WORKLOADS[args.workload].N2:
        res = bench_mx_linear(args, torch, mx, synth)
    elif synth.WORKLOADS[args.workload].fmt == "attn":
        res = bench_attention(args, torch, mx, synth)
    else:
        res = bench_variant(args, torch, mx, synth)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
