#!/usr/bin/env python3
"""Benchmark of the int8 linear layer's hot path on one MI355X.

One step = the whole path over one batch for every linear of the workload:
for each layer, the forward call (fp16 cast, outlier columns, row-wise int8
quantization, int8 MFMA GEMM with fused dequant / outlier product / bias /
cast) and the memory-efficient backward call (fp16 MFMA GEMM over int8
weights dequantized on the fly, plus grad_bias when the layer has a bias).
Weights are quantized once before timing (offline step of the layer).

Default workload: the 7B decoder-block linear set (q, k, v, o 4096x4096;
gate/up 4096->11008; down 11008->4096; 4096 tokens, bf16, 0.1 % outlier
columns x20, threshold 6.0). Inputs are synthetic and resident in HBM;
several input sets rotate so the footprint exceeds the 256 MB Infinity Cache.

Prints ONE JSON line. value = effective TOPS = sum over layers of 4*M*N*K
(2MNK int8 ops forward + 2MNK fp16 flops backward) / time per step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "int8 linear fwd+bwd effective TOPS at 7B shapes; % of int8 MFMA peak"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
PEAK_F16_TFLOPS = 2500.0     # MI355X dense fp16 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s

TORCH_DT = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_gpu_inputs(wl, n_sets, seed_base=1234):
    """Per layer: weights (quantized by the library) and n_sets (A, G) pairs drawn on the GPU
    with the workload's recipe (N(0,1) activations, seeded outlier columns scaled, grad ~ N(0, std))."""
    import torch

    import int8_quantized_linear_rowwise_amd as I8
    import workloads

    dt = getattr(torch, TORCH_DT[wl.dtype])
    dev = "cuda:0"
    layers = []
    for li, L in enumerate(wl.layers):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed_base + 101 * li)
        W = torch.randn((L.N, L.K), generator=gen, device=dev, dtype=torch.float32) * wl.w_std
        CB, SCB = I8.quantize_weight(W)
        del W
        bias = None
        if L.has_bias:
            bias = (torch.randn((L.N,), generator=gen, device=dev) * wl.bias_std).to(dt)
        cols = torch.from_numpy(workloads.outlier_columns(wl.wid, li, L.K, L.n_outliers)).to(dev)
        sets = []
        for s in range(n_sets):
            A = torch.randn((L.M, L.K), generator=gen, device=dev, dtype=torch.float32) * wl.act_std
            if cols.numel():
                A[:, cols] *= wl.outlier_scale
            G = torch.randn((L.M, L.N), generator=gen, device=dev, dtype=torch.float32) * wl.grad_std
            sets.append((A.to(dt).contiguous(), G.to(dt).contiguous()))
            del A, G
        layers.append(dict(L=L, CB=CB, SCB=SCB, bias=bias, sets=sets,
                           out=torch.empty((L.M, L.N), dtype=dt, device=dev),
                           gA=torch.empty((L.M, L.K), dtype=dt, device=dev),
                           gb=torch.empty((L.N,), dtype=dt, device=dev) if L.has_bias else None,
                           cap=I8.default_cap(L.K),
                           wsf=I8.forward_workspace(L.M, L.K, L.N, I8.default_cap(L.K), dev),
                           wsb=torch.empty((max(1, I8.lib.int8_linear_backward_workspace_bytes(
                               L.M, L.N, int(L.has_bias))),), dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()
    return layers


def run_gpu(wl, steps, warmup, n_sets, threshold):
    import torch

    import int8_quantized_linear_rowwise_amd as I8

    layers = make_gpu_inputs(wl, n_sets)
    nl = len(layers)

    def call_fwd(ly, s):
        A, _ = ly["sets"][s]
        I8.int8_linear_forward(A, ly["CB"], ly["SCB"], ly["bias"], threshold, ly["cap"], out=ly["out"],
                               workspace=ly["wsf"])

    def call_bwd(ly, s):
        _, G = ly["sets"][s]
        I8.int8_linear_backward_input(G, ly["CB"], ly["SCB"], with_grad_bias=ly["gb"] is not None,
                                      grad_A=ly["gA"], grad_bias=ly["gb"], workspace=ly["wsb"])

    for w in range(warmup):
        for ly in layers:
            call_fwd(ly, w % n_sets)
            call_bwd(ly, w % n_sets)
    torch.cuda.synchronize()
    # outlier columns found by the forward (any number is handled; the first
    # `cap` are staged, later ones read from the input by the epilogue)
    n_outliers = [I8.forward_check(ly["wsf"], ly["L"].M, ly["L"].K, ly["L"].N, ly["cap"]) for ly in layers]

    # one step = forward of every layer (in order), then backward of every layer
    # (reverse order), as in a training step; one event pair brackets each phase
    # so that the backward GEMM's launches run back to back between two events
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for k in range(steps):
        s = k % n_sets
        e0, e1, e2 = ev[k]
        e0.record(stream)
        for ly in layers:
            call_fwd(ly, s)
        e1.record(stream)
        for ly in reversed(layers):
            call_bwd(ly, s)
        e2.record(stream)
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    gpu_ms = ev[0][0].elapsed_time(ev[-1][2])
    step_ms = [e[0].elapsed_time(e[2]) for e in ev]
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps

    # quantizer alone (diagnostic, outside the timed region): the same rotation over
    # every layer's activations (footprint beyond the Infinity Cache), same stream
    dev = "cuda:0"
    qbuf = []
    for ly in layers:
        L = ly["L"]
        wsb = I8.lib.int8_quantize_rowwise_workspace_bytes(L.M, L.K)
        qbuf.append(dict(codes=torch.empty((L.M, L.K), dtype=torch.int8, device=dev),
                         scale=torch.empty((L.M,), dtype=torch.float32, device=dev),
                         idx=torch.empty((L.K,), dtype=torch.int32, device=dev),
                         cnt=torch.empty((1,), dtype=torch.int32, device=dev),
                         sub=torch.empty((L.M, L.K), dtype=torch.float16, device=dev),
                         ws=torch.empty((wsb,), dtype=torch.uint8, device=dev), wsb=wsb))
    reps = 4
    qev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in layers]
           for _ in range(reps + 1)]
    for rr in range(reps + 1):
        for li, ly in enumerate(layers):
            L, qb = ly["L"], qbuf[li]
            A2 = ly["sets"][rr % n_sets][0]
            qev[rr][li][0].record(stream)
            I8.check(I8.lib.int8_quantize_rowwise(A2.data_ptr(), I8.DTYPE_CODE[A2.dtype], L.M, L.K, threshold,
                                                  qb["codes"].data_ptr(), qb["scale"].data_ptr(),
                                                  qb["idx"].data_ptr(), qb["cnt"].data_ptr(),
                                                  qb["sub"].data_ptr(), L.K, qb["ws"].data_ptr(), qb["wsb"],
                                                  stream.cuda_stream), "int8_quantize_rowwise")
            qev[rr][li][1].record(stream)
    torch.cuda.synchronize()
    q_ms = [sum(qev[rr][li][0].elapsed_time(qev[rr][li][1]) for rr in range(1, reps + 1)) / reps
            for li in range(nl)]
    del qbuf

    # int8 backward variant (diagnostic, outside the timed region): G quantized
    # row-wise times a second int8 weight copy quantized along the input
    # features; the same rotation, every layer in reverse order, same stream
    for ly in layers:
        L = ly["L"]
        gen = torch.Generator(device=dev)
        gen.manual_seed(1234 + 101 * layers.index(ly))
        W = torch.randn((L.N, L.K), generator=gen, device=dev, dtype=torch.float32) * wl.w_std
        ly["CBt"], ly["SCBt"] = I8.quantize_weight_colwise(W)
        ly["ws8"] = I8.backward_int8_workspace(L.M, L.N, ly["gb"] is not None, dev)
        del W

    def call_bwd8(ly, s):
        _, G = ly["sets"][s]
        I8.int8_linear_backward_input_int8(G, ly["CBt"], ly["SCBt"], with_grad_bias=ly["gb"] is not None,
                                           grad_A=ly["gA"], grad_bias=ly["gb"], workspace=ly["ws8"])

    for w in range(2):
        for ly in reversed(layers):
            call_bwd8(ly, w % n_sets)
    b8 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for k in range(steps):
        b8[k][0].record(stream)
        for ly in reversed(layers):
            call_bwd8(ly, k % n_sets)
        b8[k][1].record(stream)
    torch.cuda.synchronize()
    bwd8_ms = sum(a.elapsed_time(b) for a, b in b8) / steps
    for ly in layers:
        del ly["CBt"], ly["SCBt"], ly["ws8"]

    # weight gradient of the trainable-weight mode (diagnostic, outside the
    # timed region): every layer in reverse order, same rotation and stream
    for ly in layers:
        L = ly["L"]
        ly["gW"] = torch.empty((L.N, L.K), dtype=ly["gA"].dtype, device=dev)

    def call_wgrad(ly, s):
        A, G = ly["sets"][s]
        I8.int8_linear_backward_weight(G, A, grad_W=ly["gW"])

    for w in range(2):
        for ly in reversed(layers):
            call_wgrad(ly, w % n_sets)
    wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for k in range(steps):
        wev[k][0].record(stream)
        for ly in reversed(layers):
            call_wgrad(ly, k % n_sets)
        wev[k][1].record(stream)
    torch.cuda.synchronize()
    wgrad_ms = sum(a.elapsed_time(b) for a, b in wev) / steps
    for ly in layers:
        del ly["gW"]

    # producer-side outlier flags (diagnostic): for the layer with the widest
    # input, its input made by the SiLU kernel from a same-shaped tensor, then
    # the forward with its own flagging pass against the flagged forward
    ly = max(layers, key=lambda l: l["L"].K)
    L = ly["L"]
    Hs = [ly["sets"][s][0] for s in range(n_sets)]
    As = [torch.empty_like(h) for h in Hs]
    fls = [I8.outlier_flags_buffer(L.M, L.K, dev) for _ in Hs]

    def silu_leg(s):
        I8.silu_outlier_flags(Hs[s], threshold, A=As[s], flags=fls[s])

    def fwd_plain(s):
        I8.int8_linear_forward(As[s], ly["CB"], ly["SCB"], ly["bias"], threshold, ly["cap"], out=ly["out"],
                               workspace=ly["wsf"])

    def fwd_flagged(s):
        I8.int8_linear_forward_flagged(As[s], fls[s], ly["CB"], ly["SCB"], ly["bias"], ly["cap"], out=ly["out"],
                                       workspace=ly["wsf"])

    def timed_leg(f, reps=10):
        for w in range(2):
            f(w % n_sets)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for k in range(reps):
            evs[k][0].record(stream)
            f(k % n_sets)
            evs[k][1].record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]

    pf = dict(layer=f"{L.name} {L.M}x{L.K}", silu_flags_ms=timed_leg(silu_leg), forward_ms=timed_leg(fwd_plain),
              forward_flagged_ms=timed_leg(fwd_flagged))
    del As, fls
    return dict(layers=layers, gpu_ms=gpu_ms, host_s=h1 - h0, fwd_ms=fwd_ms, bwd_ms=bwd_ms, q_ms=q_ms,
                bwd8_ms=bwd8_ms, wgrad_ms=wgrad_ms, pf=pf, step_ms=step_ms, n_outliers=n_outliers)


def copy_calibration(nbytes=1 << 30):
    """A plain device-to-device copy of known size (read nbytes, write nbytes), three times."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def traffic_from_profile(kernel_src: str, name: str):
    """HBM bytes per launch of the dominant kernel from the committed counter summary,
    valid only while the kernel's source is byte-identical to the profiled one."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", name)
    src = os.path.join(ROOT, "int8_quantized_linear_rowwise_amd", "csrc", kernel_src)
    if not (os.path.exists(prof) and os.path.exists(src)):
        return None
    vals = {}
    for line in open(prof):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if vals.get("source_sha256") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def percentile(xs, p):
    """p-th percentile (linear interpolation between order statistics)."""
    v = sorted(xs)
    if not v:
        return None
    x = (len(v) - 1) * p / 100.0
    i = int(x)
    j = min(i + 1, len(v) - 1)
    return v[i] + (v[j] - v[i]) * (x - i)


def combined_ceiling(wl, reads=2):
    """The workload's best possible effective TOPS as a share of the int8
    peak: every quantizer at full HBM bandwidth (its input read `reads` times:
    2 for the two-pass quantizer used, 1 for the one-read minimum), every
    forward GEMM at the int8 MFMA peak and every backward GEMM at the fp16
    MFMA peak (its operands are fp16 by the method's definition)."""
    isz = 4 if wl.dtype == "f32" else 2
    ops = t = 0.0
    for L in wl.layers:
        q_bytes = reads * L.M * L.K * isz + L.M * L.K + 4 * L.M + L.K
        t += q_bytes / (PEAK_HBM_GBS * 1e9) + 2 * L.M * L.N * L.K / (PEAK_INT8_TOPS * 1e12) \
            + 2 * L.M * L.N * L.K / (PEAK_F16_TFLOPS * 1e12)
        ops += 4 * L.M * L.N * L.K
    return 100.0 * ops / t / 1e12 / PEAK_INT8_TOPS


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, target_s, threshold):
    """The oracle, untuned, on a bounded sample: every layer of the workload at a reduced token count."""
    import numpy as np

    import oracle
    import workloads

    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    qw = []
    for li in range(len(wl.layers)):
        qw.append(oracle.quantize_weight(workloads.make_weight(wl, li)))

    # calibrate on a small sample, then size the sample to about target_s seconds
    def timed(Ms):
        tt = 0.0
        ops = 0
        for li, L in enumerate(wl.layers):
            A = workloads.make_activation(wl, li, rows=Ms)
            G = workloads.make_grad(wl, li, rows=Ms)
            b = workloads.make_bias(wl, li)
            cb, scb = qw[li]
            t1 = time.perf_counter()
            oracle.linear_forward(A, wl.dtype, cb, scb, b, threshold)
            oracle.linear_backward_input(G, wl.dtype, cb, scb)
            if b is not None:
                oracle.grad_bias(G, wl.dtype)
            tt += time.perf_counter() - t1
            ops += 4 * Ms * L.N * L.K
        return ops, tt

    # grow the token sample until one pass takes about target_s (fixed costs
    # dominate small samples, so scale in a few steps)
    Mmax = wl.layers[0].M
    Ms = 64
    ops, tt = timed(Ms)
    for _ in range(4):
        if tt >= 0.6 * target_s or Ms >= Mmax:
            break
        Ms = int(min(Mmax, max(2 * Ms, Ms * target_s / max(tt, 1e-3))))
        Ms = max(64, (Ms // 64) * 64)
        ops, tt = timed(Ms)
    return {"value": ops / tt / 1e12, "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "host_cpu": host_cpu_model(), "host_threads_visible": len(os.sched_getaffinity(0)),
            "sample": f"all {len(wl.layers)} layers of {wl.name} at {Ms} tokens (of {Mmax}): quantize + "
                      f"forward + backward, numpy float64, {tt:.1f} s"}


def run_peaks():
    """Roofline constants measured on this GPU: MFMA-only loops (the two
    instructions of the layer's GEMMs, one and two waves per SIMD) with the
    shader clock they ran at, and HBM read / copy bandwidth of large buffers."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "int8_quantized_linear_rowwise_amd", "libi8lpeaks.so"))
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    lib.i8l_peak_mfma.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.i8l_peak_mfma_macs.restype = i64
    lib.i8l_peak_mfma_macs.argtypes = [i32]
    lib.i8l_peak_read.argtypes = [vp, i64, vp, i32, vp]
    lib.i8l_peak_copy.argtypes = [vp, vp, i64, i32, vp]
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    out = {"mfma": [], "hbm": []}

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None else min(best, t)
        return best

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for kind, name, peak in ((0, "v_mfma_i32_32x32x32_i8", PEAK_INT8_TOPS), (1, "v_mfma_f32_32x32x16_f16", PEAK_F16_TFLOPS)):
        for wps in (1, 2):
            blocks, iters = cus * wps, 40000
            sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
            clk = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)

            def go():
                rc = lib.i8l_peak_mfma(kind, blocks, iters, sink.data_ptr(), clk.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"i8l_peak_mfma: hip error {rc}")

            t = timed(go, 3)
            c = clk.view(-1, 4).cpu().double()
            ghz = ((c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100e6) / 1e9).median().item()
            ops = blocks * 4 * iters * 8 * 2 * lib.i8l_peak_mfma_macs(kind)
            rate = ops / t / 1e12
            out["mfma"].append({"instruction": name, "waves_per_simd": wps, "tops": round(rate, 1),
                                "pct_published": round(100 * rate / peak, 1), "published": peak,
                                "shader_clock_ghz": round(ghz, 3),
                                "pct_of_published_at_that_clock": round(100 * rate / (peak * ghz / 2.4), 1)})
            log(f"[peaks] {name} {wps} wave/SIMD: {rate:.0f} T/s at {ghz:.2f} GHz")
    nbytes = 4 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    blocks = cus * 8
    t = timed(lambda: lib.i8l_peak_read(src.data_ptr(), nbytes, sink.data_ptr(), blocks, stream.cuda_stream), 5)
    out["hbm"].append({"kernel": "read 4 GiB", "gbs": round(nbytes / t / 1e9, 1),
                       "pct_published": round(100 * nbytes / t / 1e9 / PEAK_HBM_GBS, 1)})
    t = timed(lambda: lib.i8l_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks, stream.cuda_stream), 5)
    out["hbm"].append({"kernel": "copy 4 GiB (read + write)", "gbs": round(2 * nbytes / t / 1e9, 1),
                       "pct_published": round(100 * 2 * nbytes / t / 1e9 / PEAK_HBM_GBS, 1)})
    t = timed(lambda: dst.copy_(src), 5)
    out["hbm"].append({"kernel": "torch copy_ 4 GiB (read + write)", "gbs": round(2 * nbytes / t / 1e9, 1),
                       "pct_published": round(100 * 2 * nbytes / t / 1e9 / PEAK_HBM_GBS, 1)})
    out["compute_units"] = cus
    out["device"] = torch.cuda.get_device_name(0)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first ~10 steps after an idle GPU run up to 1 % slower than the steady state
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="llama7b_block")
    ap.add_argument("--sets", type=int, default=2, help="rotating input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--peaks", action="store_true",
                    help="measure the roofline constants (MFMA-only loops, HBM read/copy) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.peaks:
        print(json.dumps({"peaks": run_peaks()}), flush=True)
        return

    import workloads
    wl = workloads.WORKLOADS[args.workload]
    threshold = wl.threshold
    log(f"[bench] workload {wl.name}: {len(wl.layers)} layers, steps={args.steps} warmup={args.warmup}")
    if args.copy_calibration:
        copy_calibration()
    r = run_gpu(wl, args.steps, args.warmup, args.sets, threshold)
    ms = r["gpu_ms"] / args.steps
    ops = sum(4 * L.M * L.N * L.K for L in wl.layers)
    tops = ops / (ms * 1e-3) / 1e12
    bwd_flops = sum(2 * L.M * L.N * L.K for L in wl.layers)
    bwd_ms = r["bwd_ms"]
    fwd_ms = r["fwd_ms"]
    q_ms = sum(r["q_ms"])
    bwd_tflops = bwd_flops / (bwd_ms * 1e-3) / 1e12
    fwd_gemm_ms = max(fwd_ms - q_ms, 1e-9)
    fwd_tops = bwd_flops / (fwd_gemm_ms * 1e-3) / 1e12
    isz = 2 if wl.dtype != "f32" else 4
    qbytes = sum(L.M * L.K * isz + L.M * L.K + 4 * L.M + L.K for L in wl.layers)  # 1-read minimum (+ |O| terms ~0)
    q_gbs = qbytes / (q_ms * 1e-3) / 1e9

    line = {
        "metric": METRIC, "value": round(tops, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8+fp16", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.layers[0].M,
                   "layers": ", ".join(f"{L.name} {L.K}->{L.N}" for L in wl.layers), "io_dtype": wl.dtype,
                   "threshold": threshold, "input_sets": args.sets},
        "pct_int8_peak": round(100.0 * tops / PEAK_INT8_TOPS, 2),
        "ceiling_pct_int8_peak": round(combined_ceiling(wl, reads=2), 1),
        "ceiling_pct_int8_peak_one_read": round(combined_ceiling(wl, reads=1), 1),
        "step_ms": {"median": round(percentile(r["step_ms"], 50), 4), "p10": round(percentile(r["step_ms"], 10), 4),
                    "p90": round(percentile(r["step_ms"], 90), 4), "min": round(min(r["step_ms"]), 4),
                    "max": round(max(r["step_ms"]), 4)},
        "outlier_columns_per_layer": r["n_outliers"],
        "roofline": {"kernel": "k_gemm_bwd_w8 (memory-efficient backward grad_A, fp16 MFMA)", "bound": "mfma",
                     "achieved": round(bwd_tflops, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bwd_tflops / PEAK_F16_TFLOPS, 4),
                     "traffic": traffic_from_profile("gemm_bwd.hip", f"k_gemm_bwd_w8_{wl.name}_traffic.txt")},
        "breakdown_ms_per_step": {"forward_calls": round(fwd_ms, 4), "backward_calls": round(bwd_ms, 4),
                                  "quantizer_alone": round(q_ms, 4), "forward_gemm_est": round(fwd_gemm_ms, 4)},
        "per_gemm": {"fwd_int8_tops_est": round(fwd_tops, 1),
                     "fwd_pct_int8_peak": round(100 * fwd_tops / PEAK_INT8_TOPS, 2),
                     "bwd_fp16_tflops": round(bwd_tflops, 1),
                     "bwd_pct_fp16_peak": round(100 * bwd_tflops / PEAK_F16_TFLOPS, 2),
                     "quantizer_gbs_1read": round(q_gbs, 1),
                     "quantizer_pct_hbm": round(100 * q_gbs / PEAK_HBM_GBS, 2)},
        "int8_backward": {"calls_ms": round(r["bwd8_ms"], 4),
                          "int8_tops": round(bwd_flops / (r["bwd8_ms"] * 1e-3) / 1e12, 1),
                          "step_tops_with_it": round(ops / ((fwd_ms + r["bwd8_ms"]) * 1e-3) / 1e12, 1),
                          "note": "backward variant with G quantized to int8 (quantizer + int8 GEMM + grad_bias); "
                                  "timed separately, not part of value"},
        "weight_grad": {"calls_ms": round(r["wgrad_ms"], 4),
                        "fp16_tflops": round(bwd_flops / (r["wgrad_ms"] * 1e-3) / 1e12, 1),
                        "pct_fp16_peak": round(100 * bwd_flops / (r["wgrad_ms"] * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 2),
                        "note": "trainable-weight mode's grad_W = fp16(G)^T fp16(A) of every layer; timed "
                                "separately, not part of value"},
        "producer_flags": {"layer": r["pf"]["layer"], "silu_and_flags_ms": round(r["pf"]["silu_flags_ms"], 4),
                           "forward_ms": round(r["pf"]["forward_ms"], 4),
                           "forward_with_producer_flags_ms": round(r["pf"]["forward_flagged_ms"], 4),
                           "note": "the widest-input layer's forward with its own flagging pass, and with the "
                                   "flags the SiLU kernel made while producing its input (median of 10 calls); "
                                   "not part of value"},
        "host_wall_s": round(r["host_s"], 3),
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, threshold)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
