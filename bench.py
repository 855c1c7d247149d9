"""Benchmark of the FP4 quantized linear forward on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload llama7b_gate_up]

A step is one fp4_linear_forward (quantile + clamp + dA, token-wise quantization of A,
channel-wise quantization of W, FP4 GEMM with dequantization, compensation pass) over one
batch of seeded synthetic input already resident in HBM.  Default workload: the
LLaMA-7B FFN gate+up projection (M=16384 tokens, K=4096, N=22016, bf16 in and out,
clamp quantile 0.999).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import quantized_linear_layers_fp4_amd as fp4  # noqa: E402
from workloads import WORKLOADS, make_layer  # noqa: E402

METRIC = "FP4 quantized-linear TFLOPS & % dense FP4 MFMA peak; quantizer HBM GB/s"
PEAK_FP4_TFLOPS = 10100.0   # MI355X dense FP4 matrix peak (10.1 PFLOP/s)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (8 TB/s)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 matrix peak (5.0 PFLOP/s)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_llama7b_gate_up.json")
GEMM_SRC = os.path.join(ROOT, "quantized_linear_layers_fp4_amd", "csrc", "gemm.hip")
COMP_SRC = os.path.join(ROOT, "quantized_linear_layers_fp4_amd", "csrc", "comp.hip")
QUANT_SRC = os.path.join(ROOT, "quantized_linear_layers_fp4_amd", "csrc", "quant.hip")
# the forward's quantizer launches (both sides in one stage call)
QUANT_KERNELS = ("k_zero_u32", "k_hist_rowmax", "k_select_colmax", "k_quant_rows", "k_coo_qcols")


def b_in(dtype: torch.dtype) -> int:
    return 2 if dtype == torch.bfloat16 else 4


def quantizer_bytes(M, K, N, bi, nnz, with_w: bool = True) -> int:
    """Algorithmic HBM bytes of the quantizer stages: A read twice (histogram pass, then
    clamp+quantize: T must be known before any code), codes, scales, dA; W read once,
    codes, scales."""
    a = 2 * M * K * bi + M * K // 2 + 4 * M + 12 * nnz + 4 * (M + 1)
    w = K * N * bi + K * N // 2 + 4 * N
    return a + (w if with_w else 0)


def comp_bytes(M, N, b_out, nnz) -> int:
    """Algorithmic HBM bytes of the compensation pass: the GEMM's two-byte accumulators read
    and Y written, plus the dA list and the row scales; the W rows it gathers and the column
    scales are counted as L2 traffic, not HBM (each is reused by many tasks)."""
    return M * N * 2 + M * N * b_out + 8 * nnz + 4 * (M + 1) + 4 * M


def time_on_stream(fn, steps: int, warmup: int, rounds: int = 3) -> float:
    """Average milliseconds of fn() per call, HIP events on the current stream (the stream
    every launch of fn goes to): the median over `rounds` runs of `steps` back-to-back calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    out = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(steps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return sorted(out)[len(out) // 2]


def gemm_kernel(M: int, N: int, K: int) -> str:
    """Name of the GEMM kernel the library launches for this shape on this device (the
    library's own selection rule, exported through the C ABI)."""
    return fp4.gemm_kernel_name(M, N, K, torch.cuda.get_device_properties(0).multi_processor_count)


def _kernel_is(name: str):
    """Predicate on rocprofv3 kernel names: the templated kernel `name`, no other."""
    return lambda n: n.replace("void ", "").startswith(f"fp4::{name}<")


def _kernel_named(name: str):
    """Predicate on rocprofv3 kernel names: the kernel `name`, templated or not."""
    return lambda n: n.replace("void ", "").startswith((f"fp4::{name}<", f"fp4::{name}("))


def _gemm_main(name: str):
    """The GEMM launch among rocprofv3 kernel names: the kernel `name` (the escape kernel that
    follows a two-byte product is another kernel, k_q16_escapes)."""
    return _kernel_is(name)


def gemm_src_sha() -> str:
    return hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()[:16]


def comp_src_sha() -> str:
    return hashlib.sha256(open(COMP_SRC, "rb").read()).hexdigest()[:16]


def quant_src_sha() -> str:
    return hashlib.sha256(open(QUANT_SRC, "rb").read()).hexdigest()[:16]


def load_traffic(launch_bytes_alg: float, what: str = "gemm"):
    """HBM bytes per launch of the GEMM (what="gemm"), of the compensation pass (what="comp"), or
    per quantizer stage call (what="quant", the sum over its launches) from the committed
    rocprofv3 --pmc summary, if it was taken on the current source of those kernels; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if what == "gemm":
        return rec.get("hbm_bytes_per_launch") if rec.get("gemm_src_sha") == gemm_src_sha() else None
    if what == "quant":
        return rec.get("quant_hbm_bytes_per_call") if rec.get("quant_src_sha") == quant_src_sha() else None
    return rec.get("comp_hbm_bytes_per_launch") if rec.get("comp_src_sha") == comp_src_sha() else None


def cpu_baseline(A, W, L, rows: int = 256) -> dict:
    """The oracle, as it stands, on a bounded sample of the same workload: every
    quantizer step at full size, the accumulator/dequant/compensation on `rows` sampled
    rows (the first, the last and seeded others) x all N columns, extrapolated linearly to
    M rows."""
    import oracle
    from workloads import as_numpy_bits
    Anp, Wnp = as_numpy_bits(A), as_numpy_bits(W)
    M, K, N = L.M, L.K, L.N
    t0 = time.perf_counter()
    T = oracle.abs_quantile(Anp, L.q)
    cl = oracle.clamp_coo(Anp, T, want_clamped=True, cap=oracle.capacity(M, K, L.q))
    Aq, sA = oracle.quant_rows(cl.pop("A_clamped"))
    Wq, sW = oracle.quant_cols(Wnp)
    t1 = time.perf_counter()
    # the first and last rows, and rows - 2 seeded others
    rest = np.random.default_rng(0).choice(np.arange(1, M - 1), rows - 2, replace=False)
    rs = np.sort(np.concatenate([[0, M - 1], rest]))
    ms = np.repeat(rs, N).astype(np.int64)
    ns = np.tile(np.arange(N, dtype=np.int64), rows)
    acc = oracle.accumulate_pairs(Aq, Wq, K, ms, ns)
    oracle.output_pairs(acc, sA, sW, ms, ns, cl["row_ptr"], cl["coo_col"], cl["coo_val"], Wnp)
    t2 = time.perf_counter()
    t_full = (t1 - t0) + (t2 - t1) * M / rows
    return {
        "value": round(2.0 * M * N * K / t_full / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
        "sample": (f"{L.name}: quantile, clamp+dA and A/W quantization at full size ({t1 - t0:.2f} s); "
                   f"accumulator+dequant+compensation on {rows} of {M} rows x {N} cols ({t2 - t1:.2f} s), "
                   f"extrapolated x{M // rows} to the full step ({t_full:.1f} s)"),
        "host_cpu": _cpu_model(), "host_threads_available": os.cpu_count(),
    }


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def _counter_per_dispatch(d: str, counter: str, kernel_pred) -> float:
    """Mean over dispatches of one counter for the kernels kernel_pred accepts, from a
    rocprofv3 --pmc csv output directory."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel_pred(r["Kernel_Name"]):
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows in {d}")
    return sum(vals) / len(vals)


def write_traffic(gemm_fetch: str, gemm_write: str, copy_fetch: str, copy_write: str):
    """HBM bytes per GEMM launch (and per k_comp_apply launch) on the 7B gate+up shape:
    FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by the bytes a plain 1 GiB copy moves
    per unit of the same counter, and the same summed over the forward's quantizer launches.
    Written with the hashes of the GEMM, compensation and quantizer sources it was measured on."""
    # the GEMM kernel the library picked for this shape: the one present in the counters
    kname = "k_fp4_gemm_wide"
    try:
        _counter_per_dispatch(gemm_fetch, "FETCH_SIZE", _gemm_main(kname))
    except SystemExit:
        kname = "k_fp4_gemm"
    is_gemm = _gemm_main(kname)
    is_comp = _kernel_is("k_comp_apply")
    is_copy = lambda n: "copyBuffer" in n  # noqa: E731
    c_f = _counter_per_dispatch(copy_fetch, "FETCH_SIZE", is_copy)
    c_w = _counter_per_dispatch(copy_write, "WRITE_SIZE", is_copy)
    f_fetch, f_write = (1 << 30) / c_f, (1 << 30) / c_w
    rec = {"gemm_src_sha": gemm_src_sha(), "comp_src_sha": comp_src_sha(), "workload": "llama7b_gate_up",
           "gemm_kernel": kname,
           "copy_fetch_size": c_f, "copy_write_size": c_w,
           "bytes_per_fetch_unit": f_fetch, "bytes_per_write_unit": f_write}
    for name, pred in (("gemm", is_gemm), ("comp", is_comp)):
        fs = _counter_per_dispatch(gemm_fetch, "FETCH_SIZE", pred)
        ws = _counter_per_dispatch(gemm_write, "WRITE_SIZE", pred)
        pre = "" if name == "gemm" else "comp_"
        rec.update({f"{pre}fetch_size_per_launch": fs, f"{pre}write_size_per_launch": ws,
                    f"{pre}hbm_read_bytes_per_launch": fs * f_fetch, f"{pre}hbm_write_bytes_per_launch": ws * f_write,
                    f"{pre}hbm_bytes_per_launch": round(fs * f_fetch + ws * f_write)})
    qf = sum(_counter_per_dispatch(gemm_fetch, "FETCH_SIZE", _kernel_named(k)) for k in QUANT_KERNELS)
    qw = sum(_counter_per_dispatch(gemm_write, "WRITE_SIZE", _kernel_named(k)) for k in QUANT_KERNELS)
    rec.update({"quant_src_sha": quant_src_sha(), "quant_kernels": list(QUANT_KERNELS),
                "quant_hbm_read_bytes_per_call": qf * f_fetch, "quant_hbm_write_bytes_per_call": qw * f_write,
                "quant_hbm_bytes_per_call": round(qf * f_fetch + qw * f_write)})
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def mfma_probe(iters: int = 20000) -> dict:
    """The FP4 matrix-core rate this device sustains with nothing else running (the probe
    library: one workgroup of four waves per CU, each wave a chain of independent 32x32x64
    FP4 MFMAs on register operands), and the shader clock its loop ran at (shader-clock
    counter against the 100 MHz real-time counter)."""
    L = C.CDLL(os.path.join(ROOT, "quantized_linear_layers_fp4_amd", "libfp4probe.so"))
    L.fp4_probe_mfma_fp4.restype = C.c_int32
    L.fp4_probe_mfma_fp4.argtypes = [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    clocks = torch.zeros(cus * 4 * 4, dtype=torch.int64, device="cuda")
    sink = torch.empty(cus * 256, dtype=torch.float32, device="cuda")
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    run = lambda: L.fp4_probe_mfma_fp4(cus, iters, C.c_void_p(clocks.data_ptr()), C.c_void_p(sink.data_ptr()), st)  # noqa
    assert run() == 0
    ms = time_on_stream(run, 3, 1)
    flops = cus * 4 * iters * 8 * 131072
    c = clocks.view(-1, 4).cpu().numpy().astype(np.float64)
    ghz = float(np.median((c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2]) * 0.1))
    tf = flops / ms / 1e9
    return {"what": "chains of independent FP4 32x32x64 MFMAs on register operands, one 4-wave workgroup per CU",
            "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "frac_of_peak": round(tf / PEAK_FP4_TFLOPS, 4),
            "clock_GHz": round(ghz, 3), "peak_at_that_clock_TFLOP/s": round(PEAK_FP4_TFLOPS * ghz / 2.4, 1)}


def vendor_gemm(M: int, N: int, K: int, ours_ms: float | None = None) -> dict:
    """A same-box reference for the FP4 GEMM: torch._scaled_mm on MX-FP4 operands (which PyTorch
    for ROCm hands to hipBLASLt on gfx950) at the same M, N, K, with random codes, E8M0 block
    scales of 32 all equal to 1 and a bf16 output.  Not part of the forward; recorded beside it."""
    what = ("torch._scaled_mm, MX-FP4 operands (float4_e2m1fn_x2, E8M0 block scales of 32, all 1), bf16 out, "
            "same M, N, K, random codes")
    try:
        dev = torch.device("cuda:0")
        g = torch.Generator(device=dev).manual_seed(20250128)
        a = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=dev, generator=g)
        b = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=g)
        a, b = a.view(torch.float4_e2m1fn_x2), b.view(torch.float4_e2m1fn_x2)
        sa = torch.full((M, K // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
        sb = torch.full((N, K // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
        f = lambda: torch._scaled_mm(a, b.t(), sa, sb, out_dtype=torch.bfloat16)  # noqa: E731
        f()
        ms = time_on_stream(f, 20, 3)
    except Exception as ex:  # noqa: BLE001 - a reference only: report why it is absent
        return {"what": what, "error": repr(ex)[:300]}
    out = {"what": what, "ms": round(ms, 4), "TFLOP/s": round(2.0 * M * N * K / ms / 1e9, 1)}
    if ours_ms:
        out["ours_over_vendor_speed"] = round(ms / ours_ms, 3)
    return out


def hbm_copy_probe(steps: int = 10) -> dict:
    """The device-to-device copy rate of this machine (1 GiB, read + write bytes over the time): what
    a bandwidth-bound pass can reach here, beside the published 8 TB/s."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = time_on_stream(lambda: dst.copy_(src), steps, 2)
    del src, dst
    return {"what": "1 GiB device copy", "ms": round(ms, 4), "GB/s": round(2 * (1 << 30) / ms / 1e6, 1)}


def run_copy(steps: int):
    """Plain 1 GiB device copy: the calibration kernel for the HBM byte counters."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = time_on_stream(lambda: dst.copy_(src), steps, 2)
    print(json.dumps({"copy_bytes": 1 << 30, "ms_per_copy": ms, "GB/s_read+write": 2 * (1 << 30) / ms / 1e6}))


def run_fp8codec(steps: int, warmup: int):
    """FP8 (E4M3) gradient codec on a gradient the size of the 7B gate+up weight (4096 x 22016
    bf16, seeded Student-t(3) x 1e-4): quantize (amax pass + encode pass; X read twice) and
    dequantize to bf16.  HBM-bound: algorithmic bytes / time against 8 TB/s."""
    n = 4096 * 22016
    rng = np.random.default_rng(20250128)
    g = torch.from_numpy((rng.standard_t(3, n) * 1e-4).astype(np.float32)).to(torch.bfloat16).to("cuda")
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    scale = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(fp4.lib().fp4_fp8_workspace_bytes(), dtype=torch.uint8, device="cuda")
    y = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    st = fp4._stream(g)
    q = lambda: fp4.lib().fp4_fp8_quantize(fp4._ptr(g), fp4.FP4_BF16, n, fp4._ptr(codes), fp4._ptr(scale),  # noqa
                                           fp4._ptr(ws), ws.numel(), st)
    d = lambda: fp4.lib().fp4_fp8_dequantize(fp4._ptr(codes), n, fp4._ptr(scale), fp4._ptr(y), fp4.FP4_BF16, st)  # noqa
    ms_q = time_on_stream(q, steps, warmup)
    ms_d = time_on_stream(d, steps, warmup)
    bq, bd = 2 * n * 2 + n, n + n * 2
    print(json.dumps({
        "metric": "FP8 gradient codec GB/s", "workload": "gradient of llama7b gate+up weight, 4096x22016 bf16",
        "quantize": {"ms": round(ms_q, 4), "algorithmic_bytes": bq, "GB/s": round(bq / ms_q / 1e6, 1),
                     "frac_of_hbm_peak": round(bq / ms_q / 1e6 / PEAK_HBM_GBS, 4)},
        "dequantize": {"ms": round(ms_d, 4), "algorithmic_bytes": bd, "GB/s": round(bd / ms_d / 1e6, 1),
                       "frac_of_hbm_peak": round(bd / ms_d / 1e6 / PEAK_HBM_GBS, 4)}}))


def bwd_quantizer_bytes(M, K, N, bi) -> int:
    """Algorithmic HBM bytes of the backward's operand preparation: dY read twice (a column's
    maximum of H = sA * dY must be known before any of its codes; the first read also gives
    G = dY * sW its row maxima and codes), the codes and scales of G and H written, and the
    forward's codes read and written transposed."""
    reads = 2 * M * N * bi + 4 * N + 4 * M
    writes = M * N // 2 + 4 * M + M * N // 2 + 4 * N
    return reads + writes + K * N + M * K


def run_backward(args):
    """Straight-through backward of one layer: dA = dY . deq(Wq)^T and dW = deq(Aq)^T . dY,
    both on the FP4 GEMM (fp4_linear_backward), on the forward's codes of the same seeded
    workload and a seeded dY."""
    from workloads import make_grad
    A, W, L = make_layer(args.workload, 0)
    dev = torch.device("cuda:0")
    Ad, Wd, dYd = A.to(dev), W.to(dev), make_grad(args.workload, 0).to(dev)
    M, K, N = L.M, L.K, L.N
    ws_f = fp4.workspace(Ad, N, L.q)
    fp4.linear_forward(Ad, Wd, L.q, ws=ws_f)
    it = fp4.forward_intermediates(ws_f, M, K, N, A.dtype, L.q)
    lay = fp4.backward_layout(M, K, N)
    ws = torch.empty(lay.total, dtype=torch.uint8, device=dev)
    odt = dYd.dtype
    dA = torch.empty((M, K), dtype=odt, device=dev)
    dW = torch.empty((K, N), dtype=odt, device=dev)
    st = fp4._stream(dYd)
    step = lambda: fp4.linear_backward(dYd, it["Aq"], it["sA"], it["Wq"], it["sW"], K, ws=ws, dA=dA, dW=dW)  # noqa
    ms_step = time_on_stream(step, args.steps, args.warmup)
    P = lambda off: C.c_void_p(ws.data_ptr() + off)  # noqa: E731
    ga = lambda: fp4.lib().fp4_gemm(P(lay.Gq), P(lay.sG), P(lay.WqT), P(lay.ones), M, K, N, None, None, None, 0,  # noqa
                                    None, fp4.FP4_BF16, fp4._ptr(dA), fp4._dt(dA), None, None, 0, st)
    gw = lambda: fp4.lib().fp4_gemm(P(lay.AqT), P(lay.ones), P(lay.Hq), P(lay.sH), K, N, M, None, None, None, 0,  # noqa
                                    None, fp4.FP4_BF16, fp4._ptr(dW), fp4._dt(dW), None, None, 0, st)
    ms_a = time_on_stream(ga, args.steps, 2)
    ms_w = time_on_stream(gw, args.steps, 2)
    flops = 2 * L.flops
    q_ms = max(ms_step - ms_a - ms_w, 1e-9)
    qb = bwd_quantizer_bytes(M, K, N, b_in(A.dtype))
    g_tf = flops / (ms_a + ms_w) / 1e9
    print(json.dumps({
        "metric": "FP4 quantized-linear backward TFLOPS (dA and dW, straight-through)",
        "value": round(flops / ms_step / 1e9, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "dtype": "fp4e2m1 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": L.name + "_backward", "M": M, "K": K, "N": N, "in_dtype": L.dtype,
                   "out_dtype": L.dtype, "grad_std": 1e-3},
        "roofline": {"bound": "mfma", "kernel": {"dA": gemm_kernel(M, K, N), "dW": gemm_kernel(K, N, M)},
                     "achieved": round(g_tf, 1), "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(g_tf / PEAK_FP4_TFLOPS, 4),
                     "ms_dA": round(ms_a, 4), "ms_dW": round(ms_w, 4)},
        "operand_prep": {"bound": "hbm", "ms": round(q_ms, 4), "algorithmic_bytes": qb,
                         "achieved": round(qb / q_ms / 1e6, 1), "unit": "GB/s",
                         "frac": round(qb / q_ms / 1e6 / PEAK_HBM_GBS, 4)},
        "device": torch.cuda.get_device_properties(0).gcnArchName}))


def _rocm_version() -> str | None:
    try:
        return open("/opt/rocm/.info/version").read().strip()
    except OSError:
        return None


def _smi_clocks() -> str | None:
    """The current clock levels as rocm-smi reports them (after the timed work), or None."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    lines = [ln.strip() for ln in r.stdout.splitlines() if "clk" in ln.lower() and "(" in ln]
    return "; ".join(lines[:6]) or None


def _pct(xs, p):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), p))


def per_step_times(fn, steps: int, warmup: int, nsets: int):
    """fn(set_index) `steps` times after `warmup` untimed calls, input sets rotated when nsets > 1,
    with a HIP event on the current stream between consecutive steps.  The timed region is
    bracketed by device synchronizations.  Returns (per-step ms list, total ms, wall s)."""
    s = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i % nsets)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    w0 = time.perf_counter()
    ev[0].record(s)
    for i in range(steps):
        fn(i % nsets)
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)], ev[0].elapsed_time(ev[steps]), wall


def _spread(ts: list) -> dict:
    return {"mean": round(sum(ts) / len(ts), 4), "p10": round(_pct(ts, 10), 4), "p50": round(_pct(ts, 50), 4),
            "p90": round(_pct(ts, 90), 4), "n": len(ts)}


def run_full(args):
    """The whole forward, per layer of the workload, over inputs resident in HBM: cold-cache
    steps (two input sets rotated, together larger than the 256 MB memory-side cache) are the
    primary number; hot-cache steps (one set) and the per-stage breakdown follow."""
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    nsets = 1 if args.hot_only else 2
    sets, host0 = [], []
    for r in range(nsets):
        layers = []
        for li in range(len(wl.layers)):
            A, W, L = make_layer(args.workload, li, replica=r)
            if r == 0:
                host0.append((A, W, L))
            Ad, Wd = A.to(dev), W.to(dev)
            ydt = torch.bfloat16 if L.out_dtype == "bf16" else torch.float32
            layers.append(dict(A=Ad, W=Wd, L=L, ws=fp4.workspace(Ad, L.N, L.q, ydt),
                               Y=torch.empty((L.M, L.N), dtype=ydt, device=dev)))
            if args.wq != "per-step":
                layers[-1]["Wq"], layers[-1]["sW"] = fp4.quantize_weights(Wd)
        sets.append(layers)
    torch.cuda.synchronize()
    main_s = torch.cuda.current_stream()
    side = torch.cuda.Stream(device=dev)  # default priority

    def forward(si: int):
        layers = sets[si]
        if args.wq == "per-step":
            for d in layers:
                fp4.linear_forward(d["A"], d["W"], d["L"].q, ws=d["ws"], Y=d["Y"])
        elif args.wq == "cached":
            for d in layers:
                fp4.linear_forward_wq(d["A"], d["W"], d["Wq"], d["sW"], d["L"].q, ws=d["ws"], Y=d["Y"])
        else:  # overlap: every layer's W quantized on a second stream, each forward waits for its own
            side.wait_stream(main_s)
            ready = []
            with torch.cuda.stream(side):
                for d in layers:
                    fp4._check(fp4.lib().fp4_quantize(fp4._ptr(d["W"]), fp4._dt(d["W"]), d["L"].K, d["L"].N,
                                                      fp4.FP4_PER_COL, None, fp4._ptr(d["Wq"]), fp4._ptr(d["sW"]),
                                                      fp4._stream(d["W"])))
                    ev = torch.cuda.Event()
                    ev.record(side)
                    ready.append(ev)
            for d, ev in zip(layers, ready):
                main_s.wait_event(ev)
                fp4.linear_forward_wq(d["A"], d["W"], d["Wq"], d["sW"], d["L"].q, ws=d["ws"], Y=d["Y"])

    flops = sum(d["L"].flops for d in sets[0])
    cold, cold_total, wall = per_step_times(forward, args.steps, args.warmup, nsets)
    ms_step = cold_total / args.steps
    if args.mode == "forward":
        print(json.dumps({"ms_per_step": ms_step}))
        return
    hot, hot_total, _ = per_step_times(forward, args.steps, args.warmup, 1)

    # the stages of the forward, each between events of its own (hot cache, set 0): the
    # quantizer as the forward calls it (A and W in one call, whose W passes share launches
    # with the A side's), then the product (GEMM + compensation + escape kernel); with cached
    # weight codes the whole cached-weight forward is the second stage (not split)
    def stage_times(parts):
        recs = []

        def step(_si: int):
            rec = []
            for d in sets[0]:
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
                ev[0].record(main_s)
                for k, f in enumerate(parts):
                    f(d)
                    ev[k + 1].record(main_s)
                rec.append(ev)
            recs.append(rec)
        per_step_times(step, args.steps, args.warmup, 1)
        return [float(np.median([sum(ev[k].elapsed_time(ev[k + 1]) for ev in rec) for rec in recs[args.warmup:]]))
                for k in range(len(parts))]

    def q_call(stages):
        return lambda d: fp4.forward_quantize(d["A"] if stages & fp4.FP4_STAGE_A else None,
                                              d["W"] if stages & fp4.FP4_STAGE_W else None, d["L"].M, d["L"].K,
                                              d["L"].N, d["A"].dtype, d["L"].q, d["ws"], stages=stages)
    per_step_w = args.wq == "per-step"
    if per_step_w:
        second = lambda d: fp4.forward_product(d["W"], d["L"].M, d["L"].q, d["ws"], d["Y"])  # noqa: E731
    else:
        second = lambda d: fp4.linear_forward_wq(d["A"], d["W"], d["Wq"], d["sW"], d["L"].q,  # noqa: E731
                                                 ws=d["ws"], Y=d["Y"])
    quant_ms, product_ms = stage_times([q_call(fp4.FP4_STAGE_A | (fp4.FP4_STAGE_W if per_step_w else 0)), second])
    # each side of the quantizer in a call of its own (its own launches), for the split
    quant_a_ms, quant_w_ms = stage_times([q_call(fp4.FP4_STAGE_A), q_call(fp4.FP4_STAGE_W)]) if per_step_w \
        else (quant_ms, None)

    # the dominant kernel alone, as the forward launches it: the GEMM with the two-byte
    # accumulator hand-over (FP4_Q16) and its escape kernel (which finds no block to redo here)
    gemm_ms, nnz_total, qa_bytes, qw_bytes, cbytes = 0.0, 0, 0, 0, 0
    per_layer = []
    for d in sets[0]:
        L, Ad, Wd, ws, Y = d["L"], d["A"], d["W"], d["ws"], d["Y"]
        it = fp4.forward_intermediates(ws, L.M, L.K, L.N, Ad.dtype, L.q)
        nnz = int(it["nnz"].item())
        qb = fp4.lib().fp4_gemm_workspace_bytes(L.M, L.N, fp4.FP4_Q16, 0)
        hand = torch.empty(qb, dtype=torch.uint8, device=dev)
        yq = torch.empty((L.M, L.N), dtype=torch.int16, device=dev)
        g = lambda: fp4.lib().fp4_gemm(  # noqa: E731
            fp4._ptr(it["Aq"]), fp4._ptr(it["sA"]), fp4._ptr(it["Wq"]), fp4._ptr(it["sW"]), L.M, L.N, L.K, None, None,
            None, 0, None, fp4._dt(Wd), fp4._ptr(yq), fp4.FP4_Q16, None, fp4._ptr(hand), qb, fp4._stream(Ad))
        ms_g = time_on_stream(g, args.steps, 2)
        del hand, yq
        gemm_ms += ms_g
        nnz_total += nnz
        bi = b_in(Ad.dtype)
        qa_bytes += quantizer_bytes(L.M, L.K, L.N, bi, nnz, with_w=False)
        qw_bytes += quantizer_bytes(L.M, L.K, L.N, bi, nnz) - quantizer_bytes(L.M, L.K, L.N, bi, nnz, with_w=False)
        cbytes += comp_bytes(L.M, L.N, Y.element_size(), nnz)
        per_layer.append({"layer": L.name, "M": L.M, "K": L.K, "N": L.N, "q": L.q, "nnz": nnz,
                          "gemm_kernel": gemm_kernel(L.M, L.N, L.K), "gemm_ms": round(ms_g, 4),
                          "gemm_TFLOP/s": round(L.flops / ms_g / 1e9, 1),
                          "comp_kernel": fp4.comp_kernel_name(L.M, fp4.outlier_capacity(L.M, L.K, L.q))})
    if args.wq != "per-step":
        qw_bytes = 0
    comp_ms = max(product_ms - gemm_ms, 1e-9)
    gemm_tflops = flops / gemm_ms / 1e9
    fwd_tflops = flops / ms_step / 1e9
    first = sets[0][0]["L"]
    traffic = load_traffic(None) if args.workload == "llama7b_gate_up" else None
    comp_traffic = load_traffic(None, "comp") if args.workload == "llama7b_gate_up" else None
    quant_traffic = load_traffic(None, "quant") if args.workload == "llama7b_gate_up" and per_step_w else None
    name = first.name if len(sets[0]) == 1 else f"{args.workload}(x{len(sets[0])} layers)"
    sha = hashlib.sha256()
    for A, W, _ in host0:
        sha.update(A.contiguous().view(torch.uint8).numpy().tobytes() if A.dtype != torch.bfloat16
                   else A.contiguous().view(torch.int16).numpy().tobytes())
        sha.update(W.contiguous().view(torch.int16).numpy().tobytes() if W.dtype == torch.bfloat16
                   else W.contiguous().numpy().tobytes())
    hbm = lambda b, ms: {"achieved": round(b / ms / 1e6, 1), "frac": round(b / ms / 1e6 / PEAK_HBM_GBS, 4),  # noqa
                         "ms": round(ms, 4), "algorithmic_bytes": b}
    out = {
        "metric": METRIC,
        "value": round(fwd_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4e2m1 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": name, "M": first.M, "K": first.K, "N": first.N, "in_dtype": first.dtype,
                   "out_dtype": first.out_dtype, "q": first.q, "layers": len(sets[0]), "w_quant": args.wq,
                   "parallelism": "none (1 GPU)"},
        "timing": {"primary": "cold" if nsets == 2 else "hot",
                   "cold": dict(_spread(cold), what="two seeded input sets rotated step by step (inputs not "
                                                     "cache-resident); value and ms_per_step are this mean"),
                   "hot": dict(_spread(hot), what="one input set repeated"),
                   "hot_TFLOP/s": round(flops / (hot_total / args.steps) / 1e9, 2)},
        "forward_frac_of_fp4_peak": round(fwd_tflops / PEAK_FP4_TFLOPS, 4),
        # the product stage (GEMM, compensation and escape scan): 2MNK over its own time
        "product_stage_frac_of_fp4_peak": round(flops / product_ms / 1e9 / PEAK_FP4_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": gemm_kernel(first.M, first.N, first.K), "achieved": round(gemm_tflops, 1),
                     "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP4_TFLOPS, 4),
                     "traffic": traffic, "ms_per_launch": round(gemm_ms, 4)},
        "stages_hot_ms": {"quantizer": round(quant_ms, 4), "product": round(product_ms, 4), "gemm": round(gemm_ms, 4),
                          "quant_A_alone": round(quant_a_ms, 4),
                          "quant_W_alone": round(quant_w_ms, 4) if quant_w_ms is not None else None},
        "compensation": dict({"bound": "hbm", "kernel": per_layer[0]["comp_kernel"], "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "how": "product stage minus the GEMM launch, both timed directly",
                              # counted HBM bytes of one k_comp_apply launch (rocprofv3 FETCH_SIZE +
                              # WRITE_SIZE, scaled by a plain copy's counts), and that over its time
                              "traffic": comp_traffic,
                              "traffic_GB/s": round(comp_traffic / comp_ms / 1e6, 1) if comp_traffic else None},
                             **hbm(cbytes, comp_ms)),
        "quantizer": dict({"bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "how": "the forward's quantizer stage call (A and W in one call, its own launches), "
                                  "between events of its own; A_alone / W_alone: each side in a call of its own",
                           "A_alone": hbm(qa_bytes, quant_a_ms),
                           "W_alone": hbm(qw_bytes, quant_w_ms) if qw_bytes else None,
                           # counted HBM bytes of the stage call's launches (W read twice), and over its time
                           "traffic": quant_traffic,
                           "traffic_GB/s": round(quant_traffic / quant_ms / 1e6, 1) if quant_traffic else None},
                          **hbm(qa_bytes + qw_bytes, quant_ms)),
        "nnz": nnz_total,
        "layers": per_layer,
        "wall_s_timed": round(wall, 3),
        "env": {"device": torch.cuda.get_device_properties(0).gcnArchName, "rocm": _rocm_version(),
                "torch": torch.__version__, "input_sha256": sha.hexdigest(), "smi_clocks_after": _smi_clocks()},
    }
    if not args.no_probe:
        out["mfma_probe"] = mfma_probe()
        out["hbm_copy"] = hbm_copy_probe()
        # each bound against what this machine sustains (the probes) besides the published peaks
        out["roofline"]["frac_of_probe_peak"] = round(gemm_tflops / out["mfma_probe"]["TFLOP/s"], 4)
        cp = out["hbm_copy"]["GB/s"]
        for k in ("compensation", "quantizer"):
            out[k]["frac_of_copy_rate"] = round(out[k]["achieved"] / cp, 4)
        L0 = sets[0][0]["L"]
        out["vendor_gemm"] = vendor_gemm(L0.M, L0.N, L0.K, gemm_ms if len(sets[0]) == 1 else None)
    if args.emu:
        emu_ms = nat_ms = 0.0
        for d in sets[0]:
            L, Ad, Wd, ws, Y = d["L"], d["A"], d["W"], d["ws"], d["Y"]
            it = fp4.forward_intermediates(ws, L.M, L.K, L.N, Ad.dtype, L.q)
            common = (fp4._ptr(it["Aq"]), fp4._ptr(it["sA"]), fp4._ptr(it["Wq"]), fp4._ptr(it["sW"]), L.M, L.N, L.K)
            ews = torch.empty(fp4.lib().fp4_gemm_fp8emu_workspace_bytes(L.M, L.N, L.K), dtype=torch.uint8, device=dev)
            emu = lambda: fp4.lib().fp4_gemm_fp8emu(  # noqa: E731
                *common, fp4._ptr(Y), fp4._dt(Y), None, fp4._ptr(ews), ews.numel(), fp4._stream(Ad))
            nat = lambda: fp4.lib().fp4_gemm(  # noqa: E731
                *common, None, None, None, 0, None, fp4._dt(Wd), fp4._ptr(Y), fp4._dt(Y), None, None, 0,
                fp4._stream(Ad))
            emu_ms += time_on_stream(emu, args.steps, 2)
            nat_ms += time_on_stream(nat, args.steps, 2)
            del ews
        out["fp8_emulation"] = {
            "what": "E2M1 codes expanded to E4M3 bytes, product on the FP8 MFMA (the pages' execution mode); "
                    "native = the FP4 MFMA on the same codes; both without the dA term",
            "emulated_ms": round(emu_ms, 4), "native_ms": round(nat_ms, 4),
            "emulated_TFLOP/s": round(flops / emu_ms / 1e9, 1), "native_TFLOP/s": round(flops / nat_ms / 1e9, 1),
            "emulated_frac_of_fp8_peak": round(flops / emu_ms / 1e9 / PEAK_FP8_TFLOPS, 4),
            "speedup_native": round(emu_ms / nat_ms, 3)}
    if not args.no_cpu_baseline:
        A, W, L = host0[0]
        out["cpu_baseline"] = cpu_baseline(A, W, L)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b_gate_up", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the matrix-core issue-rate probe and the vendor GEMM reference")
    ap.add_argument("--hot-only", action="store_true", help="one input set only (no cold-cache rotation)")
    ap.add_argument("--emu", action="store_true",
                    help="also time the FP4-on-FP8 emulation of the product (E4M3 expansion + FP8 MFMA) against "
                         "the native FP4 product on the same codes, both without the dA term")
    ap.add_argument("--wq", default="per-step", choices=["per-step", "cached", "overlap"],
                    help="W quantization: inside every forward (the pages' scheme, default); once before the "
                         "timed steps (fixed inference weights); or on a second stream, each layer's under the "
                         "previous layer's forward")
    ap.add_argument("--mode", default="full", choices=["full", "copy", "forward", "traffic", "fp8codec",
                                                          "backward", "mfma-peak", "vendor-gemm"])
    ap.add_argument("--traffic-dirs", nargs=4, metavar=("GEMM_FETCH", "GEMM_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="--mode traffic: rocprofv3 --pmc output directories of FETCH_SIZE and WRITE_SIZE for "
                         "the full bench and for --mode copy")
    args = ap.parse_args()
    if args.mode == "traffic":
        write_traffic(*args.traffic_dirs)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): this forward is built and "
              "measured on a single GPU; sharding it over several is a design note, not a run.", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.mode == "copy":
        run_copy(args.steps)
        return
    if args.mode == "fp8codec":
        run_fp8codec(args.steps, args.warmup)
        return
    if args.mode == "mfma-peak":
        print(json.dumps(mfma_probe()))
        return
    if args.mode == "vendor-gemm":
        L = WORKLOADS[args.workload].layers[0]
        print(json.dumps(vendor_gemm(L.M, L.N, L.K)))
        return
    if args.mode == "backward":
        run_backward(args)
        return
    run_full(args)


if __name__ == "__main__":
    main()
