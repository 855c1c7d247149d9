"""MI355X (gfx950) FP4 quantized linear-layer forward: Python binding of libfp4lin.so.

Argument marshalling only: torch supplies device memory and the current HIP stream,
and every step of the forward runs in the library's HIP kernels (include/fp4lin.h is
the ABI).  There is no CPU fallback: without the built library every call raises.

    Y = linear_forward(A, W, q)            # A: M x K, W: K x N (cuda, bf16 or fp32)

The method (quantization of A per token and W per output channel into E2M1, outlier
clamping at a quantile of |A| with sparse compensation dA) follows the pages on
"Optimizing Large Language Model Training Using FP4 Quantization" (QbitAI report:
granularity, forward-quantization and outlier paragraphs).
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4lin.so")

FP4_F32, FP4_BF16 = 0, 1
FP4_Q16 = 2  # fp4_gemm output only: int16 4*acc with fp32 escapes in the workspace
FP4_PER_ROW, FP4_PER_COL = 0, 1
FP4_STAGE_A, FP4_STAGE_W = 1, 2

EXPORTS = (
    "fp4_quantize", "fp4_outlier_capacity", "fp4_outlier_workspace_bytes", "fp4_outlier_clamp",
    "fp4_outlier_clamp_noalloc",
    "fp4_gemm_workspace_bytes", "fp4_gemm", "fp4_forward_layout", "fp4_forward_workspace_bytes", "fp4_linear_forward",
    "fp4_linear_forward_wq", "fp4_forward_quantize", "fp4_forward_product", "fp4_gemm_fp8emu_workspace_bytes", "fp4_gemm_fp8emu",
    "fp4_fp8_workspace_bytes", "fp4_fp8_quantize", "fp4_fp8_dequantize",
    "fp4_backward_layout", "fp4_backward_workspace_bytes", "fp4_linear_backward",
    "fp4_gemm_kernel_name", "fp4_comp_kernel_name", "fp4_status_string",
)


class WsLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("total", "T", "nnz", "row_ptr", "coo_row", "coo_col", "coo_val",
                                          "Aq", "sA", "Wq", "sW", "handoff", "scratch")] + [("capacity", C.c_int64)]


class BwdLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("total", "Gq", "sG", "Hq", "sH", "WqT", "AqT", "ones", "part")]


class Fp4Error(RuntimeError):
    pass


_lib = None


def lib():
    """Load libfp4lin.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise Fp4Error(f"{LIB_PATH} is missing: build it with `python -m quantized_linear_layers_fp4_amd.build`")
    L = C.CDLL(LIB_PATH)
    vp, i64, i32, dbl, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_double, C.c_size_t
    sig = {
        "fp4_quantize": (i32, [vp, i32, i64, i64, i32, vp, vp, vp, vp]),
        "fp4_outlier_capacity": (i64, [i64, i64, dbl]),
        "fp4_outlier_workspace_bytes": (sz, [i64, i64, i32, dbl]),
        "fp4_outlier_clamp": (i32, [vp, i32, i64, i64, dbl, vp, vp, vp, vp, i64, vp, vp, vp, sz, vp]),
        "fp4_outlier_clamp_noalloc": (i32, [vp, i32, i64, i64, dbl, vp, vp, vp, vp, i64, vp, vp, vp]),
        "fp4_gemm_workspace_bytes": (sz, [i64, i64, i32, i32]),
        "fp4_gemm": (i32, [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, i64, vp, i32, vp, i32, vp, vp, sz, vp]),
        "fp4_forward_layout": (i32, [i64, i64, i64, i32, i32, dbl, C.POINTER(WsLayout)]),
        "fp4_forward_workspace_bytes": (sz, [i64, i64, i64, i32, i32, dbl]),
        "fp4_linear_forward": (i32, [vp, vp, i32, i64, i64, i64, dbl, vp, i32, vp, sz, vp]),
        "fp4_linear_forward_wq": (i32, [vp, vp, vp, vp, i32, i64, i64, i64, dbl, vp, i32, vp, sz, vp]),
        "fp4_forward_quantize": (i32, [vp, vp, i32, i64, i64, i64, dbl, i32, vp, sz, vp]),
        "fp4_forward_product": (i32, [vp, i32, i64, i64, i64, dbl, vp, i32, vp, sz, vp]),
        "fp4_gemm_fp8emu_workspace_bytes": (sz, [i64, i64, i64]),
        "fp4_fp8_workspace_bytes": (sz, []),
        "fp4_fp8_quantize": (i32, [vp, i32, i64, vp, vp, vp, sz, vp]),
        "fp4_fp8_dequantize": (i32, [vp, i64, vp, vp, i32, vp]),
        "fp4_gemm_fp8emu": (i32, [vp, vp, vp, vp, i64, i64, i64, vp, i32, vp, vp, sz, vp]),
        "fp4_backward_layout": (i32, [i64, i64, i64, C.POINTER(BwdLayout)]),
        "fp4_backward_workspace_bytes": (sz, [i64, i64, i64]),
        "fp4_linear_backward": (i32, [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, i32, vp, sz, vp]),
        "fp4_gemm_kernel_name": (C.c_char_p, [i64, i64, i64, i32]),
        "fp4_comp_kernel_name": (C.c_char_p, [i64, i64]),
        "fp4_status_string": (C.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise Fp4Error(f"fp4 status {status}: {lib().fp4_status_string(status).decode()}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FP4_BF16
    if t.dtype == torch.float32:
        return FP4_F32
    raise TypeError(f"expected bfloat16 or float32, got {t.dtype}")


def _ptr(t: torch.Tensor | None):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on a HIP device")


def _out_dtype_code(d: torch.dtype) -> int:
    return {torch.bfloat16: FP4_BF16, torch.float32: FP4_F32}[d]


# --------------------------------------------------------------------------- calls
def quantize(X: torch.Tensor, axis: int = FP4_PER_ROW, clamp_T: torch.Tensor | None = None):
    """E2M1 codes and fp32 scales of X (R x C).  PER_ROW: codes R x C/2, scales R.
    PER_COL: codes C x R/2 (transposed), scales C."""
    _need_cuda(X, clamp_T)
    R, Cn = X.shape
    if axis == FP4_PER_ROW:
        codes = torch.empty((R, Cn // 2), dtype=torch.uint8, device=X.device)
        scales = torch.empty(R, dtype=torch.float32, device=X.device)
    else:
        codes = torch.empty((Cn, R // 2), dtype=torch.uint8, device=X.device)
        scales = torch.empty(Cn, dtype=torch.float32, device=X.device)
    _check(lib().fp4_quantize(_ptr(X), _dt(X), R, Cn, axis, _ptr(clamp_T), _ptr(codes), _ptr(scales), _stream(X)))
    return codes, scales


def gemm_kernel_name(M: int, N: int, K: int, num_cus: int) -> str:
    """The FP4 GEMM kernel the library launches for an M x N x K product on num_cus CUs."""
    r = lib().fp4_gemm_kernel_name(M, N, K, num_cus)
    if r is None:
        raise Fp4Error(f"no GEMM kernel for M={M} N={N} K={K} on {num_cus} CUs")
    return r.decode()


def comp_kernel_name(M: int, capacity: int) -> str:
    """The compensation kernel the library launches for M rows and a dA list of `capacity`."""
    r = lib().fp4_comp_kernel_name(M, capacity)
    if r is None:
        raise Fp4Error(f"no compensation kernel for M={M} capacity={capacity}")
    return r.decode()


def outlier_capacity(M: int, K: int, q: float) -> int:
    return int(lib().fp4_outlier_capacity(M, K, float(q)))


def outlier_clamp(A: torch.Tensor, q: float, trim: bool = True) -> dict:
    """Threshold T and the COO list of dA for A (M x K).  With trim=True the COO arrays
    are cut to nnz (this reads nnz back and synchronizes)."""
    _need_cuda(A)
    M, K = A.shape
    L = lib()
    cap = int(L.fp4_outlier_capacity(M, K, float(q)))
    if cap < 0:
        _check(2)
    dev = A.device
    capn = max(cap, 1)
    T = torch.empty(4, dtype=torch.float32, device=dev)
    coo_row = torch.empty(capn, dtype=torch.int32, device=dev)
    coo_col = torch.empty(capn, dtype=torch.int32, device=dev)
    coo_val = torch.empty(capn, dtype=torch.float32, device=dev)
    row_ptr = torch.empty(M + 1, dtype=torch.int32, device=dev)
    nnz = torch.empty(2, dtype=torch.int64, device=dev)
    wsb = int(L.fp4_outlier_workspace_bytes(M, K, _dt(A), float(q)))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _check(L.fp4_outlier_clamp(_ptr(A), _dt(A), M, K, float(q), _ptr(T), _ptr(coo_row), _ptr(coo_col),
                               _ptr(coo_val), capn, _ptr(row_ptr), _ptr(nnz), _ptr(ws), wsb, _stream(A)))
    out = dict(T=T[:1], row_ptr=row_ptr, nnz=nnz[:1], coo_row=coo_row, coo_col=coo_col, coo_val=coo_val)
    if trim:
        n = int(nnz[0].item())
        out.update(coo_row=coo_row[:n], coo_col=coo_col[:n], coo_val=coo_val[:n])
    return out


def gemm(Aq: torch.Tensor, sA: torch.Tensor, Wq: torch.Tensor, sW: torch.Tensor, K: int,
         row_ptr: torch.Tensor | None = None, coo_col: torch.Tensor | None = None,
         coo_val: torch.Tensor | None = None, W: torch.Tensor | None = None,
         out_dtype: torch.dtype = torch.bfloat16, acc_out: bool = False, ws: torch.Tensor | None = None,
         capacity: int | None = None):
    """Y = fl(fl(acc * sA) * sW) (+ dA . W when row_ptr, coo_col, coo_val and W are given)."""
    _need_cuda(Aq, sA, Wq, sW, row_ptr, coo_col, coo_val, W, ws)
    M, N = Aq.shape[0], Wq.shape[0]
    Y = torch.empty((M, N), dtype=out_dtype, device=Aq.device)
    acc = torch.empty((M, N), dtype=torch.float32, device=Aq.device) if acc_out else None
    wdt = _dt(W) if W is not None else FP4_BF16
    with_comp = int(row_ptr is not None and coo_col is not None and coo_val is not None)
    if ws is None:
        nbytes = lib().fp4_gemm_workspace_bytes(M, N, _out_dtype_code(out_dtype), with_comp)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=Aq.device) if nbytes else None
    cap = capacity if capacity is not None else (coo_col.numel() if coo_col is not None else 0)
    _check(lib().fp4_gemm(_ptr(Aq), _ptr(sA), _ptr(Wq), _ptr(sW), M, N, K, _ptr(row_ptr), _ptr(coo_col),
                          _ptr(coo_val), cap, _ptr(W), wdt, _ptr(Y), _out_dtype_code(out_dtype), _ptr(acc), _ptr(ws),
                          ws.numel() if ws is not None else 0, _stream(Aq)))
    return (Y, acc) if acc_out else Y


def gemm_q16(Aq: torch.Tensor, sA: torch.Tensor, Wq: torch.Tensor, sW: torch.Tensor, K: int,
             acc_out: bool = False):
    """The exact accumulator in two bytes (FP4_Q16): (Yq int16 M x N, esc fp32 M x N), where
    Yq = 4*acc, except in the escaped 128 x 64 blocks (those around some |acc| > 8191.75):
    there Yq = -32768 and esc = fl(fl(acc*sA)*sW)."""
    _need_cuda(Aq, sA, Wq, sW)
    M, N = Aq.shape[0], Wq.shape[0]
    Yq = torch.empty((M, N), dtype=torch.int16, device=Aq.device)
    acc = torch.empty((M, N), dtype=torch.float32, device=Aq.device) if acc_out else None
    nbytes = lib().fp4_gemm_workspace_bytes(M, N, FP4_Q16, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=Aq.device)
    _check(lib().fp4_gemm(_ptr(Aq), _ptr(sA), _ptr(Wq), _ptr(sW), M, N, K, None, None, None, 0, None, FP4_BF16,
                          _ptr(Yq), FP4_Q16, _ptr(acc), _ptr(ws), nbytes, _stream(Aq)))
    esc = ws[:M * N * 4].view(torch.float32).view(M, N)  # the escape values come first in the workspace
    return (Yq, esc, acc) if acc_out else (Yq, esc)


def gemm_fp8emu(Aq: torch.Tensor, sA: torch.Tensor, Wq: torch.Tensor, sW: torch.Tensor, K: int,
                out_dtype: torch.dtype = torch.bfloat16, acc_out: bool = False, ws: torch.Tensor | None = None):
    """The product on E4M3 matrix cores after an exact E2M1 -> E4M3 expansion (no dA term)."""
    _need_cuda(Aq, sA, Wq, sW, ws)
    M, N = Aq.shape[0], Wq.shape[0]
    Y = torch.empty((M, N), dtype=out_dtype, device=Aq.device)
    acc = torch.empty((M, N), dtype=torch.float32, device=Aq.device) if acc_out else None
    if ws is None:
        nbytes = lib().fp4_gemm_fp8emu_workspace_bytes(M, N, K)
        if nbytes == 0:
            raise Fp4Error("shape out of range for the FP8 emulation")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=Aq.device)
    _check(lib().fp4_gemm_fp8emu(_ptr(Aq), _ptr(sA), _ptr(Wq), _ptr(sW), M, N, K, _ptr(Y), _out_dtype_code(out_dtype),
                                 _ptr(acc), _ptr(ws), ws.numel(), _stream(Aq)))
    return (Y, acc) if acc_out else Y


def fp8_quantize(X: torch.Tensor):
    """FP8 (E4M3) gradient codec: (codes u8[n], scale fp32[1]) with one per-tensor scale."""
    _need_cuda(X)
    n = X.numel()
    codes = torch.empty(n, dtype=torch.uint8, device=X.device)
    scale = torch.empty(1, dtype=torch.float32, device=X.device)
    ws = torch.empty(lib().fp4_fp8_workspace_bytes(), dtype=torch.uint8, device=X.device)
    _check(lib().fp4_fp8_quantize(_ptr(X), _dt(X), n, _ptr(codes), _ptr(scale), _ptr(ws), ws.numel(), _stream(X)))
    return codes, scale


def fp8_dequantize(codes: torch.Tensor, scale: torch.Tensor, out_dtype: torch.dtype = torch.float32):
    _need_cuda(codes, scale)
    Y = torch.empty(codes.numel(), dtype=out_dtype, device=codes.device)
    _check(lib().fp4_fp8_dequantize(_ptr(codes), codes.numel(), _ptr(scale), _ptr(Y), _out_dtype_code(out_dtype),
                                    _stream(codes)))
    return Y


def forward_layout(M: int, K: int, N: int, dtype: torch.dtype, q: float,
                   out_dtype: torch.dtype | None = None) -> WsLayout:
    """The forward workspace's layout for inputs of dtype and Y of out_dtype (default: dtype)."""
    lay = WsLayout()
    _check(lib().fp4_forward_layout(M, K, N, _out_dtype_code(dtype), _out_dtype_code(out_dtype or dtype), float(q),
                                    C.byref(lay)))
    return lay


def workspace(A: torch.Tensor, N: int, q: float, out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """A workspace tensor sized for linear_forward(A, W (K x N), q, out_dtype)."""
    M, K = A.shape
    lay = forward_layout(M, K, N, A.dtype, q, out_dtype)
    return torch.empty(lay.total, dtype=torch.uint8, device=A.device)


def linear_forward(A: torch.Tensor, W: torch.Tensor, q: float, out_dtype: torch.dtype | None = None,
                   ws: torch.Tensor | None = None, Y: torch.Tensor | None = None) -> torch.Tensor:
    """FP4 linear forward Y = dequant(Aq . Wq) + dA . W on the current stream."""
    _need_cuda(A, W, ws, Y)
    if A.dtype != W.dtype:
        raise TypeError("A and W must share a dtype")
    M, K = A.shape
    N = W.shape[1]
    out_dtype = out_dtype or A.dtype
    if ws is None:
        ws = workspace(A, N, q, out_dtype)
    if Y is None:
        Y = torch.empty((M, N), dtype=out_dtype, device=A.device)
    _check(lib().fp4_linear_forward(_ptr(A), _ptr(W), _dt(A), M, K, N, float(q), _ptr(Y), _dt(Y), _ptr(ws),
                                    ws.numel(), _stream(A)))
    return Y


def forward_quantize(A: torch.Tensor | None, W: torch.Tensor | None, M: int, K: int, N: int, dtype: torch.dtype,
                     q: float, ws: torch.Tensor, stages: int = FP4_STAGE_A | FP4_STAGE_W):
    """The forward's quantizer stages (FP4_STAGE_A and/or FP4_STAGE_W) into the workspace."""
    _need_cuda(A, W, ws)
    dt = FP4_BF16 if dtype == torch.bfloat16 else FP4_F32
    ref = A if A is not None else W
    _check(lib().fp4_forward_quantize(_ptr(A), _ptr(W), dt, M, K, N, float(q), stages, _ptr(ws), ws.numel(),
                                      _stream(ref)))


def forward_product(W: torch.Tensor, M: int, q: float, ws: torch.Tensor, Y: torch.Tensor):
    """The forward's product stage (GEMM, dequantization, compensation) from the workspace."""
    _need_cuda(W, ws, Y)
    K, N = W.shape
    _check(lib().fp4_forward_product(_ptr(W), _dt(W), M, K, N, float(q), _ptr(Y), _dt(Y), _ptr(ws), ws.numel(),
                                     _stream(W)))
    return Y


def quantize_weights(W: torch.Tensor):
    """(Wq, sW) of a K x N weight matrix: per-output-channel codes (N x K/2) and scales."""
    _need_cuda(W)
    K, N = W.shape
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    sW = torch.empty(N, dtype=torch.float32, device=W.device)
    _check(lib().fp4_quantize(_ptr(W), _dt(W), K, N, FP4_PER_COL, None, _ptr(Wq), _ptr(sW), _stream(W)))
    return Wq, sW


def linear_forward_wq(A: torch.Tensor, W: torch.Tensor, Wq: torch.Tensor, sW: torch.Tensor, q: float,
                      out_dtype: torch.dtype | None = None, ws: torch.Tensor | None = None,
                      Y: torch.Tensor | None = None) -> torch.Tensor:
    """The forward with W's codes and scales from quantize_weights(W) (W unchanged since)."""
    _need_cuda(A, W, Wq, sW, ws, Y)
    if A.dtype != W.dtype:
        raise TypeError("A and W must share a dtype")
    M, K = A.shape
    N = W.shape[1]
    out_dtype = out_dtype or A.dtype
    if ws is None:
        ws = workspace(A, N, q, out_dtype)
    if Y is None:
        Y = torch.empty((M, N), dtype=out_dtype, device=A.device)
    _check(lib().fp4_linear_forward_wq(_ptr(A), _ptr(W), _ptr(Wq), _ptr(sW), _dt(A), M, K, N, float(q), _ptr(Y),
                                       _dt(Y), _ptr(ws), ws.numel(), _stream(A)))
    return Y


def forward_intermediates(ws: torch.Tensor, M: int, K: int, N: int, dtype: torch.dtype, q: float) -> dict:
    """Views of T, nnz, the COO list, codes and scales inside a forward workspace."""
    lay = forward_layout(M, K, N, dtype, q)
    cap = max(int(lay.capacity), 1)

    def view(off, count, dt, shape=None):
        nbytes = count * torch.tensor([], dtype=dt).element_size()
        t = ws[off:off + nbytes].view(dt)
        return t.view(shape) if shape else t

    return dict(
        T=view(lay.T, 1, torch.float32), nnz=view(lay.nnz, 1, torch.int64),
        row_ptr=view(lay.row_ptr, M + 1, torch.int32), coo_row=view(lay.coo_row, cap, torch.int32),
        coo_col=view(lay.coo_col, cap, torch.int32), coo_val=view(lay.coo_val, cap, torch.float32),
        Aq=view(lay.Aq, M * (K // 2), torch.uint8, (M, K // 2)), sA=view(lay.sA, M, torch.float32),
        Wq=view(lay.Wq, N * (K // 2), torch.uint8, (N, K // 2)), sW=view(lay.sW, N, torch.float32),
        capacity=int(lay.capacity))


# --------------------------------------------------------------------------- backward
def backward_layout(M: int, K: int, N: int) -> BwdLayout:
    lay = BwdLayout()
    _check(lib().fp4_backward_layout(M, K, N, C.byref(lay)))
    return lay


def linear_backward(dY: torch.Tensor, Aq: torch.Tensor | None, sA: torch.Tensor | None, Wq: torch.Tensor | None,
                    sW: torch.Tensor | None, K: int, want_dA: bool = True, want_dW: bool = True,
                    out_dtype: torch.dtype | None = None, ws: torch.Tensor | None = None,
                    dA: torch.Tensor | None = None, dW: torch.Tensor | None = None):
    """Straight-through backward of the quantized product: (dA, dW), each None when not
    wanted.  Aq/sA/Wq/sW are the forward's codes and scales (forward_intermediates)."""
    _need_cuda(dY, Aq, sA, Wq, sW, ws, dA, dW)
    M, N = dY.shape
    out_dtype = out_dtype or dY.dtype
    if ws is None:
        ws = torch.empty(backward_layout(M, K, N).total, dtype=torch.uint8, device=dY.device)
    if want_dA and dA is None:
        dA = torch.empty((M, K), dtype=out_dtype, device=dY.device)
    if want_dW and dW is None:
        dW = torch.empty((K, N), dtype=out_dtype, device=dY.device)
    dA = dA if want_dA else None
    dW = dW if want_dW else None
    _check(lib().fp4_linear_backward(_ptr(dY), _dt(dY), M, K, N, _ptr(Aq), _ptr(sA), _ptr(Wq), _ptr(sW), _ptr(dA),
                                     _dt(dA) if dA is not None else FP4_F32, _ptr(dW),
                                     _dt(dW) if dW is not None else FP4_F32, _ptr(ws), ws.numel(), _stream(dY)))
    return dA, dW


def backward_intermediates(ws: torch.Tensor, M: int, K: int, N: int) -> dict:
    """Views of Gq, sG, Hq, sH, WqT and AqT inside a backward workspace."""
    lay = backward_layout(M, K, N)

    def view(off, nbytes, dt, shape):
        return ws[off:off + nbytes].view(dt).view(shape)

    return dict(Gq=view(lay.Gq, M * (N // 2), torch.uint8, (M, N // 2)), sG=view(lay.sG, 4 * M, torch.float32, (M,)),
                Hq=view(lay.Hq, N * (M // 2), torch.uint8, (N, M // 2)), sH=view(lay.sH, 4 * N, torch.float32, (N,)),
                WqT=view(lay.WqT, K * (N // 2), torch.uint8, (K, N // 2)),
                AqT=view(lay.AqT, K * (M // 2), torch.uint8, (K, M // 2)))
