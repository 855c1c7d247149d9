"""CPU oracle for the FP4 quantized linear forward (ctypes wrapper over fp4_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` are the only callers.  The product path never imports this
package, and this package never imports the product.

All functions take and return numpy arrays.  bf16 tensors are passed as uint16 arrays
holding the bf16 bit patterns; the C code widens them to fp32 exactly.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "fp4_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

F32, BF16 = 0, 1

_lib = None


class using:
    """Context manager: route every oracle call through another build of the library
    (the planted-mistake tests load deliberately broken copies this way)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def build(src: str = SRC, out: str = LIB, extra: tuple = ()) -> str:
    """Compile the oracle with gcc (no GPU toolchain involved)."""
    cmd = ["gcc", *CFLAGS, *extra, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _p(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def load(path: str = LIB):
    """Load (building if needed) the oracle library and declare its signatures."""
    global _lib
    if path == LIB and _lib is not None:
        return _lib
    if not os.path.exists(path) or (path == LIB and os.path.getmtime(path) < os.path.getmtime(SRC)):
        build(out=path)
    lib = C.CDLL(path)
    vp, i64, i32, dbl = C.c_void_p, C.c_int64, C.c_int, C.c_double
    sig = {
        "orc_e2m1_value": (C.c_double, [i32]),
        "orc_e2m1_encode": (i32, [C.c_float]),
        "orc_e4m3_value": (C.c_double, [i32]),
        "orc_e2m1_to_e4m3": (i32, [i32]),
        "orc_expand_e4m3": (None, [vp, i64, vp]),
        "orc_e4m3_encode": (i32, [C.c_float]),
        "orc_e4m3_encode_array": (None, [vp, i64, vp]),
        "orc_fp8_quantize": (None, [vp, i32, i64, vp, vp]),
        "orc_fp8_dequantize": (None, [vp, i64, C.c_float, vp]),
        "orc_encode_array": (None, [vp, i64, vp]),
        "orc_quant_rows": (None, [vp, i64, i64, vp, vp]),
        "orc_quant_cols": (None, [vp, i32, i64, i64, vp, vp]),
        "orc_quantile_index": (i64, [i64, dbl]),
        "orc_abs_quantile": (C.c_float, [vp, i32, i64, dbl]),
        "orc_clamp_coo": (i64, [vp, i32, i64, i64, C.c_float, vp, vp, vp, vp, i64, vp]),
        "orc_accumulate": (None, [vp, vp, i64, i64, i64, vp]),
        "orc_accumulate_pairs": (None, [vp, vp, i64, vp, vp, i64, vp]),
        "orc_output": (None, [vp, vp, vp, i64, i64, vp, vp, vp, vp, i32, vp, vp]),
        "orc_output_pairs": (None, [vp, vp, vp, i64, vp, vp, i64, vp, vp, vp, vp, i32, vp, vp]),
        "orc_to_bf16": (None, [vp, i64, vp]),
        "orc_forward": (i64, [vp, vp, i32, i64, i64, i64, dbl, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp]),
        "orc_transpose_codes": (None, [vp, i64, i64, vp]),
        "orc_scaled_quant_rows": (None, [vp, i32, i64, i64, vp, vp, vp]),
        "orc_scaled_quant_cols": (None, [vp, i32, i64, i64, vp, vp, vp]),
        "orc_scale_pairs": (None, [vp, vp, vp, i64, vp]),
        "orc_backward": (None, [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path == LIB:
        _lib = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle inputs are float32 or bf16-as-uint16, got {a.dtype}")


def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) or float32 -> float32 values (exact)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32, copy=False)


# ----------------------------------------------------------------------------- codec
def e2m1_value(code: int) -> float:
    return load().orc_e2m1_value(int(code))


def e2m1_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32)).reshape(-1)
    out = np.empty(y.size, dtype=np.uint8)
    load().orc_encode_array(_p(y), y.size, _p(out))
    return out


def e4m3_value(b: int) -> float:
    return load().orc_e4m3_value(int(b))


def e2m1_to_e4m3(code: int) -> int:
    return load().orc_e2m1_to_e4m3(int(code))


def expand_e4m3(packed: np.ndarray) -> np.ndarray:
    """Packed E2M1 codes (R x C/2) -> E4M3 bytes (R x C), the FP4-on-FP8 operand form."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    load().orc_expand_e4m3(_p(packed), packed.size, _p(out))
    return out


def e4m3_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32)).reshape(-1)
    out = np.empty(y.size, dtype=np.uint8)
    load().orc_e4m3_encode_array(_p(y), y.size, _p(out))
    return out


def fp8_quantize(X: np.ndarray) -> tuple[np.ndarray, float]:
    """FP8 (E4M3) gradient codec, per-tensor scale: (codes u8[n], s)."""
    X = np.ascontiguousarray(X).reshape(-1)
    codes = np.empty(X.size, dtype=np.uint8)
    s = np.zeros(1, dtype=np.float32)
    load().orc_fp8_quantize(_p(X), _dtype_code(X), X.size, _p(codes), _p(s))
    return codes, float(s[0])


def fp8_dequantize(codes: np.ndarray, s: float) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    out = np.empty(codes.size, dtype=np.float32)
    load().orc_fp8_dequantize(_p(codes), codes.size, float(np.float32(s)), _p(out))
    return out


def unpack_codes(packed: np.ndarray, cols: int) -> np.ndarray:
    """rows x cols/2 packed bytes -> rows x cols codes (low nibble = even index)."""
    p = packed.reshape(-1, cols // 2)
    out = np.empty((p.shape[0], cols), dtype=np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


# ----------------------------------------------------------------------------- steps
def quantile_index(n: int, q: float) -> int:
    return int(load().orc_quantile_index(int(n), float(q)))


def abs_quantile(A: np.ndarray, q: float) -> float:
    A = np.ascontiguousarray(A)
    return float(np.float32(load().orc_abs_quantile(_p(A), _dtype_code(A), A.size, float(q))))


def capacity(M: int, K: int, q: float) -> int:
    """Upper bound on nnz: entries strictly above the (k+1)-th smallest."""
    return M * K - 1 - quantile_index(M * K, q)


def clamp_coo(A: np.ndarray, T: float, want_clamped: bool = True, cap: int | None = None) -> dict:
    A = np.ascontiguousarray(A)
    M, K = A.shape
    cap = M * K if cap is None else max(int(cap), 1)
    Ac = np.empty((M, K), dtype=np.float32) if want_clamped else None
    row = np.empty(cap, dtype=np.int32)
    col = np.empty(cap, dtype=np.int32)
    val = np.empty(cap, dtype=np.float32)
    row_ptr = np.empty(M + 1, dtype=np.int32)
    nnz = load().orc_clamp_coo(_p(A), _dtype_code(A), M, K, C.c_float(T), _p(Ac), _p(row), _p(col),
                               _p(val), cap, _p(row_ptr))
    if nnz > cap:
        raise RuntimeError("oracle: nnz exceeded the given capacity")
    return dict(nnz=int(nnz), coo_row=row[:nnz].copy(), coo_col=col[:nnz].copy(),
                coo_val=val[:nnz].copy(), row_ptr=row_ptr, A_clamped=Ac)


def quant_rows(X: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    X = np.ascontiguousarray(widen(X))
    R, Cc = X.shape
    codes = np.empty((R, Cc // 2), dtype=np.uint8)
    scales = np.empty(R, dtype=np.float32)
    load().orc_quant_rows(_p(X), R, Cc, _p(codes), _p(scales))
    return codes, scales


def quant_cols(W: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    W = np.ascontiguousarray(W)
    K, N = W.shape
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty(N, dtype=np.float32)
    load().orc_quant_cols(_p(W), _dtype_code(W), K, N, _p(codes), _p(scales))
    return codes, scales


def accumulate(Aq: np.ndarray, Wq: np.ndarray, K: int) -> np.ndarray:
    Aq, Wq = np.ascontiguousarray(Aq), np.ascontiguousarray(Wq)
    M, N = Aq.shape[0], Wq.shape[0]
    acc = np.empty((M, N), dtype=np.float32)
    load().orc_accumulate(_p(Aq), _p(Wq), M, N, K, _p(acc))
    return acc


def accumulate_pairs(Aq, Wq, K, ms, ns) -> np.ndarray:
    Aq, Wq = np.ascontiguousarray(Aq), np.ascontiguousarray(Wq)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    acc = np.empty(ms.size, dtype=np.float32)
    load().orc_accumulate_pairs(_p(Aq), _p(Wq), K, _p(ms), _p(ns), ms.size, _p(acc))
    return acc


def output(acc, sA, sW, row_ptr, coo_col, coo_val, W) -> tuple[np.ndarray, np.ndarray]:
    acc = np.ascontiguousarray(acc, dtype=np.float32)
    M, N = acc.shape
    W = np.ascontiguousarray(W)
    Y = np.empty((M, N), dtype=np.float32)
    denom = np.empty((M, N), dtype=np.float64)
    load().orc_output(_p(acc), _p(np.ascontiguousarray(sA)), _p(np.ascontiguousarray(sW)), M, N,
                      _p(row_ptr), _p(coo_col), _p(coo_val), _p(W), _dtype_code(W), _p(Y), _p(denom))
    return Y, denom


def output_pairs(acc, sA, sW, ms, ns, row_ptr, coo_col, coo_val, W) -> tuple[np.ndarray, np.ndarray]:
    W = np.ascontiguousarray(W)
    N = W.shape[1]
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    acc = np.ascontiguousarray(acc, dtype=np.float32)
    Y = np.empty(ms.size, dtype=np.float32)
    denom = np.empty(ms.size, dtype=np.float64)
    load().orc_output_pairs(_p(acc), _p(np.ascontiguousarray(sA)), _p(np.ascontiguousarray(sW)), N,
                            _p(ms), _p(ns), ms.size, _p(row_ptr), _p(coo_col), _p(coo_val), _p(W),
                            _dtype_code(W), _p(Y), _p(denom))
    return Y, denom


def to_bf16(Y: np.ndarray) -> np.ndarray:
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    out = np.empty(Y.shape, dtype=np.uint16)
    load().orc_to_bf16(_p(Y), Y.size, _p(out))
    return out


# ----------------------------------------------------------------------------- forward
def forward(A: np.ndarray, W: np.ndarray, q: float) -> dict:
    """Whole forward on small inputs: every intermediate and the fp32 output."""
    A, W = np.ascontiguousarray(A), np.ascontiguousarray(W)
    if _dtype_code(A) != _dtype_code(W):
        raise TypeError("A and W must share a dtype")
    M, K = A.shape
    N = W.shape[1]
    cap = capacity(M, K, q)
    T = np.zeros(1, dtype=np.float32)
    row = np.empty(max(cap, 1), dtype=np.int32)
    col = np.empty(max(cap, 1), dtype=np.int32)
    val = np.empty(max(cap, 1), dtype=np.float32)
    row_ptr = np.empty(M + 1, dtype=np.int32)
    Aq = np.empty((M, K // 2), dtype=np.uint8)
    sA = np.empty(M, dtype=np.float32)
    Wq = np.empty((N, K // 2), dtype=np.uint8)
    sW = np.empty(N, dtype=np.float32)
    acc = np.empty((M, N), dtype=np.float32)
    Y = np.empty((M, N), dtype=np.float32)
    denom = np.empty((M, N), dtype=np.float64)
    nnz = load().orc_forward(_p(A), _p(W), _dtype_code(A), M, K, N, float(q), _p(T), _p(row), _p(col),
                             _p(val), cap, _p(row_ptr), _p(Aq), _p(sA), _p(Wq), _p(sW), _p(acc), _p(Y),
                             _p(denom))
    if nnz < 0:
        raise RuntimeError("oracle: nnz exceeded the capacity bound")
    return dict(T=float(T[0]), nnz=int(nnz), coo_row=row[:nnz].copy(), coo_col=col[:nnz].copy(),
                coo_val=val[:nnz].copy(), row_ptr=row_ptr, Aq=Aq, sA=sA, Wq=Wq, sW=sW, acc=acc, Y=Y,
                denom=denom)


# ----------------------------------------------------------------------------- backward
def transpose_codes(codes: np.ndarray, R: int, Cc: int) -> np.ndarray:
    """R x Cc codes packed R x Cc/2 -> the transposed codes packed Cc x R/2."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty((Cc, R // 2), dtype=np.uint8)
    load().orc_transpose_codes(_p(codes), R, Cc, _p(out))
    return out


def scaled_quant_rows(X: np.ndarray, col_mult: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Token-wise quantization of fl(X * col_mult[None, :])."""
    X = np.ascontiguousarray(X)
    R, Cc = X.shape
    mult = np.ascontiguousarray(col_mult, dtype=np.float32)
    codes = np.empty((R, Cc // 2), dtype=np.uint8)
    scales = np.empty(R, dtype=np.float32)
    load().orc_scaled_quant_rows(_p(X), _dtype_code(X), R, Cc, _p(mult), _p(codes), _p(scales))
    return codes, scales


def scaled_quant_cols(X: np.ndarray, row_mult: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Channel-wise quantization of fl(row_mult[:, None] * X); codes are C x R/2."""
    X = np.ascontiguousarray(X)
    R, Cc = X.shape
    mult = np.ascontiguousarray(row_mult, dtype=np.float32)
    codes = np.empty((Cc, R // 2), dtype=np.uint8)
    scales = np.empty(Cc, dtype=np.float32)
    load().orc_scaled_quant_cols(_p(X), _dtype_code(X), R, Cc, _p(mult), _p(codes), _p(scales))
    return codes, scales


def scale_pairs(acc: np.ndarray, s: np.ndarray, idx) -> np.ndarray:
    """fl(acc[i] * s[idx[i]]): a backward output from its exact accumulator."""
    acc = np.ascontiguousarray(acc, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(acc.size, dtype=np.float32)
    load().orc_scale_pairs(_p(acc), _p(s), _p(idx), acc.size, _p(out))
    return out


def backward(dY: np.ndarray, Aq: np.ndarray, sA: np.ndarray, Wq: np.ndarray, sW: np.ndarray, K: int) -> dict:
    """Straight-through backward of the quantized product on small inputs."""
    dY = np.ascontiguousarray(dY)
    M, N = dY.shape
    Gq = np.empty((M, N // 2), dtype=np.uint8)
    sG = np.empty(M, dtype=np.float32)
    Hq = np.empty((N, M // 2), dtype=np.uint8)
    sH = np.empty(N, dtype=np.float32)
    WqT = np.empty((K, N // 2), dtype=np.uint8)
    AqT = np.empty((K, M // 2), dtype=np.uint8)
    dA = np.empty((M, K), dtype=np.float32)
    dW = np.empty((K, N), dtype=np.float32)
    load().orc_backward(_p(dY), _dtype_code(dY), M, K, N, _p(np.ascontiguousarray(Aq)),
                        _p(np.ascontiguousarray(sA, dtype=np.float32)), _p(np.ascontiguousarray(Wq)),
                        _p(np.ascontiguousarray(sW, dtype=np.float32)), _p(Gq), _p(sG), _p(Hq), _p(sH),
                        _p(WqT), _p(AqT), _p(dA), _p(dW))
    return dict(Gq=Gq, sG=sG, Hq=Hq, sH=sH, WqT=WqT, AqT=AqT, dA=dA, dW=dW)


def backward_sampled(dY: np.ndarray, Aq, sA, Wq, sW, K: int, mk, kn) -> dict:
    """Full-size intermediates of the backward, and dA at the (m, k) pairs mk and dW at
    the (k, n) pairs kn only."""
    dY = np.ascontiguousarray(dY)
    M, N = dY.shape
    Gq, sG = scaled_quant_rows(dY, sW)
    Hq, sH = scaled_quant_cols(dY, sA)
    WqT = transpose_codes(Wq, N, K)
    AqT = transpose_codes(Aq, M, K)
    ms, ks = np.asarray(mk[0], dtype=np.int64), np.asarray(mk[1], dtype=np.int64)
    ks2, ns2 = np.asarray(kn[0], dtype=np.int64), np.asarray(kn[1], dtype=np.int64)
    accA = accumulate_pairs(Gq, WqT, N, ms, ks)
    accW = accumulate_pairs(AqT, Hq, M, ks2, ns2)
    return dict(Gq=Gq, sG=sG, Hq=Hq, sH=sH, WqT=WqT, AqT=AqT, accA=accA, accW=accW,
                dA=scale_pairs(accA, sG, ms), dW=scale_pairs(accW, sH, ns2))
