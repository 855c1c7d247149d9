"""Helpers shared by the GPU parity tests: comparisons against the oracle's outputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads import as_numpy_bits

# Y tolerance (fp32): |Y_gpu - Y_oracle| <= REL * (|Y_main| + sum_k |delta_k * W[k][n]|).
# The dequantized product is bit-exact; only the compensation sum differs in rounding
# order (fp32 in ascending k on the GPU, double in the oracle).  Each fp32 step adds at
# most 2^-24 of the running magnitude, so n terms stay below (n + 1) * 2^-24 of the
# denominator: 1e-5 covers rows with up to ~160 compensation terms in the worst case,
# and the observed errors (random-walk) are far below it.
REL = 1e-5


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_y_close(y_gpu: np.ndarray, y_ref: np.ndarray, denom: np.ndarray, what: str = "Y"):
    """Checks |Y_gpu - Y_ref| <= REL * denom element by element (denom = |Y_main| + the row's
    sum |delta_k * W[k][n]|, the scale of the forward error of the compensation sum in any
    order) and returns the largest err / denom."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64))
    bound = REL * denom
    bad = np.nonzero(err > bound)
    if bad[0].size:
        i = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} entries beyond tolerance; first at {i}: gpu={y_gpu[i]!r} "
                             f"ref={y_ref[i]!r} denom={denom[i]!r}")
    return float((err / np.maximum(denom, 1e-300)).max()) if err.size else 0.0


def plain_rel_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    """The plain relative error max |Y_gpu - Y_ref| / |Y_ref| over the entries with
    |Y_ref| >= 1e-3 * rms(Y_ref) (entries near zero, where Y_main and the compensation cancel,
    are left out: there only the tolerance above is meaningful).  Reported beside it."""
    r = y_ref.astype(np.float64).reshape(-1)
    g = y_gpu.astype(np.float64).reshape(-1)
    if r.size == 0:
        return 0.0
    keep = np.abs(r) >= 1e-3 * np.sqrt(np.mean(r * r))
    if not keep.any():
        return 0.0
    return float((np.abs(g[keep] - r[keep]) / np.abs(r[keep])).max())


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_bf16_close(y_bits: np.ndarray, y_ref: np.ndarray, denom: np.ndarray, what: str = "Y(bf16)"):
    """The bf16 output is a round-to-nearest of a value within tolerance of the oracle's Y."""
    g = bf16_to_f64(y_bits)
    r = y_ref.astype(np.float64)
    tol = REL * denom
    lo = oracle.to_bf16((r - tol).astype(np.float32))
    hi = oracle.to_bf16((r + tol).astype(np.float32))
    lo_v, hi_v = bf16_to_f64(lo), bf16_to_f64(hi)
    ok = (g >= np.minimum(lo_v, hi_v)) & (g <= np.maximum(lo_v, hi_v))
    if not np.all(ok):
        i = tuple(b[0] for b in np.nonzero(~ok))
        raise AssertionError(f"{what}: first mismatch at {i}: gpu={g[i]} ref={r[i]} tol={tol[i]}")


def coo_dense(row_ptr, col, val, M, K):
    d = np.zeros((M, K), dtype=np.float32)
    rows = np.repeat(np.arange(M), np.diff(row_ptr))
    d[rows, col] = val
    return d


def oracle_inputs(A: torch.Tensor, W: torch.Tensor):
    return as_numpy_bits(A.cpu()), as_numpy_bits(W.cpu())
