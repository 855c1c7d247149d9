"""Seeded synthetic inputs for the FP4 quantized linear forward.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic (no quantization, no quantile, no clamp, no product).
Both the oracle side and the HIP side take their inputs from here.

The shapes mirror the LLaMA-family linear layers that the FP4 training paper
trains (1.3B / 7B / 13B models; "Optimizing Large Language Model Training Using
FP4 Quantization", abstract and experiment summary): no dataset or trained
weight is involved, the value distributions are the synthetic stand-ins stated
per configuration below.

Recipe (all draws host-side, numpy PCG64 seeded by [20250128, seed_id, layer, stream]):
  stream 0 = base values of A, stream 1 = A structure (outlier positions,
  channels, per-row RMS), stream 2 = W, stream 3 = the output gradient dY of the
  backward (N(0, 1e-3), the magnitude of a loss-scaled activation gradient).  Values are drawn in float32; every
  scaling is applied in float32; bf16 tensors are the round-to-nearest-even
  cast of the float32 draw (torch CPU cast).
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np
import torch

SEED_ROOT = 20250128


@dataclasses.dataclass(frozen=True)
class Layer:
    """One linear layer workload: A is M x K (tokens x in), W is K x N (in x out)."""
    name: str
    M: int
    K: int
    N: int
    dtype: str          # "fp32" or "bf16" for A and W
    out_dtype: str      # "fp32" or "bf16" for Y
    q: float            # clamp quantile of |A|
    a_kind: str         # value structure of A (see _draw_A)
    w_std: float
    a_param: tuple = ()

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named set of layers; seed_id keys its random streams."""
    seed_id: int
    layers: tuple


# name -> workload.  llama7b_block is a chain of four independent layers (one LLaMA-7B block's
# projections at 8192 tokens).
WORKLOADS: dict[str, Workload] = {
    "tiny": Workload(1, (Layer("tiny", 128, 256, 128, "fp32", "fp32", 0.99, "normal_sparse_outliers", 0.02, (0.005, 50.0)),)),
    "llama1.3b_qkv": Workload(2, (Layer("llama1.3b_qkv", 8192, 2048, 6144, "bf16", "bf16", 0.99, "normal_channel_outliers", 0.02, (8, 30.0)),)),
    "llama7b_gate_up": Workload(3, (Layer("llama7b_gate_up", 16384, 4096, 22016, "bf16", "bf16", 0.999, "lognormal_rows_sparse_outliers", 0.015, (0.5, 0.001, 40.0)),)),
    "llama13b_down": Workload(4, (Layer("llama13b_down", 16384, 13824, 5120, "bf16", "bf16", 0.99, "student_t", 0.01, (3.0,)),)),
    "llama7b_block": Workload(5, (
        Layer("llama7b_qkv", 8192, 4096, 12288, "bf16", "bf16", 0.99, "normal_channel_outliers", 0.02, (6, 50.0)),
        Layer("llama7b_o", 8192, 4096, 4096, "bf16", "bf16", 0.99, "normal_channel_outliers", 0.02, (6, 50.0)),
        Layer("llama7b_gate_up", 8192, 4096, 22016, "bf16", "bf16", 0.99, "normal_channel_outliers", 0.02, (6, 50.0)),
        Layer("llama7b_down", 8192, 11008, 4096, "bf16", "bf16", 0.99, "normal_channel_outliers", 0.02, (6, 50.0)),
    )),
}
# the 7B layer chain with the quantile of the gate+up shape (0.999) instead of 0.99: the same
# seeded inputs (seed_id 5), fewer outliers per row
WORKLOADS["llama7b_block_q999"] = Workload(5, tuple(dataclasses.replace(L, q=0.999)
                                                    for L in WORKLOADS["llama7b_block"].layers))


def _rng(seed_id: int, layer: int, stream: int, replica: int = 0) -> np.random.Generator:
    key = [SEED_ROOT, seed_id, layer, stream] + ([replica] if replica else [])
    return np.random.Generator(np.random.PCG64(key))


def _normal(rng, shape, std=1.0, chunk_rows=2048) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    for r0 in range(0, shape[0], chunk_rows):
        blk = rng.standard_normal((min(chunk_rows, shape[0] - r0), shape[1]), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        out[r0:r0 + blk.shape[0]] = blk
    return out


def _draw_A(L: Layer, seed_id: int, li: int, replica: int = 0) -> np.ndarray:
    M, K = L.M, L.K
    base = _rng(seed_id, li, 0, replica)
    struct = _rng(seed_id, li, 1, replica)
    if L.a_kind == "normal_sparse_outliers":
        frac, mult = L.a_param
        A = _normal(base, (M, K))
        n_out = int(frac * M * K)
        pos = struct.choice(M * K, size=n_out, replace=False)
        A.reshape(-1)[pos] *= np.float32(mult)
    elif L.a_kind == "normal_channel_outliers":
        n_ch, mult = L.a_param
        A = _normal(base, (M, K))
        ch = struct.choice(K, size=n_ch, replace=False)
        A[:, ch] *= np.float32(mult)
    elif L.a_kind == "lognormal_rows_sparse_outliers":
        sigma, frac, mult = L.a_param
        A = _normal(base, (M, K))
        rms = struct.lognormal(0.0, sigma, size=M).astype(np.float32)
        A *= rms[:, None]
        n_out = int(frac * M * K)
        pos = struct.choice(M * K, size=n_out, replace=False)
        A.reshape(-1)[pos] *= np.float32(mult)
    elif L.a_kind == "student_t":
        (df,) = L.a_param
        A = np.empty((M, K), dtype=np.float32)
        for r0 in range(0, M, 1024):
            r1 = min(M, r0 + 1024)
            A[r0:r1] = base.standard_t(df, size=(r1 - r0, K)).astype(np.float32)
    else:  # pragma: no cover - table above is closed
        raise ValueError(L.a_kind)
    return A


def _to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def make_layer(workload: str, li: int = 0, replica: int = 0) -> tuple[torch.Tensor, torch.Tensor, Layer]:
    """Return (A, W, layer) as CPU tensors of the layer's dtype.  replica > 0 draws another
    input set of the same shapes and distributions from streams of its own (a benchmark
    rotates sets so that its inputs are not cache-resident); replica 0 is the reference set."""
    wl = WORKLOADS[workload]
    L = wl.layers[li]
    A = _draw_A(L, wl.seed_id, li, replica)
    W = _normal(_rng(wl.seed_id, li, 2, replica), (L.K, L.N), std=L.w_std)
    return _to_dtype(A, L.dtype), _to_dtype(W, L.dtype), L


GRAD_STD = 1e-3


def make_grad(workload: str, li: int = 0) -> torch.Tensor:
    """dY (M x N) for the backward of the layer, as a CPU tensor of the layer's dtype."""
    wl = WORKLOADS[workload]
    L = wl.layers[li]
    return _to_dtype(_normal(_rng(wl.seed_id, li, 3), (L.M, L.N), std=GRAD_STD), L.dtype)


def make_custom_grad(M: int, N: int, dtype: str = "bf16", seed: int = 0) -> torch.Tensor:
    """Small seeded dY for parity tests of arbitrary shapes."""
    rng = np.random.Generator(np.random.PCG64([SEED_ROOT, 2000 + seed, M, N]))
    return _to_dtype(rng.standard_normal((M, N), dtype=np.float32) * np.float32(GRAD_STD), dtype)


def make_custom(M: int, K: int, N: int, dtype: str = "bf16", seed: int = 0,
                kind: str = "normal_sparse_outliers", outlier_frac: float = 0.005,
                outlier_mult: float = 50.0, w_std: float = 0.02) -> tuple[torch.Tensor, torch.Tensor]:
    """Small seeded inputs for parity tests of arbitrary (ragged) shapes."""
    rng = np.random.Generator(np.random.PCG64([SEED_ROOT, 1000 + seed, M, K, N]))
    A = rng.standard_normal((M, K), dtype=np.float32)
    if kind == "normal_sparse_outliers":
        n_out = int(outlier_frac * M * K)
        if n_out:
            pos = rng.choice(M * K, size=n_out, replace=False)
            A.reshape(-1)[pos] *= np.float32(outlier_mult)
    elif kind == "student_t":
        A = rng.standard_t(3.0, size=(M, K)).astype(np.float32)
    elif kind == "plain":
        pass
    else:
        raise ValueError(kind)
    W = rng.standard_normal((K, N), dtype=np.float32) * np.float32(w_std)
    return _to_dtype(A, dtype), _to_dtype(W, dtype)


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()


def as_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy array holding the same bytes (bf16 as uint16)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()
