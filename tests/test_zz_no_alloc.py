"""The no-allocation outlier pass (fp4_outlier_clamp_noalloc, fixed device scratch) against
fp4_outlier_clamp with a caller workspace: T, nnz, row_ptr and the COO list bit-exact, on two
calls in a row, the second with a smaller input (the scratch keeps the first call's contents),
and against the oracle on the second."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import quantized_linear_layers_fp4_amd as fp4
from workloads import as_numpy_bits, make_custom

DEV = torch.device("cuda:0")


def _p(t):
    return C.c_void_p(t.data_ptr())


def _noalloc(A: torch.Tensor, q: float) -> dict:
    M, K = A.shape
    L = fp4.lib()
    cap = max(int(L.fp4_outlier_capacity(M, K, float(q))), 1)
    T = torch.empty(4, dtype=torch.float32, device=DEV)
    row = torch.empty(cap, dtype=torch.int32, device=DEV)
    col = torch.empty(cap, dtype=torch.int32, device=DEV)
    val = torch.empty(cap, dtype=torch.float32, device=DEV)
    row_ptr = torch.empty(M + 1, dtype=torch.int32, device=DEV)
    nnz = torch.empty(2, dtype=torch.int64, device=DEV)
    st = L.fp4_outlier_clamp_noalloc(_p(A), fp4._dt(A), M, K, float(q), _p(T), _p(row), _p(col), _p(val), cap,
                                     _p(row_ptr), _p(nnz), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.fp4_status_string(st)
    n = int(nnz[0].item())
    return dict(T=T[:1], nnz=n, row_ptr=row_ptr, coo_row=row[:n], coo_col=col[:n], coo_val=val[:n])


def _same(a: dict, b: dict):
    assert a["nnz"] == int(b["nnz"][0].item())
    for k in ("T", "row_ptr", "coo_row", "coo_col", "coo_val"):
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k


@pytest.mark.gpu
def test_outlier_clamp_noalloc_matches_workspace_call():
    # call 1: bf16, 4096 x 4096, q = 0.999, with ten rows far past the staging slots (their
    # outliers are found again by the overflow path)
    A1, _ = make_custom(4096, 4096, 8, dtype="bf16", seed=61)
    A1[[3, 700, 4095]] *= 40.0
    A1 = A1.to(DEV)
    got1 = _noalloc(A1, 0.999)
    ref1 = fp4.outlier_clamp(A1, 0.999, trim=True)
    torch.cuda.synchronize()
    _same(got1, ref1)
    assert got1["nnz"] > 0 and int(torch.diff(got1["row_ptr"]).max().item()) > 128
    # call 2: smaller, fp32, 300 x 512, q = 0.99
    A2, _ = make_custom(300, 512, 8, dtype="fp32", seed=62)
    A2d = A2.to(DEV)
    got2 = _noalloc(A2d, 0.99)
    ref2 = fp4.outlier_clamp(A2d, 0.99, trim=True)
    torch.cuda.synchronize()
    _same(got2, ref2)
    cl = oracle.clamp_coo(as_numpy_bits(A2), oracle.abs_quantile(as_numpy_bits(A2), 0.99), want_clamped=False,
                          cap=oracle.capacity(300, 512, 0.99))
    assert got2["nnz"] == cl["nnz"]
    assert np.array_equal(got2["row_ptr"].cpu().numpy(), cl["row_ptr"])
    assert np.array_equal(got2["coo_col"].cpu().numpy(), cl["coo_col"])
    assert np.array_equal(got2["coo_val"].cpu().numpy(), cl["coo_val"])
