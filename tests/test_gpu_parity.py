"""HIP path vs the CPU oracle on the same seeded inputs (needs an MI355X).

Bit-exact: E2M1 codes, scales, T, nnz, the COO list of dA, row_ptr and the raw
accumulator.  Y (fp32) within the tolerance in parity_util.REL; bf16 Y a correct
rounding of a value within that tolerance.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_linear_layers_fp4_amd as fp4
from parity_util import (assert_bf16_close, assert_y_close, bf16_to_f64, oracle_inputs, plain_rel_err, to_np)
from workloads import WORKLOADS, as_numpy_bits, make_custom, make_custom_grad, make_layer

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dt(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


# ----------------------------------------------------------------------------- codec
def test_codec_every_bf16_pattern():
    # every bf16 magnitude up to 6, both signs, in rows whose maximum is exactly 6 so the
    # multiplier r = fl(6/6) = 1 and the codes are the plain E2M1 rounding of the input
    _say("codec sweep bf16")
    pats = np.arange(0, 0x40C1, dtype=np.uint16)
    vals = np.concatenate([pats, pats | 0x8000]).astype(np.uint16)
    per_row = 511
    nrows = -(-vals.size // per_row)
    X = np.zeros((nrows, 512), dtype=np.uint16)
    flat = np.zeros(nrows * per_row, dtype=np.uint16)
    flat[:vals.size] = vals
    X[:, 1:] = flat.reshape(nrows, per_row)
    X[:, 0] = 0x40C0  # 6.0
    Xt = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(DEV)
    codes, scales = fp4.quantize(Xt, fp4.FP4_PER_ROW)
    ref_c, ref_s = oracle.quant_rows(X)
    assert np.array_equal(to_np(scales), ref_s)
    assert np.array_equal(to_np(codes), ref_c)


def test_codec_fp32_sweep():
    _say("codec sweep fp32")
    rng = np.random.default_rng(2)
    pats = np.arange(0, 0x40C00001, 9973, dtype=np.uint32).view(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), mids, np.nextafter(mids, np.float32(9))])
    vals = np.concatenate([pats, near, rng.uniform(0, 6, 100000).astype(np.float32)])
    vals = np.concatenate([vals, -vals])
    per_row = 1023
    nrows = -(-vals.size // per_row)
    X = np.zeros((nrows, 1024), dtype=np.float32)
    flat = np.zeros(nrows * per_row, dtype=np.float32)
    flat[:vals.size] = vals
    X[:, 1:] = flat.reshape(nrows, per_row)
    X[:, 0] = 6.0
    codes, scales = fp4.quantize(torch.from_numpy(X).to(DEV), fp4.FP4_PER_ROW)
    ref_c, ref_s = oracle.quant_rows(X)
    assert np.array_equal(to_np(scales), ref_s)
    assert np.array_equal(to_np(codes), ref_c)


# ----------------------------------------------------------------------------- quantizers
ROW_SHAPES = [(1, 32), (37, 96), (257, 1056), (300, 4096), (4, 65536)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_quantize_rows(dtype, shape):
    R, C = shape
    _say(f"quantize rows {dtype} {shape}")
    rng = np.random.default_rng(R * 7 + C)
    X = (rng.standard_normal((R, C)) * rng.lognormal(0, 2, (R, 1))).astype(np.float32)
    if R > 3:
        X[1] = 0.0  # all-zero row: scale 0, sign-only codes
        X[2, : C // 2] = -0.0
    Xt = torch.from_numpy(X).to(_dt(dtype))
    codes, scales = fp4.quantize(Xt.to(DEV), fp4.FP4_PER_ROW)
    ref_c, ref_s = oracle.quant_rows(as_numpy_bits(Xt))
    assert np.array_equal(to_np(scales), ref_s)
    assert np.array_equal(to_np(codes), ref_c)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_rows_clamped(dtype):
    R, C = 130, 512
    _say(f"quantize rows clamped {dtype}")
    A, _ = make_custom(R, C, 8, dtype=dtype, seed=5)
    Anp = as_numpy_bits(A)
    T = oracle.abs_quantile(Anp, 0.99)
    Tt = torch.tensor([T], dtype=torch.float32, device=DEV)
    codes, scales = fp4.quantize(A.to(DEV), fp4.FP4_PER_ROW, clamp_T=Tt)
    Ac = oracle.clamp_coo(Anp, T)["A_clamped"]
    ref_c, ref_s = oracle.quant_rows(Ac)
    assert np.array_equal(to_np(scales), ref_s)
    assert np.array_equal(to_np(codes), ref_c)


COL_SHAPES = [(32, 8), (96, 264), (1056, 520), (4096, 1000), (288, 4104)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", COL_SHAPES)
def test_quantize_cols(dtype, shape):
    K, N = shape
    _say(f"quantize cols {dtype} {shape}")
    rng = np.random.default_rng(K + 3 * N)
    W = (rng.standard_normal((K, N)) * rng.lognormal(-3, 1, (1, N))).astype(np.float32)
    W[:, 3] = 0.0
    Wt = torch.from_numpy(W).to(_dt(dtype))
    codes, scales = fp4.quantize(Wt.to(DEV), fp4.FP4_PER_COL)
    ref_c, ref_s = oracle.quant_cols(as_numpy_bits(Wt))
    assert np.array_equal(to_np(scales), ref_s)
    assert np.array_equal(to_np(codes), ref_c)


# ----------------------------------------------------------------------------- outliers
OUT_CASES = [
    ("bf16", 64, 128, 0.99, "student_t"), ("bf16", 300, 1056, 0.99, "normal_sparse_outliers"),
    ("bf16", 1000, 4096, 0.999, "normal_sparse_outliers"), ("fp32", 128, 256, 0.99, "normal_sparse_outliers"),
    ("fp32", 333, 512, 0.9, "student_t"), ("bf16", 17, 64, 0.0, "plain"), ("bf16", 40, 96, 1.0, "plain"),
    ("fp32", 9, 32, 0.5, "plain"), ("bf16", 2000, 2048, 0.5, "student_t"),
    # more rows than one COO workgroup sums for its own offset: the row offsets come from a scan
    ("bf16", 16400, 64, 0.99, "student_t"),
]


@pytest.mark.parametrize("dtype,M,K,q,kind", OUT_CASES)
def test_outlier_clamp(dtype, M, K, q, kind):
    _say(f"outlier clamp {dtype} {M}x{K} q={q} {kind}")
    A, _ = make_custom(M, K, 8, dtype=dtype, seed=M + K, kind=kind)
    out = fp4.outlier_clamp(A.to(DEV), q)
    Anp = as_numpy_bits(A)
    T = oracle.abs_quantile(Anp, q)
    ref = oracle.clamp_coo(Anp, T, want_clamped=False)
    assert float(out["T"].item()) == T
    assert int(out["nnz"].item()) == ref["nnz"] <= oracle.capacity(M, K, q)
    assert np.array_equal(to_np(out["row_ptr"]), ref["row_ptr"])
    assert np.array_equal(to_np(out["coo_row"]), ref["coo_row"])
    assert np.array_equal(to_np(out["coo_col"]), ref["coo_col"])
    assert np.array_equal(to_np(out["coo_val"]), ref["coo_val"])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows", [(3,), (1, 2, 30, 31, 64, 100, 101, 200, 254, 255)], ids=["one_row", "ten_rows"])
def test_outlier_clamp_row_overflow(dtype, rows):
    # nearly every outlier in a few rows: those rows outgrow their staging slots and are read
    # again when the COO list is assembled
    M, K, q = 256, 1024, 0.995
    _say(f"outlier overflow {dtype} rows={rows}")
    A, W = make_custom(M, K, 64, dtype=dtype, seed=77, kind="plain")
    for r in rows:
        A[r] *= 100
    A[200, 7] = 1000.0
    out = fp4.outlier_clamp(A.to(DEV), q)
    Anp = as_numpy_bits(A)
    T = oracle.abs_quantile(Anp, q)
    ref = oracle.clamp_coo(Anp, T, want_clamped=False)
    assert max(ref["row_ptr"][r + 1] - ref["row_ptr"][r] for r in rows) > 64  # beyond the per-row slots
    assert float(out["T"].item()) == T
    assert np.array_equal(to_np(out["row_ptr"]), ref["row_ptr"])
    assert np.array_equal(to_np(out["coo_col"]), ref["coo_col"])
    assert np.array_equal(to_np(out["coo_val"]), ref["coo_val"])
    assert np.array_equal(to_np(out["coo_row"]), ref["coo_row"])
    _check_forward_small(A, W, q, torch.float32)


# ----------------------------------------------------------------------------- GEMM
def _random_codes(rng, R, K):
    return rng.integers(0, 256, (R, K // 2), dtype=np.uint8)


GEMM_SHAPES = [(256, 256, 256), (300, 264, 320), (513, 776, 1056), (64, 8, 32), (1, 520, 4096), (777, 1032, 2080)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_accumulator_exact(M, N, K):
    _say(f"gemm acc {M}x{N}x{K}")
    rng = np.random.default_rng(M * N + K)
    Aq, Wq = _random_codes(rng, M, K), _random_codes(rng, N, K)
    sA = rng.lognormal(-2, 1, M).astype(np.float32)
    sW = rng.lognormal(-4, 1, N).astype(np.float32)
    t = lambda x: torch.from_numpy(x).to(DEV)
    Y, acc = fp4.gemm(t(Aq), t(sA), t(Wq), t(sW), K, out_dtype=torch.float32, acc_out=True)
    ref_acc = oracle.accumulate(Aq, Wq, K)
    assert np.array_equal(to_np(acc), ref_acc)
    ref_y, denom = oracle.output(ref_acc, sA, sW, None, None, None, np.zeros((K, N), dtype=np.float32))
    assert np.array_equal(to_np(Y), ref_y)  # no compensation: the dequantized product is bit-exact


# More output tiles than the chip has CUs, ragged in both dimensions, K a multiple of 512: the
# product then walks several tiles per workgroup (the last two shapes have over 1024 tiles of
# 256 x 256, at least two per CU, so they run on the persistent kernel).  Checked at sampled outputs plus whole
# edge rows and columns.
@pytest.mark.parametrize("M,N,K,out", [(4200, 4136, 1024, "fp32"), (4352, 4360, 512, "bf16"), (1030, 9000, 2048, "fp32"),
                                       (8192, 8200, 512, "bf16"), (8200, 8192, 1024, "fp32")])
def test_gemm_many_tiles(M, N, K, out):
    _say(f"gemm many tiles {M}x{N}x{K} -> {out}")
    rng = np.random.default_rng(M + N + K)
    Aq, Wq = _random_codes(rng, M, K), _random_codes(rng, N, K)
    sA = rng.lognormal(-2, 1, M).astype(np.float32)
    sW = rng.lognormal(-4, 1, N).astype(np.float32)
    t = lambda x: torch.from_numpy(x).to(DEV)
    Y, acc = fp4.gemm(t(Aq), t(sA), t(Wq), t(sW), K, out_dtype=_dt(out), acc_out=True)
    ms = np.concatenate([rng.integers(0, M, 20000), np.full(N, M - 1), np.arange(M), np.zeros(N, dtype=np.int64)])
    ns = np.concatenate([rng.integers(0, N, 20000), np.arange(N), np.full(M, N - 1), np.arange(N)])
    idx = torch.from_numpy(ms * N + ns).to(DEV)
    g_acc = acc.view(-1)[idx].cpu().numpy()
    r_acc = oracle.accumulate_pairs(Aq, Wq, K, ms, ns)
    assert np.array_equal(g_acc, r_acc)
    r_y, _ = oracle.output_pairs(r_acc, sA, sW, ms, ns, None, None, None, np.zeros((1, N), dtype=np.float32))
    g_y = to_np(Y.view(-1)[idx])
    assert np.array_equal(g_y, r_y if out == "fp32" else oracle.to_bf16(r_y))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 264, 320), (513, 776, 1056), (64, 8, 32), (257, 136, 96)])
def test_gemm_fp8_emulation(M, N, K):
    """FP4 codes expanded to E4M3 and multiplied on the FP8 matrix cores: the accumulator
    is the oracle's exact sum and Y is bit-identical to the native FP4 product (fp32 and
    bf16 outputs).  K = 96 and 1056 leave a partial last stage."""
    _say(f"gemm fp8 emulation {M}x{N}x{K}")
    rng = np.random.default_rng(M * N + K + 1)
    Aq, Wq = _random_codes(rng, M, K), _random_codes(rng, N, K)
    sA = rng.lognormal(-2, 1, M).astype(np.float32)
    sW = rng.lognormal(-4, 1, N).astype(np.float32)
    t = lambda x: torch.from_numpy(x).to(DEV)
    Y8, acc8 = fp4.gemm_fp8emu(t(Aq), t(sA), t(Wq), t(sW), K, out_dtype=torch.float32, acc_out=True)
    Y4 = fp4.gemm(t(Aq), t(sA), t(Wq), t(sW), K, out_dtype=torch.float32)
    Yb8 = fp4.gemm_fp8emu(t(Aq), t(sA), t(Wq), t(sW), K, out_dtype=torch.bfloat16)
    Yb4 = fp4.gemm(t(Aq), t(sA), t(Wq), t(sW), K, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(acc8), oracle.accumulate(Aq, Wq, K))
    assert torch.equal(Y8.view(torch.int32), Y4.view(torch.int32))
    assert torch.equal(Yb8.view(torch.int16), Yb4.view(torch.int16))


def test_gemm_fp8_emulation_full_size():
    """The same identity on the gate+up shape's own codes (M=16384, K=4096, N=22016)."""
    _say("gemm fp8 emulation llama7b_gate_up")
    A, W, L = make_layer("llama7b_gate_up", 0)
    Ad, Wd = A.to(DEV), W.to(DEV)
    ws = fp4.workspace(Ad, L.N, L.q)
    fp4.linear_forward(Ad, Wd, L.q, ws=ws)
    it = fp4.forward_intermediates(ws, L.M, L.K, L.N, A.dtype, L.q)
    Y8 = fp4.gemm_fp8emu(it["Aq"], it["sA"], it["Wq"], it["sW"], L.K, out_dtype=torch.bfloat16)
    Y4 = fp4.gemm(it["Aq"], it["sA"], it["Wq"], it["sW"], L.K, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(Y8.view(torch.int16), Y4.view(torch.int16))


def test_gemm_accumulator_extremes():
    # every product +-36 over the longest K: |acc| = 36 * 65536, still exact in fp32
    M, N, K = 40, 24, 65536
    _say("gemm acc extremes K=65536")
    Aq = np.full((M, K // 2), 0x77, dtype=np.uint8)
    Aq[1::2] = 0xFF
    Wq = np.full((N, K // 2), 0x77, dtype=np.uint8)
    Wq[::3] = 0xF7  # alternating +-6 along k
    t = lambda x: torch.from_numpy(x).to(DEV)
    ones_m = torch.ones(M, device=DEV)
    ones_n = torch.ones(N, device=DEV)
    _, acc = fp4.gemm(t(Aq), ones_m, t(Wq), ones_n, K, out_dtype=torch.float32, acc_out=True)
    assert np.array_equal(to_np(acc), oracle.accumulate(Aq, Wq, K))
    assert to_np(acc)[0, 1] == 36.0 * K and to_np(acc)[1, 1] == -36.0 * K


@pytest.mark.parametrize("shape", ["chunk512", "block64"])
@pytest.mark.parametrize("M,N,K,wdt", [(300, 264, 512, "bf16"), (513, 520, 1056, "fp32"), (64, 8, 96, "bf16"),
                                       (70, 776, 128, "fp32")])
def test_gemm_with_compensation(M, N, K, wdt, shape):
    """Both shapes of the compensation kernel (the capacity hint picks one: more than 64
    entries per row selects the 8-row x 64-column blocks)."""
    _say(f"gemm comp {M}x{N}x{K} {wdt} {shape}")
    wide = shape != "block64"
    A, W = make_custom(M, K, N, dtype=wdt, seed=11)
    Anp, Wnp = oracle_inputs(A, W)
    q = 0.98
    ref = oracle.forward(Anp, Wnp, q)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    args = (t(ref["Aq"]), t(ref["sA"]), t(ref["Wq"]), t(ref["sW"]), K)
    kw = dict(row_ptr=t(ref["row_ptr"]), coo_col=t(ref["coo_col"]), coo_val=t(ref["coo_val"]), W=W.to(DEV),
              capacity={"chunk512": 0, "block64": 65 * M}[shape])
    Y32 = fp4.gemm(*args, **kw, out_dtype=torch.float32)
    Y16 = fp4.gemm(*args, **kw, out_dtype=torch.bfloat16)
    assert_y_close(to_np(Y32), ref["Y"], ref["denom"])
    # the bf16 output is the round-to-nearest-even of the same fp32 result
    assert np.array_equal(to_np(Y16), to_np(Y32.to(torch.bfloat16)))


def _escape_codes(rng, M, N, K, rows, cols):
    """Random codes, except rows of Aq and of Wq (output channels) holding +6 everywhere:
    their products reach acc = 36 K, past the two-byte hand-over's range once K > 227."""
    Aq, Wq = _random_codes(rng, M, K), _random_codes(rng, N, K)
    Aq[list(rows)] = 0x77
    Wq[list(cols)] = 0x77
    return Aq, Wq


def _check_q16(Yq, esc, acc, sA, sW):
    """The FP4_Q16 contract element by element: the int16 4*acc, or -32768 with esc holding
    fl(fl(acc*sA)*sW) in fp32; every |acc| > 8191.75 is escaped, escapes come in whole aligned
    128 x 64 blocks (clipped at the edges), and each escaped block lies in an aligned 128 x 128
    block that holds such an accumulator.  Returns the number of escaped elements."""
    yq = Yq.cpu().numpy().astype(np.int64)
    a = acc.cpu().numpy()
    escaped = yq == -32768
    big = np.abs(a) > 8191.75
    assert np.all(escaped[big])
    assert np.array_equal(yq[~escaped], (a[~escaped] * 4).astype(np.int64))
    if escaped.any():
        e = esc.cpu().numpy()
        ymain = (a[escaped] * sA[np.nonzero(escaped)[0]]).astype(np.float32) * sW[np.nonzero(escaped)[1]]
        assert np.array_equal(e[escaped], ymain.astype(np.float32))
        M, N = a.shape
        cm, cn = (M + 127) // 128, (N + 127) // 128 * 2  # 128 x 64 cells, whole 128 x 128 blocks
        pad = lambda x: np.pad(x, ((0, cm * 128 - M), (0, cn * 64 - N)))  # noqa: E731
        inside = pad(np.ones_like(escaped)).reshape(cm, 128, cn, 64)
        cells = pad(escaped).reshape(cm, 128, cn, 64)
        esc_cell = cells.any(axis=(1, 3))
        assert np.all((cells | ~inside).all(axis=(1, 3))[esc_cell])  # whole cells
        hot = pad(big).reshape(cm, 128, cn // 2, 128).any(axis=(1, 3))
        r, c = np.nonzero(esc_cell)
        assert np.all(hot[r, c // 2])
    return int(escaped.sum())


@pytest.mark.parametrize("M,N,K", [(300, 264, 512), (513, 776, 1056), (64, 8, 256), (257, 136, 96)])
def test_gemm_q16_handover(M, N, K):
    """The GEMM's two-byte accumulator output (the hand-over to the compensation pass) on the
    256 x 128 kernel: exact 4*acc, escapes where |acc| > 8191.75 (rows and channels of +6
    codes; none for K = 96, where 36 K < 8192), fp32 values there."""
    _say(f"gemm q16 {M}x{N}x{K}")
    rng = np.random.default_rng(M + 3 * N + K)
    rows, cols = {0, M // 2, M - 1}, {0, N // 2, N - 1}
    Aq, Wq = _escape_codes(rng, M, N, K, rows, cols)
    sA = rng.lognormal(-2, 1, M).astype(np.float32)
    sW = rng.lognormal(-4, 1, N).astype(np.float32)
    t = lambda x: torch.from_numpy(x).to(DEV)
    Yq, esc, acc = fp4.gemm_q16(t(Aq), t(sA), t(Wq), t(sW), K, acc_out=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(acc), oracle.accumulate(Aq, Wq, K))
    n_esc = _check_q16(Yq, esc, acc, sA, sW)
    assert (n_esc > 0) == (36 * K > 8191.75)


@pytest.mark.parametrize("M,N,K", [(8192, 8192, 512), (8200, 8192, 1024)])
def test_gemm_q16_handover_wide(M, N, K):
    """The same contract on the persistent 256 x 256 kernel (1024 or more tiles), the escape
    kernel recomputing only the marked blocks.  K = 1024 (eight K-stages) is the first depth at
    which a tile's last pairs are stored under the next tile's first steps; M = 8200 adds a
    ragged row of tiles."""
    _say(f"gemm q16 wide {M}x{N}x{K}")
    rng = np.random.default_rng(77)
    rows, cols = {0, 4000, M - 1}, {5, 4100, N - 1}
    Aq, Wq = _escape_codes(rng, M, N, K, rows, cols)
    sA = rng.lognormal(-2, 1, M).astype(np.float32)
    sW = rng.lognormal(-4, 1, N).astype(np.float32)
    t = lambda x: torch.from_numpy(x).to(DEV)
    Yq, esc, acc = fp4.gemm_q16(t(Aq), t(sA), t(Wq), t(sW), K, acc_out=True)
    torch.cuda.synchronize()
    ms = np.concatenate([rng.integers(0, M, 20000), np.repeat(sorted(rows), N)])
    ns = np.concatenate([rng.integers(0, N, 20000), np.tile(np.arange(N), len(rows))])
    g = acc.view(-1)[torch.from_numpy(ms * N + ns).to(DEV)].cpu().numpy()
    assert np.array_equal(g, oracle.accumulate_pairs(Aq, Wq, K, ms, ns))
    n_esc = _check_q16(Yq, esc, acc, sA, sW)
    assert n_esc > 0


@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("fp32", "fp32")])
def test_forward_rows_of_every_length(dtype, out):
    """A high clamp quantile with rows of 0, 1-8, 9-16 and up to 64+ entries (one, two and
    several groups of eight W segments, and more than 64 entries: two windows of (k, delta)
    pairs), including the first and last rows."""
    _say(f"forward row lengths {dtype} out={out}")
    M, K, N = 300, 1024, 776
    A, W = make_custom(M, K, N, dtype=dtype, seed=31, outlier_frac=0.0)
    rng = np.random.default_rng(5)
    for r, n in ((0, 40), (3, 17), (50, 12), (51, 9), (100, 70), (200, 3), (M - 1, 30)):
        cols = rng.choice(K, n, replace=False)
        A[r, cols] = torch.from_numpy((rng.choice([-1.0, 1.0], n) * rng.uniform(60, 90, n)).astype(np.float32)).to(A.dtype)
    q = 0.999  # about 300 entries: the 175 planted ones and the largest normal values
    assert fp4.outlier_capacity(M, K, q) <= 8 * M
    _check_forward_small(A, W, q, _dt(out))


@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("bf16", "fp32"), ("fp32", "fp32")])
def test_forward_with_escaped_accumulators(dtype, out):
    """Rows of A and columns of W that quantize to +6 everywhere give acc = 36 K = 18432, past
    the two-byte hand-over: the GEMM marks those blocks, the compensation pass skips them and
    the escape kernel writes their Y from the codes; the whole Y must still be the oracle's."""
    _say(f"forward escapes {dtype} out={out}")
    A, W = make_custom(300, 512, 264, dtype=dtype, seed=21)
    A[5:8] = 1.0
    W[:, 10:13] = 0.02
    W[:, 200] = -0.02
    _check_forward_small(A, W, 0.99, _dt(out))


@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("fp32", "fp32")])
def test_forward_heavy_row_in_escaped_block(dtype, out):
    """A row with many dA entries inside an escaped block.  Row 130 holds 70 planted outliers
    (+80) and 1.0 elsewhere, and against W's column 40 (0.02 everywhere) its accumulator is past
    the two-byte range: its compensation task (a chain of 70 entries, nine groups of W segments)
    must leave that escaped 128 x 64 block to the escape kernel, which walks the same 70 entries,
    and write the rest of its chunk; row 3 carries 78 entries in a block that does not escape."""
    _say(f"forward heavy row in an escaped block {dtype} out={out}")
    M, K, N = 300, 1024, 264
    A, W = make_custom(M, K, N, dtype=dtype, seed=61)
    rng = np.random.default_rng(7)
    A[130] = 1.0
    for r in (130, 3):
        cols = rng.choice(K, 70, replace=False)
        A[r, cols] = 80.0
    W[:, 40] = 0.02
    q = 0.99
    assert fp4.outlier_capacity(M, K, q) <= 64 * M  # the 512-column chunk tasks
    _check_forward_small(A, W, q, _dt(out))
    Anp, Wnp = oracle_inputs(A, W)
    cl = oracle.clamp_coo(Anp, oracle.abs_quantile(Anp, q), want_clamped=True, cap=oracle.capacity(M, K, q))
    assert np.diff(cl["row_ptr"])[[3, 130]].min() > 64
    Aq = oracle.quant_rows(cl["A_clamped"])[0]
    Wq = oracle.quant_cols(Wnp)[0]
    assert abs(oracle.accumulate(Aq[130:131], Wq[40:41], K)[0, 0]) > 8191.75  # that block escaped


# ----------------------------------------------------------------------------- forward
def _check_forward_small(A, W, q, out_dtype):
    M, K = A.shape
    N = W.shape[1]
    Ad, Wd = A.to(DEV), W.to(DEV)
    ws = fp4.workspace(Ad, N, q, out_dtype)
    Y = fp4.linear_forward(Ad, Wd, q, out_dtype=out_dtype, ws=ws)
    torch.cuda.synchronize()
    inter = fp4.forward_intermediates(ws, M, K, N, A.dtype, q)
    Anp, Wnp = oracle_inputs(A, W)
    ref = oracle.forward(Anp, Wnp, q)
    nnz = int(inter["nnz"].item())
    assert float(inter["T"].item()) == ref["T"]
    assert nnz == ref["nnz"]
    assert np.array_equal(to_np(inter["row_ptr"]), ref["row_ptr"])
    assert np.array_equal(to_np(inter["coo_row"][:nnz]), ref["coo_row"])
    assert np.array_equal(to_np(inter["coo_col"][:nnz]), ref["coo_col"])
    assert np.array_equal(to_np(inter["coo_val"][:nnz]), ref["coo_val"])
    assert np.array_equal(to_np(inter["Aq"]), ref["Aq"])
    assert np.array_equal(to_np(inter["sA"]), ref["sA"])
    assert np.array_equal(to_np(inter["Wq"]), ref["Wq"])
    assert np.array_equal(to_np(inter["sW"]), ref["sW"])
    if out_dtype == torch.float32:
        return assert_y_close(to_np(Y), ref["Y"], ref["denom"])
    assert_bf16_close(to_np(Y), ref["Y"], ref["denom"])
    return None


def test_forward_tiny():
    _say("forward tiny")
    A, W, L = make_layer("tiny")
    err = _check_forward_small(A, W, L.q, torch.float32)
    _say(f"tiny max rel err {err:.3e}")


@pytest.mark.parametrize("dtype,M,K,N,q,out", [
    ("bf16", 300, 512, 264, 0.99, "fp32"), ("bf16", 513, 1056, 776, 0.999, "bf16"),
    ("fp32", 257, 288, 136, 0.95, "fp32"), ("bf16", 1, 32, 8, 0.5, "fp32"), ("bf16", 64, 64, 64, 1.0, "bf16"),
    ("bf16", 520, 2048, 264, 0.9, "fp32"),
    # more rows than one COO workgroup sums for its own offset (the scan launch, then the COO
    # build beside W's quantize pass)
    ("bf16", 16400, 64, 72, 0.99, "bf16"), ("fp32", 16448, 96, 40, 0.995, "fp32"),
])
def test_forward_small(dtype, M, K, N, q, out):
    _say(f"forward {dtype} {M}x{K}x{N} q={q} out={out}")
    A, W = make_custom(M, K, N, dtype=dtype, seed=M + N)
    _check_forward_small(A, W, q, _dt(out))


def _random_forward_cases(n: int = 24, seed: int = 2024):
    """Seeded random shapes within the limits (K % 32 == 0, N % 8 == 0), sized for the oracle:
    ragged against every tile (256-row and 128/256-column GEMM tiles, 64-row COO groups,
    512-column compensation chunks, 128 x 64 escape blocks), both dtypes and output types, and
    quantiles from 0 to 1; a quantile below 0.95 at K >= 640 gives more than 64 entries per row,
    so those cases take the 8-row block compensation."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(rng.integers(1, 1200))
        K = 32 * int(rng.integers(1, 48))
        N = 8 * int(rng.integers(1, 160))
        while M * K * N > 1.5e8:
            M = max(1, M // 2)
        q = float(rng.choice([0.0, 0.5, 0.9, 0.97, 0.99, 0.999, 1.0]))
        dtype = str(rng.choice(["bf16", "fp32"]))
        out = str(rng.choice(["bf16", "fp32"])) if dtype == "bf16" else "fp32"
        kind = str(rng.choice(["normal_sparse_outliers", "student_t", "plain"]))
        cases.append((i, dtype, M, K, N, q, out, kind))
    return cases


@pytest.mark.parametrize("i,dtype,M,K,N,q,out,kind", _random_forward_cases(),
                         ids=lambda v: str(v) if not isinstance(v, float) else f"q{v}")
def test_forward_random_shapes(i, dtype, M, K, N, q, out, kind):
    """Every intermediate (T, nnz, row_ptr, the COO list, Aq, sA, Wq, sW) bit-exact and Y within
    tolerance, on seeded random shapes."""
    _say(f"forward random #{i} {dtype} {M}x{K}x{N} q={q} out={out} {kind}")
    A, W = make_custom(M, K, N, dtype=dtype, seed=500 + i, kind=kind)
    _check_forward_small(A, W, q, _dt(out))


def test_forward_zero_rows_and_columns():
    _say("forward zero rows/cols")
    A, W = make_custom(96, 256, 72, dtype="bf16", seed=3)
    A[5] = 0
    A[7, :100] = -0.0
    W[:, 9] = 0
    _check_forward_small(A, W, 0.99, torch.float32)


def test_forward_is_deterministic():
    _say("determinism")
    A, W = make_custom(1024, 2048, 1032, dtype="bf16", seed=9, kind="student_t")
    Ad, Wd = A.to(DEV), W.to(DEV)
    q = 0.99
    ws1, ws2 = fp4.workspace(Ad, 1032, q, torch.float32).zero_(), fp4.workspace(Ad, 1032, q, torch.float32).zero_()
    Y1 = fp4.linear_forward(Ad, Wd, q, out_dtype=torch.float32, ws=ws1)
    Y2 = fp4.linear_forward(Ad, Wd, q, out_dtype=torch.float32, ws=ws2)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))
    lay = fp4.forward_layout(1024, 2048, 1032, A.dtype, q)
    assert torch.equal(ws1[: lay.scratch], ws2[: lay.scratch])


def test_forward_is_deterministic_wide():
    """The same on the persistent 256 x 256 GEMM (1056 tiles, a ragged last tile column, the two-byte
    hand-over with deferred stores and loads carried from one step to the next): five forwards,
    each Y and each workspace's results bitwise equal to the first's."""
    M, K, N, q = 8192, 4096, 8200, 0.999
    _say(f"determinism wide {M}x{K}x{N}")
    A, W = make_custom(M, K, N, dtype="bf16", seed=29, kind="student_t")
    Ad, Wd = A.to(DEV), W.to(DEV)
    assert fp4.gemm_kernel_name(M, N, K, torch.cuda.get_device_properties(0).multi_processor_count) == "k_fp4_gemm_wide"
    lay = fp4.forward_layout(M, K, N, A.dtype, q)
    # zeroed: parts of the results region (the COO arrays past nnz) are not written
    ws0 = fp4.workspace(Ad, N, q, torch.bfloat16).zero_()
    Y0 = fp4.linear_forward(Ad, Wd, q, out_dtype=torch.bfloat16, ws=ws0).clone()
    r0 = ws0[: lay.scratch].clone()
    ws, Y = fp4.workspace(Ad, N, q, torch.bfloat16).zero_(), torch.empty_like(Y0)
    for _ in range(4):
        fp4.linear_forward(Ad, Wd, q, out_dtype=torch.bfloat16, ws=ws, Y=Y)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y0.view(torch.int16))
        assert torch.equal(ws[: lay.scratch], r0)


@pytest.mark.parametrize("dtype,M,K,N,q,out", [
    ("bf16", 300, 512, 264, 0.99, torch.bfloat16),
    ("fp32", 130, 256, 72, 0.95, torch.float32),
    ("bf16", 1024, 2048, 1032, 0.9, torch.float32),   # many entries per row: the 8-row x 64-column blocks
])
def test_forward_with_cached_weights(dtype, M, K, N, q, out):
    """W quantized once (fp4_quantize per column) and reused: the forward on those codes is
    bit-identical to the forward that quantizes W itself, and both match the oracle."""
    _say(f"forward_wq {dtype} {M}x{K}x{N} q={q}")
    A, W = make_custom(M, K, N, dtype=dtype, seed=21)
    Ad, Wd = A.to(DEV), W.to(DEV)
    Wq, sW = fp4.quantize_weights(Wd)
    Y1 = fp4.linear_forward(Ad, Wd, q, out_dtype=out)
    Y2 = fp4.linear_forward_wq(Ad, Wd, Wq, sW, q, out_dtype=out)
    torch.cuda.synchronize()
    bits = torch.int16 if out == torch.bfloat16 else torch.int32
    assert torch.equal(Y1.view(bits), Y2.view(bits))
    Anp, Wnp = oracle_inputs(A, W)
    ref = oracle.forward(Anp, Wnp, q)
    assert np.array_equal(to_np(Wq), ref["Wq"]) and np.array_equal(to_np(sW), ref["sW"])
    if out == torch.float32:
        assert_y_close(to_np(Y2), ref["Y"], ref["denom"])


@pytest.mark.parametrize("order", ["A_then_W", "W_then_A", "both"])
@pytest.mark.parametrize("dtype,M,K,N,q,out", [("bf16", 300, 512, 264, 0.99, torch.bfloat16),
                                               ("fp32", 130, 256, 72, 0.95, torch.float32)])
def test_forward_in_stage_calls(dtype, M, K, N, q, out, order):
    """fp4_forward_quantize (A and W stages, in either order or together) + fp4_forward_product
    give the same bits as fp4_linear_forward, intermediates included."""
    _say(f"forward stages {order} {dtype} {M}x{K}x{N}")
    A, W = make_custom(M, K, N, dtype=dtype, seed=23)
    Ad, Wd = A.to(DEV), W.to(DEV)
    ws1 = fp4.workspace(Ad, N, q, out)
    Y1 = fp4.linear_forward(Ad, Wd, q, out_dtype=out, ws=ws1)
    ws2 = torch.full_like(ws1, 0x5A)  # stale contents must not matter
    if order == "both":
        fp4.forward_quantize(Ad, Wd, M, K, N, A.dtype, q, ws2)
    else:
        stages = [fp4.FP4_STAGE_A, fp4.FP4_STAGE_W] if order == "A_then_W" else [fp4.FP4_STAGE_W, fp4.FP4_STAGE_A]
        for st in stages:
            fp4.forward_quantize(Ad if st == fp4.FP4_STAGE_A else None, Wd if st == fp4.FP4_STAGE_W else None,
                                 M, K, N, A.dtype, q, ws2, stages=st)
    Y2 = fp4.forward_product(Wd, M, q, ws2, torch.empty_like(Y1))
    torch.cuda.synchronize()
    bits = torch.int16 if out == torch.bfloat16 else torch.int32
    assert torch.equal(Y1.view(bits), Y2.view(bits))
    i1 = fp4.forward_intermediates(ws1, M, K, N, A.dtype, q)
    i2 = fp4.forward_intermediates(ws2, M, K, N, A.dtype, q)
    nnz = int(i1["nnz"].item())
    for k in ("T", "nnz", "row_ptr", "coo_col", "coo_val", "Aq", "sA", "Wq", "sW"):
        a, b = (i1[k][:nnz], i2[k][:nnz]) if k.startswith("coo") else (i1[k], i2[k])
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), k


# ----------------------------------------------------------------------------- FP8 gradient codec
def test_fp8_encoder_sweep():
    """With amax = 448 the multiplier is exactly 1, so the codes are the encoder itself on
    every E4M3 value, every midpoint, their fp32 neighbours and random points."""
    _say("fp8 encoder sweep")
    rng = np.random.default_rng(81)
    vals = np.array([oracle.e4m3_value(b) for b in range(0x7F)], dtype=np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    pts = np.concatenate([vals.astype(np.float32), mids])
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0)),
                          np.exp(rng.uniform(np.log(2.0 ** -14), np.log(448.0), 300000)).astype(np.float32)])
    pts = np.clip(pts, 0, 448).astype(np.float32)
    x = np.concatenate([pts, -pts, np.float32([448.0, -0.0, 0.0])]).astype(np.float32)
    codes, scale = fp4.fp8_quantize(torch.from_numpy(x).to(DEV))
    assert to_np(scale)[0] == 1.0
    assert np.array_equal(to_np(codes), oracle.e4m3_encode(x))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("n,kind", [(1, "normal"), (7, "normal"), (8, "t"), (1000, "t"), ((1 << 20) + 3, "t"),
                                    (4096, "zeros"), (65536, "tiny")])
def test_fp8_codec(dtype, n, kind):
    """Codes, the per-tensor scale and both dequantized outputs bit-exact against the oracle."""
    _say(f"fp8 codec {dtype} n={n} {kind}")
    rng = np.random.default_rng(n + len(kind))
    if kind == "normal":
        x = rng.standard_normal(n).astype(np.float32)
    elif kind == "t":
        x = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
    elif kind == "zeros":
        x = np.zeros(n, dtype=np.float32)
        x[::3] = -0.0
    else:
        x = (rng.standard_normal(n) * 1e-38).astype(np.float32)  # amax below 2^-120: scale 0
    t = torch.from_numpy(x)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    xin = t.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else x
    codes, scale = fp4.fp8_quantize(t.to(DEV))
    ref_codes, ref_s = oracle.fp8_quantize(xin)
    assert to_np(scale)[0] == np.float32(ref_s)
    assert np.array_equal(to_np(codes), ref_codes)
    ref_y = oracle.fp8_dequantize(ref_codes, ref_s)
    y32 = fp4.fp8_dequantize(codes, scale, torch.float32)
    y16 = fp4.fp8_dequantize(codes, scale, torch.bfloat16)
    assert np.array_equal(to_np(y32).view(np.uint32), ref_y.view(np.uint32))
    assert np.array_equal(to_np(y16.view(torch.int16)).view(np.uint16), oracle.to_bf16(ref_y))


def test_fp8_codec_full_size():
    """A gradient the size of the 7B gate+up weight (4096 x 22016 bf16): the scale exactly,
    the codes at sampled positions, and decode(encode) within half an E4M3 spacing."""
    _say("fp8 codec 4096x22016")
    rng = np.random.default_rng(82)
    g = torch.from_numpy((rng.standard_t(3, 4096 * 22016) * 1e-4).astype(np.float32)).to(torch.bfloat16)
    codes, scale = fp4.fp8_quantize(g.to(DEV))
    gf = g.float().numpy()
    amax = np.float32(np.abs(gf).max())
    assert to_np(scale)[0] == np.float32(amax / np.float32(448.0))
    r = np.float32(448.0) / amax
    idx = np.concatenate([rng.integers(0, gf.size, 200000), np.argsort(np.abs(gf))[-64:], [0, gf.size - 1]])
    ref = oracle.e4m3_encode((gf[idx] * r).astype(np.float32))
    assert np.array_equal(to_np(codes)[idx], ref)


# ----------------------------------------------------------------------------- full sizes
def _sample_pairs(rng, M, N, row_ptr, count=3000):
    ms = list(rng.integers(0, M, count))
    ns = list(rng.integers(0, N, count))
    busy = np.argsort(np.diff(row_ptr))[-16:]  # rows with the most outliers
    for m in busy:
        for n in rng.integers(0, N, 8):
            ms.append(int(m))
            ns.append(int(n))
    for (m, n) in [(0, 0), (M - 1, N - 1), (0, N - 1), (M - 1, 0)]:
        ms.append(m)
        ns.append(n)
    return np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)


def _wide_tile_origin(lg, tilesM, tilesN, group=4):
    """(row, col) origin of logical tile lg of the persistent 256 x 256 GEMM: groups of `group`
    tile-rows swept across all tile-columns, column by column."""
    g = min(group, tilesM)
    grp = lg // (g * tilesN)
    first_m = grp * g
    gm = min(g, tilesM - first_m)
    ig = lg - grp * g * tilesN
    return (first_m + ig % gm) * 256, (ig // gm) * 256


def _whole_tiles(M, N, cus):
    """Output tiles compared whole at full size: the first tile, the last (ragged) one, and the
    first and last tile of the first and the last XCD's contiguous range of the persistent
    walk (the first tile of a range is a workgroup's first, whose last pairs are stored during
    its next tile; the last ends a walk and stores at once)."""
    assert fp4.gemm_kernel_name(M, N, 4096, cus) == "k_fp4_gemm_wide"
    tilesM, tilesN = -(-M // 256), -(-N // 256)
    tiles = tilesM * tilesN
    tpx = -(-tiles // 8)
    lgs = {0, tiles - 1, tpx - 1, 7 * tpx, tiles - 1}
    out = {_wide_tile_origin(lg, tilesM, tilesN) for lg in lgs if lg < tiles}
    out.add(((tilesM - 1) * 256, (tilesN - 1) * 256))
    return sorted(out)


FULL = [(w, li) for w in ("llama1.3b_qkv", "llama7b_gate_up", "llama13b_down", "llama7b_block")
        for li in range(len(WORKLOADS[w].layers))]


@pytest.mark.parametrize("wl,li", FULL, ids=[f"{w}-{WORKLOADS[w].layers[li].name}" for w, li in FULL])
def test_forward_full_size(wl, li):
    """The workload sizes, in the launch configuration the benchmark times: every
    intermediate compared in full, the accumulator and Y at sampled outputs."""
    L = WORKLOADS[wl].layers[li]
    _say(f"full size {L.name} M={L.M} K={L.K} N={L.N} q={L.q}")
    A, W, _ = make_layer(wl, li)
    M, K, N = L.M, L.K, L.N
    Ad, Wd = A.to(DEV), W.to(DEV)
    ws = fp4.workspace(Ad, N, L.q, _dt(L.out_dtype))
    Y = fp4.linear_forward(Ad, Wd, L.q, out_dtype=_dt(L.out_dtype), ws=ws)
    inter = fp4.forward_intermediates(ws, M, K, N, A.dtype, L.q)
    nnz = int(inter["nnz"].item())
    Anp, Wnp = oracle_inputs(A, W)
    T = oracle.abs_quantile(Anp, L.q)
    assert float(inter["T"].item()) == T
    cl = oracle.clamp_coo(Anp, T, want_clamped=True, cap=oracle.capacity(M, K, L.q))
    assert nnz == cl["nnz"]
    assert np.array_equal(to_np(inter["row_ptr"]), cl["row_ptr"])
    assert np.array_equal(to_np(inter["coo_row"][:nnz]), cl["coo_row"])
    assert np.array_equal(to_np(inter["coo_col"][:nnz]), cl["coo_col"])
    assert np.array_equal(to_np(inter["coo_val"][:nnz]), cl["coo_val"])
    Aq, sA = oracle.quant_rows(cl.pop("A_clamped"))
    assert np.array_equal(to_np(inter["sA"]), sA)
    assert np.array_equal(to_np(inter["Aq"]), Aq)
    Wq, sW = oracle.quant_cols(Wnp)
    assert np.array_equal(to_np(inter["sW"]), sW)
    assert np.array_equal(to_np(inter["Wq"]), Wq)
    _say(f"  intermediates bit-exact (T={T} nnz={nnz})")
    # fp32 output and raw accumulator from the same codes
    Y32, acc = fp4.gemm(inter["Aq"], inter["sA"], inter["Wq"], inter["sW"], K, row_ptr=inter["row_ptr"],
                        coo_col=inter["coo_col"], coo_val=inter["coo_val"], W=Wd,
                        out_dtype=torch.float32, acc_out=True)
    if L.out_dtype == "bf16":
        assert torch.equal(Y.view(torch.int16), Y32.to(torch.bfloat16).view(torch.int16))
    rng = np.random.default_rng(WORKLOADS[wl].seed_id * 10 + li)
    ms, ns = _sample_pairs(rng, M, N, cl["row_ptr"])
    idx = torch.from_numpy(ms * N + ns).to(DEV)
    g_acc = acc.view(-1)[idx].cpu().numpy()
    g_y = Y32.view(-1)[idx].cpu().numpy()
    r_acc = oracle.accumulate_pairs(Aq, Wq, K, ms, ns)
    assert np.array_equal(g_acc, r_acc)
    r_y, denom = oracle.output_pairs(r_acc, sA, sW, ms, ns, cl["row_ptr"], cl["coo_col"], cl["coo_val"], Wnp)
    err = assert_y_close(g_y, r_y, denom)
    if L.out_dtype == "bf16":
        assert_bf16_close(to_np(Y.view(-1)[idx]), r_y, denom)
    _say(f"  sampled acc bit-exact, Y max err/denom {err:.3e}, plain max |dY|/|Y| {plain_rel_err(g_y, r_y):.3e}")
    # whole 256 x 256 output tiles of the launch the benchmark times
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for (m0, n0) in _whole_tiles(M, N, cus):
        rows, cols = np.arange(m0, min(m0 + 256, M)), np.arange(n0, min(n0 + 256, N))
        tm, tn = np.repeat(rows, cols.size).astype(np.int64), np.tile(cols, rows.size).astype(np.int64)
        t_acc = acc[m0:m0 + rows.size, n0:n0 + cols.size].cpu().numpy().reshape(-1)
        r_acc = oracle.accumulate_pairs(Aq, Wq, K, tm, tn)
        assert np.array_equal(t_acc, r_acc), (m0, n0)
        r_y, denom = oracle.output_pairs(r_acc, sA, sW, tm, tn, cl["row_ptr"], cl["coo_col"], cl["coo_val"], Wnp)
        t_y = Y32[m0:m0 + rows.size, n0:n0 + cols.size].cpu().numpy().reshape(-1)
        e1 = assert_y_close(t_y, r_y, denom, what=f"Y tile ({m0},{n0})")
        _say(f"  tile ({m0},{n0}): acc bit-exact, Y max err/denom {e1:.3e}, plain {plain_rel_err(t_y, r_y):.3e}")
        if L.out_dtype == "bf16":
            assert_bf16_close(to_np(Y[m0:m0 + rows.size, n0:n0 + cols.size]).reshape(-1), r_y, denom,
                              what=f"Y(bf16) tile ({m0},{n0})")
    _say(f"  whole tiles {_whole_tiles(M, N, cus)} match")


@pytest.mark.parametrize("out,M,K", [("bf16", 8192, 512), ("fp32", 8192, 512), ("bf16", 8200, 1024)])
def test_forward_escapes_wide(out, M, K):
    """The forward on the persistent 256 x 256 GEMM (M x K x 8192: 1024 tiles or more) with
    accumulators past the two-byte range (rows of A and channels of W quantizing to +-6
    everywhere: acc = +-36 K): the escape kernel writes the marked blocks' Y from the codes,
    the compensation pass the rest.  Intermediates in full; the accumulator and Y at sampled
    outputs (many in the escaped rows) and over a whole escaped 128 x 128 block.  K = 1024 with
    M = 8200: deferred stores and a ragged row of tiles."""
    N = 8192
    _say(f"forward escapes wide {M}x{K}x{N} out={out}")
    A, W = make_custom(M, K, N, dtype="bf16", seed=41)
    rows, cols = (0, 4000, M - 1), (5, 4100, N - 1)
    for r in rows:
        A[r] = 1.0
    for c in cols:
        W[:, c] = 0.02 if c != 4100 else -0.02
    q = 0.99
    Ad, Wd = A.to(DEV), W.to(DEV)
    ws = fp4.workspace(Ad, N, q, _dt(out))
    Y = fp4.linear_forward(Ad, Wd, q, out_dtype=_dt(out), ws=ws)
    inter = fp4.forward_intermediates(ws, M, K, N, A.dtype, q)
    Anp, Wnp = oracle_inputs(A, W)
    T = oracle.abs_quantile(Anp, q)
    assert float(inter["T"].item()) == T
    cl = oracle.clamp_coo(Anp, T, want_clamped=True, cap=oracle.capacity(M, K, q))
    nnz = cl["nnz"]
    assert int(inter["nnz"].item()) == nnz
    assert np.array_equal(to_np(inter["row_ptr"]), cl["row_ptr"])
    assert np.array_equal(to_np(inter["coo_col"][:nnz]), cl["coo_col"])
    assert np.array_equal(to_np(inter["coo_val"][:nnz]), cl["coo_val"])
    Aq, sA = oracle.quant_rows(cl.pop("A_clamped"))
    Wq, sW = oracle.quant_cols(Wnp)
    assert np.array_equal(to_np(inter["Aq"]), Aq) and np.array_equal(to_np(inter["sA"]), sA)
    assert np.array_equal(to_np(inter["Wq"]), Wq) and np.array_equal(to_np(inter["sW"]), sW)
    rng = np.random.default_rng(43)
    ms, ns = _sample_pairs(rng, M, N, cl["row_ptr"])
    b0, c0 = rows[1] // 128 * 128, cols[1] // 128 * 128  # the aligned block around an escape
    bm, bn = np.meshgrid(np.arange(b0, b0 + 128), np.arange(c0, c0 + 128), indexing="ij")
    ms = np.concatenate([ms, np.repeat(rows, 600), np.repeat(rows, len(cols)), bm.reshape(-1)])
    ns = np.concatenate([ns, rng.integers(0, N, 600 * len(rows)), np.tile(cols, len(rows)), bn.reshape(-1)])
    r_acc = oracle.accumulate_pairs(Aq, Wq, K, ms, ns)
    assert np.abs(r_acc).max() > 8191.75  # the sample holds escaped accumulators
    r_y, denom = oracle.output_pairs(r_acc, sA, sW, ms, ns, cl["row_ptr"], cl["coo_col"], cl["coo_val"], Wnp)
    g_y = to_np(Y.view(-1)[torch.from_numpy(ms * N + ns).to(DEV)])
    if out == "fp32":
        err = assert_y_close(g_y, r_y, denom)
        _say(f"  Y max rel err {err:.3e}")
    else:
        assert_bf16_close(g_y, r_y, denom)


# ----------------------------------------------------------------------------- backward
def _fwd_codes_gpu(Ad, Wd, q):
    M, K = Ad.shape
    N = Wd.shape[1]
    ws = fp4.workspace(Ad, N, q, torch.float32)
    fp4.linear_forward(Ad, Wd, q, out_dtype=torch.float32, ws=ws)
    return fp4.forward_intermediates(ws, M, K, N, Ad.dtype, q)


def _check_backward_small(A, W, dY, q, out_dtype, want_dA=True, want_dW=True):
    M, K = A.shape
    N = W.shape[1]
    Ad, Wd, dYd = A.to(DEV), W.to(DEV), dY.to(DEV)
    inter = _fwd_codes_gpu(Ad, Wd, q)
    Anp, Wnp = oracle_inputs(A, W)
    dYnp = as_numpy_bits(dY)
    ref_f = oracle.forward(Anp, Wnp, q)
    for k in ("Aq", "sA", "Wq", "sW"):  # the backward's inputs agree before it starts
        assert np.array_equal(to_np(inter[k]), ref_f[k]), k
    ws = torch.empty(fp4.backward_layout(M, K, N).total, dtype=torch.uint8, device=DEV)
    dA, dW = fp4.linear_backward(dYd, inter["Aq"], inter["sA"], inter["Wq"], inter["sW"], K, want_dA=want_dA,
                                 want_dW=want_dW, out_dtype=out_dtype, ws=ws)
    torch.cuda.synchronize()
    bi = fp4.backward_intermediates(ws, M, K, N)
    ref = oracle.backward(dYnp, ref_f["Aq"], ref_f["sA"], ref_f["Wq"], ref_f["sW"], K)
    if want_dA:
        for k in ("Gq", "sG", "WqT"):
            assert np.array_equal(to_np(bi[k]), ref[k]), k
        exp = ref["dA"] if out_dtype == torch.float32 else oracle.to_bf16(ref["dA"])
        assert np.array_equal(to_np(dA), exp), "dA"
    else:
        assert dA is None
    if want_dW:
        for k in ("Hq", "sH", "AqT"):
            assert np.array_equal(to_np(bi[k]), ref[k]), k
        exp = ref["dW"] if out_dtype == torch.float32 else oracle.to_bf16(ref["dW"])
        assert np.array_equal(to_np(dW), exp), "dW"
    else:
        assert dW is None


# (dtype, M, K, N, out): M and N multiples of 32 (the two contractions); several GEMM
# tiles with ragged tails in every output dimension; bf16 dY with N up to 24576 takes the fused
# row pass (1, 2 or 3 chunks of 8 per thread of a 1024-thread row), wider rows and fp32 dY the
# separate passes
BWD_CASES = [("bf16", 96, 64, 160, "fp32"), ("fp32", 288, 320, 544, "fp32"), ("bf16", 544, 1056, 800, "bf16"),
             ("bf16", 32, 32, 32, "fp32"), ("fp32", 320, 96, 4128, "bf16"), ("bf16", 64, 64, 16416, "fp32"),
             ("bf16", 96, 32, 24608, "bf16"), ("bf16", 576, 96, 8224, "fp32")]


@pytest.mark.parametrize("dtype,M,K,N,out", BWD_CASES)
def test_backward_small(dtype, M, K, N, out):
    _say(f"backward {dtype} M={M} K={K} N={N} -> {out}")
    A, W = make_custom(M, K, N, dtype=dtype, seed=M + N)
    dY = make_custom_grad(M, N, dtype=dtype, seed=K)
    _check_backward_small(A, W, dY, 0.99, _dt(out))


def _random_backward_cases(n: int = 16, seed: int = 4242):
    """Seeded random shapes for the backward: M, K and N multiples of 32 (the two contractions
    need M and N so); ragged against the GEMM tiles in every output dimension, both dtypes and
    output types, N from 32 to about 26k (a bf16 dY up to 24576 takes the fused row pass, an fp32
    one the separate passes)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = 32 * int(rng.integers(1, 24))
        K = 32 * int(rng.integers(1, 40))
        N = 32 * int(rng.integers(1, 900 if i % 2 else 40))
        while M * K * N > 1.2e8:  # keep N, shrink the others
            if K > 32:
                K = max(32, (K // 2) // 32 * 32)
            else:
                M = max(32, (M // 2) // 32 * 32)
        dtype = str(rng.choice(["bf16", "fp32"]))
        out = str(rng.choice(["bf16", "fp32"]))
        cases.append((i, dtype, M, K, N, out))
    return cases


@pytest.mark.parametrize("i,dtype,M,K,N,out", _random_backward_cases())
def test_backward_random_shapes(i, dtype, M, K, N, out):
    """Gq, sG, Hq, sH, WqT, AqT, dA and dW bit-exact on seeded random shapes."""
    _say(f"backward random #{i} {dtype} M={M} K={K} N={N} -> {out}")
    A, W = make_custom(M, K, N, dtype=dtype, seed=700 + i)
    dY = make_custom_grad(M, N, dtype=dtype, seed=700 + i)
    _check_backward_small(A, W, dY, 0.99, _dt(out))


def test_backward_one_product():
    # dA alone allows any M; dW alone allows N % 8 == 0
    _say("backward dA only (M=300), dW only (N=264)")
    A, W = make_custom(300, 128, 256, dtype="bf16", seed=5)
    _check_backward_small(A, W, make_custom_grad(300, 256, dtype="bf16", seed=5), 0.99, torch.float32,
                          want_dW=False)
    A, W = make_custom(256, 128, 264, dtype="bf16", seed=6)
    _check_backward_small(A, W, make_custom_grad(256, 264, dtype="bf16", seed=6), 0.99, torch.float32,
                          want_dA=False)


def test_backward_zero_gradient_rows_and_columns():
    _say("backward with zero rows and columns of dY")
    A, W = make_custom(128, 64, 96, dtype="bf16", seed=7)
    dY = make_custom_grad(128, 96, dtype="bf16", seed=7)
    dY[5] = 0.0
    dY[:, 17] = 0.0
    _check_backward_small(A, W, dY, 0.99, torch.float32)
    _check_backward_small(A, W, torch.zeros_like(dY), 0.99, torch.float32)


BWD_FULL = [("llama1.3b_qkv", 0), ("llama7b_gate_up", 0), ("llama13b_down", 0)]


@pytest.mark.parametrize("wl,li", BWD_FULL, ids=[f"{w}-{WORKLOADS[w].layers[li].name}" for w, li in BWD_FULL])
def test_backward_full_size(wl, li):
    """The backward at the workload sizes, as the benchmark runs it: every intermediate
    compared in full, dA and dW at sampled outputs."""
    from workloads import make_grad
    L = WORKLOADS[wl].layers[li]
    M, K, N = L.M, L.K, L.N
    _say(f"backward full size {L.name} M={M} K={K} N={N}")
    A, W, _ = make_layer(wl, li)
    dY = make_grad(wl, li)
    Ad, Wd, dYd = A.to(DEV), W.to(DEV), dY.to(DEV)
    inter = _fwd_codes_gpu(Ad, Wd, L.q)
    ws = torch.empty(fp4.backward_layout(M, K, N).total, dtype=torch.uint8, device=DEV)
    dA, dW = fp4.linear_backward(dYd, inter["Aq"], inter["sA"], inter["Wq"], inter["sW"], K,
                                 out_dtype=torch.float32, ws=ws)
    torch.cuda.synchronize()
    Anp, Wnp = oracle_inputs(A, W)
    T = oracle.abs_quantile(Anp, L.q)
    cl = oracle.clamp_coo(Anp, T, want_clamped=True, cap=oracle.capacity(M, K, L.q))
    Aq, sA = oracle.quant_rows(cl.pop("A_clamped"))
    Wq, sW = oracle.quant_cols(Wnp)
    for k, v in (("Aq", Aq), ("sA", sA), ("Wq", Wq), ("sW", sW)):
        assert np.array_equal(to_np(inter[k]), v), k
    rng = np.random.default_rng(100 + WORKLOADS[wl].seed_id)
    count = 2000
    mk = (np.concatenate([rng.integers(0, M, count), [0, M - 1]]), np.concatenate([rng.integers(0, K, count), [0, K - 1]]))
    kn = (np.concatenate([rng.integers(0, K, count), [0, K - 1]]), np.concatenate([rng.integers(0, N, count), [0, N - 1]]))
    ref = oracle.backward_sampled(as_numpy_bits(dY), Aq, sA, Wq, sW, K, mk, kn)
    bi = fp4.backward_intermediates(ws, M, K, N)
    for k in ("Gq", "sG", "Hq", "sH", "WqT", "AqT"):
        assert np.array_equal(to_np(bi[k]), ref[k]), k
    _say("  backward intermediates bit-exact")
    gA = dA.view(-1)[torch.from_numpy(mk[0] * K + mk[1]).to(DEV)].cpu().numpy()
    gW = dW.view(-1)[torch.from_numpy(kn[0] * N + kn[1]).to(DEV)].cpu().numpy()
    assert np.array_equal(gA, ref["dA"])
    assert np.array_equal(gW, ref["dW"])
    _say("  sampled dA and dW bit-exact")
