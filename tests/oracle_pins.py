"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with the
closed form, invariant, library routine or brute force it is checked against.  They
are collected by tests/test_oracle_pins.py and re-run against deliberately broken
builds of the oracle by tests/test_oracle_mutants.py, which requires every planted
mistake to trip at least one of them.

Facts used (sources are the pages on "Optimizing Large Language Model Training Using
FP4 Quantization": the QbitAI report and the paper abstract):
  * E2M1 = 1 sign, 2 exponent, 1 mantissa bit (QbitAI report, format paragraph);
    with bias 1 its decoding is a closed form of the bits.
  * rounding is to the nearest representable value (QbitAI report, forward
    quantization paragraph); IEEE round-half-even on the E2M1 grid is the textbook
    rule with that property, computed here with numpy.rint on the binade spacing.
  * A is scaled per token (row), W per output channel (column) (granularity paragraph).
  * the threshold is a quantile of |A| over the tensor (outlier paragraph):
    numpy.quantile(method="lower"), numpy.sort and torch.kthvalue compute it.
  * dA is non-zero exactly where |a| exceeds the threshold and A_clamped + dA = A
    (outlier paragraph).
  * the product of the quantized operands: float64 matmul of decoded values is exact
    for these magnitudes (every partial sum is a multiple of 1/4 below 2^22).
"""
from __future__ import annotations

from fractions import Fraction

import math

import numpy as np
import torch

import oracle

MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e2m1_closed_form(code: int) -> float:
    """Decode from the bit fields: s eem, bias 1, subnormal when e == 0."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    v = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -v if s else v


def rne_e2m1(y: np.ndarray) -> np.ndarray:
    """Textbook round-half-even onto the E2M1 grid, saturating at 6; returns codes."""
    y = np.asarray(y, dtype=np.float32)
    u = np.abs(y.astype(np.float64))
    spacing = np.where(u < 2.0, 0.5, np.where(u < 4.0, 1.0, 2.0))
    v = np.minimum(np.rint(u / spacing) * spacing, 6.0)
    idx = np.searchsorted(np.array(MAGS), v).astype(np.uint8)
    assert np.array_equal(np.array(MAGS)[idx], v)
    return idx | (np.signbit(y).astype(np.uint8) << 3)


def decode(codes: np.ndarray) -> np.ndarray:
    table = np.array([e2m1_closed_form(c) for c in range(16)], dtype=np.float64)
    return table[codes]


# ------------------------------------------------------------------------- codec pins
def pin_value_table():
    for c in range(16):
        assert oracle.e2m1_value(c) == e2m1_closed_form(c), c
    vals = sorted({abs(e2m1_closed_form(c)) for c in range(16)})
    assert vals == MAGS


def pin_round_trip():
    for c in range(16):
        v = np.float32(e2m1_closed_form(c))
        if c == 8:
            v = np.float32(-0.0)
        assert int(oracle.e2m1_encode([v])[0]) == c, c


def _codec_sweep_points(rng) -> np.ndarray:
    pts = []
    # every bf16 pattern up to 8 in magnitude (both signs)
    b = np.arange(0, 0x4101, dtype=np.uint32) << 16
    pts.append(b.view(np.float32))
    # every midpoint between neighbours, and fp32 neighbours within 3 ulps
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], dtype=np.float32)
    for d in range(-3, 4):
        x = mids.copy()
        for _ in range(abs(d)):
            x = np.nextafter(x, np.float32(np.inf) if d > 0 else np.float32(-np.inf)).astype(np.float32)
        pts.append(x)
    # strided sweep over all fp32 patterns in [0, 7]
    pts.append((np.arange(0, 0x40E00000, 4099, dtype=np.uint32)).view(np.float32))
    pts.append(rng.uniform(0, 7, 200000).astype(np.float32))
    pts.append(np.array([7.0, 12.0, 1e30, 3e38, 1e-30, 1e-45], dtype=np.float32))
    x = np.concatenate(pts)
    return np.concatenate([x, -x])


def pin_encoder_vs_rne():
    x = _codec_sweep_points(np.random.default_rng(7))
    got = oracle.e2m1_encode(x)
    ref = rne_e2m1(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r} got={got[bad[0]]} ref={ref[bad[0]]}"


def pin_encoder_nearest():
    # nearest-value property independent of the tie rule: the chosen value is never
    # farther than any other grid value
    x = np.random.default_rng(3).uniform(-7, 7, 50000).astype(np.float32)
    got = decode(oracle.e2m1_encode(x))
    grid = np.array(sorted({e2m1_closed_form(c) for c in range(16)}))
    best = np.min(np.abs(x.astype(np.float64)[:, None] - grid[None, :]), axis=1)
    assert np.all(np.abs(x.astype(np.float64) - got) == best)


# ------------------------------------------------------------------------- scale pins
HALF_GAP = {0.0: 0.25, 0.5: 0.25, 1.0: 0.25, 1.5: 0.25, 2.0: 0.5, 3.0: 0.5, 4.0: 1.0, 6.0: 1.0}


def _check_quantized_rows(X: np.ndarray, codes: np.ndarray, scales: np.ndarray):
    R, Cn = X.shape
    vals = decode(oracle.unpack_codes(codes, Cn))
    amax = np.max(np.abs(X.astype(np.float64)), axis=1)
    for i in range(R):
        if amax[i] == 0:
            assert scales[i] == 0 and np.all(vals[i] == 0)
            continue
        # scale is amax/6 to within half an ulp of fp32
        assert abs(scales[i] * 6.0 - amax[i]) <= amax[i] * 2.0 ** -23, i
        # the largest-magnitude element lands on +-6 with the element's sign
        j = int(np.argmax(np.abs(X[i])))
        assert vals[i, j] == np.copysign(6.0, X[i, j]), (i, j)
        # dequantization error: at most half the grid gap next to the chosen value
        hg = np.vectorize(HALF_GAP.get)(np.abs(vals[i]))
        err = np.abs(X[i].astype(np.float64) - vals[i] * scales[i])
        assert np.all(err <= (hg + 6 * 2.0 ** -21) * scales[i]), i


def pin_row_scales():
    rng = np.random.default_rng(11)
    X = (rng.standard_normal((64, 96)) * rng.lognormal(0, 1, (64, 1))).astype(np.float32)
    X[5] = 0.0
    codes, scales = oracle.quant_rows(X)
    _check_quantized_rows(X, codes, scales)


def pin_col_scales():
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((96, 40)) * rng.lognormal(0, 1, (1, 40))).astype(np.float32)
    codes, scales = oracle.quant_cols(W)
    # channel-wise: the same as row-wise quantization of W^T
    _check_quantized_rows(np.ascontiguousarray(W.T), codes, scales)


def pin_lossless_rows():
    # rows that are exactly E2M1 values times 2^e with max 6*2^e quantize losslessly
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 16, (16, 64)).astype(np.uint8)
    codes[:, 3] = 7
    e = rng.integers(-10, 10, 16)
    X = (decode(codes) * np.exp2(e)[:, None]).astype(np.float32)
    got, scales = oracle.quant_rows(X)
    assert np.array_equal(scales, np.exp2(e).astype(np.float32))
    assert np.array_equal(oracle.unpack_codes(got, 64), codes)


def pin_nibble_order():
    # element 0 of a row sits in the low nibble of byte 0 (reading: low nibble = even index)
    X = np.zeros((1, 32), dtype=np.float32)
    X[0, 0] = 6.0
    X[0, 1] = 1.0
    codes, _ = oracle.quant_rows(X)
    assert codes[0, 0] == (0x7 | (0x2 << 4))


# ------------------------------------------------------------------------- quantile pins
def pin_quantile_index():
    # double-precision index equals the exact rational floor for the workload shapes
    for n in [128 * 256, 8192 * 2048, 16384 * 4096, 16384 * 13824, 8192 * 4096, 8192 * 11008, 1, 2, 1000]:
        for q in [0.0, 0.5, 0.99, 0.999, 1.0]:
            exact = (Fraction(q) * (n - 1)).numerator // (Fraction(q) * (n - 1)).denominator
            assert oracle.quantile_index(n, q) == exact, (n, q)


def pin_quantile_values():
    rng = np.random.default_rng(21)
    cases = []
    for n in [1, 2, 3, 7, 100, 1001, 65536]:
        cases.append(rng.standard_normal(n).astype(np.float32))
    cases.append(rng.integers(-3, 4, 5000).astype(np.float32))      # heavy ties
    cases.append(np.zeros(300, dtype=np.float32))
    cases.append(np.array([-0.0, 0.0, -0.0], dtype=np.float32))
    bf = torch.from_numpy(rng.standard_normal(40000).astype(np.float32)).to(torch.bfloat16)
    cases.append(bf.view(torch.int16).numpy().view(np.uint16))         # bf16 input, many ties
    for a in cases:
        vals = np.abs(oracle.widen(a).astype(np.float64))
        for q in [0.0, 0.3, 0.5, 0.99, 0.999, 1.0]:
            T = oracle.abs_quantile(a, q)
            k = oracle.quantile_index(a.size, q)
            assert T == np.quantile(vals, q, method="lower"), (a.size, q)
            assert T == np.sort(vals)[k]
            assert T == float(torch.kthvalue(torch.from_numpy(vals), k + 1).values)
            # order-statistic invariant
            assert np.count_nonzero(vals < T) <= k < np.count_nonzero(vals <= T)


# ------------------------------------------------------------------------- clamp pins
def _check_clamp(A: np.ndarray, q: float):
    M, K = A.shape
    T = oracle.abs_quantile(A, q)
    cl = oracle.clamp_coo(A, T)
    a = oracle.widen(A).astype(np.float32)
    nnz = cl["nnz"]
    assert nnz == np.count_nonzero(np.abs(a) > T)
    assert nnz <= oracle.capacity(M, K, q)
    Ac = cl["A_clamped"]
    assert np.all(np.abs(Ac) <= T)
    dense = np.zeros((M, K), dtype=np.float64)
    dense[cl["coo_row"], cl["coo_col"]] = cl["coo_val"]
    assert np.array_equal(dense != 0, np.abs(a) > T)
    # COO sorted by (row, col), unique, and row_ptr consistent
    key = cl["coo_row"].astype(np.int64) * K + cl["coo_col"]
    assert np.all(np.diff(key) > 0)
    assert np.array_equal(np.bincount(cl["coo_row"], minlength=M), np.diff(cl["row_ptr"]))
    # A_clamped + dA reproduces A (exact for bf16 inputs; to half an ulp of delta for fp32)
    recon = Ac.astype(np.float64) + dense
    if A.dtype == np.uint16:
        assert np.array_equal(recon, a.astype(np.float64))
    else:
        tol = np.abs(dense) * 2.0 ** -24
        assert np.all(np.abs(recon - a.astype(np.float64)) <= tol)
    return T, cl


def pin_clamp_fp32_exact_fraction():
    # continuous fp32 data has no ties, so exactly the capacity bound is clamped
    rng = np.random.default_rng(31)
    A = rng.standard_normal((64, 128)).astype(np.float32)
    T, cl = _check_clamp(A, 0.99)
    assert cl["nnz"] == oracle.capacity(64, 128, 0.99)


def pin_clamp_bf16_ties():
    rng = np.random.default_rng(32)
    A = torch.from_numpy(rng.standard_t(3, (96, 160)).astype(np.float32)).to(torch.bfloat16)
    _check_clamp(A.view(torch.int16).numpy().view(np.uint16), 0.99)


def pin_clamp_q1():
    rng = np.random.default_rng(33)
    A = rng.standard_normal((8, 32)).astype(np.float32)
    T, cl = _check_clamp(A, 1.0)
    assert cl["nnz"] == 0 and T == np.max(np.abs(A))


def pin_clamp_signs():
    A = np.array([[10.0, -10.0, 1.0, -1.0]], dtype=np.float32)
    cl = oracle.clamp_coo(A, 2.0)
    assert list(cl["coo_col"]) == [0, 1]
    assert list(cl["coo_val"]) == [8.0, -8.0]
    assert list(cl["A_clamped"][0]) == [2.0, -2.0, 1.0, -1.0]


# ------------------------------------------------------------------------- product pins
def pin_accumulator_vs_matmul():
    rng = np.random.default_rng(41)
    for (M, N, K) in [(5, 7, 32), (9, 4, 96), (16, 16, 256)]:
        ca = rng.integers(0, 16, (M, K)).astype(np.uint8)
        cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
        Aq = (ca[:, 0::2] | (ca[:, 1::2] << 4)).astype(np.uint8)
        Wq = (cw[:, 0::2] | (cw[:, 1::2] << 4)).astype(np.uint8)
        acc = oracle.accumulate(Aq, Wq, K)
        ref = decode(ca) @ decode(cw).T
        assert np.array_equal(acc.astype(np.float64), ref)
        ms = rng.integers(0, M, 20)
        ns = rng.integers(0, N, 20)
        assert np.array_equal(oracle.accumulate_pairs(Aq, Wq, K, ms, ns), acc[ms, ns])


def pin_accumulator_extremes():
    K = 65536
    Aq = np.full((1, K // 2), 0x77, dtype=np.uint8)
    Wq = np.full((2, K // 2), 0x77, dtype=np.uint8)
    Wq[1] = 0xFF
    acc = oracle.accumulate(Aq, Wq, K)
    assert acc[0, 0] == 36.0 * K and acc[0, 1] == -36.0 * K


def _perm_weight(K: int, seed: int):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(K)
    W = np.zeros((K, K), dtype=np.float32)
    W[np.arange(K), perm] = 1.0      # W[k, perm[k]] = 1
    return W, perm


def pin_forward_lossless():
    # quantization is lossless and nothing is clamped -> Y == A @ W exactly
    rng = np.random.default_rng(51)
    M, K, N = 12, 64, 10
    ca = rng.integers(0, 16, (M, K)).astype(np.uint8)
    ca[:, 0] = 7
    cw = rng.integers(0, 16, (K, N)).astype(np.uint8)
    cw[1, :] = 15
    A = (decode(ca) * np.exp2(rng.integers(-4, 4, M))[:, None]).astype(np.float32)
    W = (decode(cw) * np.exp2(rng.integers(-4, 4, N))[None, :]).astype(np.float32)
    out = oracle.forward(A, W, 1.0)
    assert out["nnz"] == 0
    assert np.array_equal(out["Y"].astype(np.float64), A.astype(np.float64) @ W.astype(np.float64))


def pin_forward_permutation():
    # W is a permutation: the product picks columns, the compensation adds dA exactly
    rng = np.random.default_rng(52)
    M, K = 16, 64
    A = rng.standard_normal((M, K)).astype(np.float32)
    A[3, 5] *= 40.0
    A[7, 60] *= -40.0
    W, perm = _perm_weight(K, 53)
    out = oracle.forward(A, W, 0.98)
    T = out["T"]
    inv = np.argsort(perm)
    dense = np.zeros((M, K))
    dense[out["coo_row"], out["coo_col"]] = out["coo_val"]
    vals = decode(oracle.unpack_codes(out["Aq"], K))
    for m in range(M):
        for n in range(K):
            k = inv[n]
            # acc = 6 * value(A code at k); W's scale is fl(1/6)
            assert out["acc"][m, n] == 6.0 * vals[m, k]
            ymain = np.float32(np.float32(out["acc"][m, n] * out["sA"][m]) * out["sW"][n])
            assert out["Y"][m, n] == np.float32(np.float64(ymain) + dense[m, k])
    assert np.count_nonzero(dense) == np.count_nonzero(np.abs(A) > T)


def pin_forward_single_outlier():
    rng = np.random.default_rng(54)
    M, K, N = 8, 64, 24
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    A[2, 17] = 1000.0
    W = rng.standard_normal((K, N)).astype(np.float32)
    q = (M * K - 1.5) / (M * K - 1)        # k = M*K - 2: T = second largest |a|
    base = oracle.forward(A, W, q)
    assert base["nnz"] == 1 and base["coo_row"][0] == 2 and base["coo_col"][0] == 17
    delta = base["coo_val"][0]
    assert delta == np.float32(1000.0 - base["T"])
    A2 = A.copy()
    A2[2, 17] = base["T"]                  # the clamped input has no outlier
    clamped = oracle.forward(A2, W, 1.0)
    assert np.array_equal(clamped["Aq"], base["Aq"]) and np.array_equal(clamped["acc"], base["acc"])
    diff = base["Y"].astype(np.float64) - clamped["Y"].astype(np.float64)
    ref = np.zeros((M, N))
    ref[2] = float(delta) * W[17].astype(np.float64)
    assert np.allclose(diff, ref, rtol=0, atol=2e-6 * (np.abs(base["Y"]).max() + abs(delta)))


def _bruteforce_forward(A: np.ndarray, W: np.ndarray, q: float):
    """Tiny brute force in Python scalars with exact rationals for the product."""
    M, K = A.shape
    N = W.shape[1]
    flat = sorted(abs(float(x)) for x in A.reshape(-1))
    k = int(Fraction(q) * (M * K - 1))
    T = flat[k]
    f32 = np.float32
    grid = sorted({e2m1_closed_form(c) for c in range(16)})

    def nearest(y):
        best = min(grid, key=lambda g: (abs(Fraction(float(y)) - Fraction(g)),
                                        # tie: even mantissa (0, 1, 2, 4, ..)
                                        0 if g in (0.0, 1.0, 2.0, 4.0, -1.0, -2.0, -4.0) else 1))
        return best

    Ac = [[float(f32(T)) * (1 if A[i, j] > 0 else -1) if abs(float(A[i, j])) > T else float(A[i, j])
           for j in range(K)] for i in range(M)]
    dA = [[float(f32(f32(A[i, j]) - f32(Ac[i][j]))) for j in range(K)] for i in range(M)]

    def quant(vec):
        amax = max(abs(v) for v in vec)
        r = f32(6.0) / f32(amax)
        s = f32(amax) / f32(6.0)
        return [nearest(f32(v) * r) for v in vec], s

    qa = [quant(Ac[i]) for i in range(M)]
    qw = [quant([float(W[k_, n]) for k_ in range(K)]) for n in range(N)]
    Y = np.zeros((M, N), dtype=np.float32)
    for i in range(M):
        for n in range(N):
            acc = sum(Fraction(qa[i][0][k_]) * Fraction(qw[n][0][k_]) for k_ in range(K))
            ym = f32(f32(f32(float(acc)) * qa[i][1]) * qw[n][1])
            comp = sum(Fraction(dA[i][k_]) * Fraction(float(W[k_, n])) for k_ in range(K))
            Y[i, n] = f32(float(Fraction(float(ym)) + comp))
    return T, Y


def pin_forward_bruteforce():
    rng = np.random.default_rng(55)
    A = rng.standard_normal((4, 32)).astype(np.float32)
    A[1, 3] *= 30
    A[2, 30] *= -30
    W = (rng.standard_normal((32, 5)) * 0.1).astype(np.float32)
    T, Y = _bruteforce_forward(A, W, 0.97)
    out = oracle.forward(A, W, 0.97)
    assert out["T"] == T
    assert np.array_equal(out["Y"], Y)


def _output_case(w_bf16: bool):
    """Inputs of the output stage built directly: accumulators that are multiples of 1/4,
    distinct scales on every row and column, a (row, col)-sorted dA list with 1 to 6
    entries per row, and more rows than columns (so a row index taken for a column index
    stays in range); W in fp32 or as bf16 bit patterns (with its float32 values)."""
    rng = np.random.default_rng(56 + int(w_bf16))
    M, K, N = 13, 64, 6
    acc = (rng.integers(-4000, 4000, (M, N)) / 4.0).astype(np.float32)
    sA = (rng.uniform(0.5, 2.0, M) * np.exp2(rng.integers(-4, 4, M))).astype(np.float32)
    sW = (rng.uniform(0.5, 2.0, N) * np.exp2(rng.integers(-9, -5, N))).astype(np.float32)
    cnt = rng.integers(1, 7, M)
    cols = [np.sort(rng.choice(K, c, replace=False)) for c in cnt]
    row_ptr = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    coo_col = np.concatenate(cols).astype(np.int32)
    coo_val = (rng.standard_normal(coo_col.size) * 30.0).astype(np.float32)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    Wpass = W
    if w_bf16:
        Wb = torch.from_numpy(W).to(torch.bfloat16)
        W = Wb.float().numpy()
        Wpass = Wb.view(torch.int16).numpy().view(np.uint16)
    assert len(np.unique(sA)) == M and len(np.unique(sW)) == N
    return acc, sA, sW, row_ptr, coo_col, coo_val, W, Wpass


def pin_output_pairs_exact():
    # the sampled output (the Y checker of every full-size comparison) against its
    # definition at (m, n) pairs: Y_main = fl(fl(acc * sA[m]) * sW[n]), then the exact
    # rational sum over row m's dA entries of delta * W[k][n], rounded once to fp32
    f32 = np.float32
    for w_bf16 in (False, True):
        acc, sA, sW, row_ptr, coo_col, coo_val, W, Wpass = _output_case(w_bf16)
        M, N = acc.shape
        rng = np.random.default_rng(57)
        ms = np.concatenate([rng.integers(0, M, 60), [0, M - 1]])
        ns = np.concatenate([rng.integers(0, N, 60), [N - 1, 0]])
        Y, _ = oracle.output_pairs(acc[ms, ns], sA, sW, ms, ns, row_ptr, coo_col, coo_val, Wpass)
        for i, (m, n) in enumerate(zip(ms, ns)):
            ym = f32(f32(acc[m, n] * sA[m]) * sW[n])
            comp = sum(Fraction(float(coo_val[e])) * Fraction(float(W[coo_col[e], n]))
                       for e in range(row_ptr[m], row_ptr[m + 1]))
            assert Y[i] == f32(float(Fraction(float(ym)) + comp)), (w_bf16, m, n)
        # the whole-output form agrees at the same points
        Yall, _ = oracle.output(acc, sA, sW, row_ptr, coo_col, coo_val, Wpass)
        assert np.array_equal(Y, Yall[ms, ns])


def pin_tolerance_denominator():
    # the scale of the Y tolerance: |Y_main| + sum over the row's entries of |delta * W[k][n]|,
    # recomputed in float64 from the dA list, for the whole output and for sampled pairs
    for w_bf16 in (False, True):
        acc, sA, sW, row_ptr, coo_col, coo_val, W, Wpass = _output_case(w_bf16)
        M, N = acc.shape
        ymain = ((acc * sA[:, None]).astype(np.float32) * sW[None, :]).astype(np.float32)
        dense = np.zeros((M, W.shape[0]))
        dense[np.repeat(np.arange(M), np.diff(row_ptr)), coo_col] = coo_val
        ref = np.abs(ymain.astype(np.float64)) + np.abs(dense) @ np.abs(W.astype(np.float64))
        _, d_all = oracle.output(acc, sA, sW, row_ptr, coo_col, coo_val, Wpass)
        assert np.allclose(d_all, ref, rtol=1e-12, atol=0)
        ms, ns = np.arange(M), np.arange(M)[::-1] % N
        _, d = oracle.output_pairs(acc[ms, ns], sA, sW, ms, ns, row_ptr, coo_col, coo_val, Wpass)
        assert np.allclose(d, ref[ms, ns], rtol=1e-12, atol=0)


def pin_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e-3, 65504.0], dtype=np.float32)
    got = oracle.to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    y = np.random.default_rng(5).standard_normal(10000).astype(np.float32)
    assert np.array_equal(oracle.to_bf16(y),
                          torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ----------------------------------------------------------------------------- FP4 held in FP8
# E4M3 values at fixed bit patterns, from the format's definition (bias 7, subnormals at
# exponent field 0, the all-ones pattern NaN, largest finite 448).
E4M3_KNOWN = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0, 0x3C: 1.5,
              0x40: 2.0, 0x44: 3.0, 0x48: 4.0, 0x4C: 6.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}


def pin_e4m3_known_values():
    for b, v in E4M3_KNOWN.items():
        assert oracle.e4m3_value(b) == v, hex(b)
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0 and oracle.e4m3_value(0x80) == 0.0
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))


def pin_e4m3_monotone_and_symmetric():
    pos = [oracle.e4m3_value(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))
    assert all(oracle.e4m3_value(0x80 | b) == -pos[b] for b in range(0x7F))


def pin_e2m1_held_in_e4m3():
    # every E2M1 value, sign included, has an exact E4M3 byte
    for c in range(16):
        b = oracle.e2m1_to_e4m3(c)
        assert 0 <= b < 256, c
        assert oracle.e4m3_value(b) == e2m1_closed_form(c), c
        assert (b >> 7) == (c >> 3), c  # -0 stays -0


def pin_expand_e4m3_order():
    # low nibble first: byte 0x71 holds 0.5 (code 1) then 6 (code 7)
    got = oracle.expand_e4m3(np.array([[0x71, 0x8F]], dtype=np.uint8))
    assert got.tolist() == [[0x30, 0x4C, 0xCC, 0x80]]


# ----------------------------------------------------------------------------- FP8 gradient codec
def _e4m3_sweep_points(rng):
    vals = np.array([oracle.e4m3_value(b) for b in range(0x7F)], dtype=np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    rnd = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 200000)).astype(np.float32)
    x = np.concatenate([pts, up, dn, rnd, np.float32(448.0)[None]])
    x = x[(x >= 0) & (x <= 448)]
    return np.concatenate([x, -x])


def pin_e4m3_encoder_vs_library():
    # torch's float8_e4m3fn cast is round-to-nearest-even on the same grid (it produces NaN
    # instead of saturating above 448, so the sweep stays within range)
    x = _e4m3_sweep_points(np.random.default_rng(71))
    got = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def pin_e4m3_round_trip_and_saturation():
    for b in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert oracle.e4m3_encode([oracle.e4m3_value(b)])[0] == b, hex(b)
    assert oracle.e4m3_encode([449.0, 1e30, -464.0, -1e30]).tolist() == [0x7E, 0x7E, 0xFE, 0xFE]


def pin_fp8_quantize_scale_and_error():
    rng = np.random.default_rng(72)
    g = (rng.standard_t(3, 50000) * 1e-3).astype(np.float32)
    codes, s = oracle.fp8_quantize(g)
    amax = np.float32(np.abs(g).max())
    assert s == np.float32(amax / np.float32(448.0))
    assert (codes & 0x7F).max() == 0x7E  # the largest magnitude maps onto 448
    back = oracle.fp8_dequantize(codes, s)
    # each value within half an E4M3 spacing (relative 2^-4, absolute 2^-10 below 2^-6) of g*r
    r = np.float32(448.0) / amax
    y = np.abs(g.astype(np.float64) * r)
    half = np.maximum(2.0 ** -10, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 4))
    assert np.all(np.abs(back.astype(np.float64) - g.astype(np.float64)) <= (half + 1e-6 * y) * s * 1.0001)


def pin_fp8_zero_and_bf16():
    codes, s = oracle.fp8_quantize(np.array([0.0, -0.0, 0.0], dtype=np.float32))
    assert s == 0.0 and codes.tolist() == [0x00, 0x80, 0x00]
    # bf16 input (as its bit patterns): amax 448 gives r = s = 1, so the codes are the
    # values' own E4M3 bytes
    x = torch.tensor([1.0, -3.5, 448.0, 2.0 ** -9], dtype=torch.bfloat16)
    codes, s = oracle.fp8_quantize(x.view(torch.int16).numpy().view(np.uint16))
    assert s == 1.0 and codes.tolist() == [0x38, 0xC6, 0x7E, 0x01]



# ------------------------------------------------------------------------- backward pins
# Straight-through backward of the quantized product (QbitAI report, backward paragraph:
# the quantizer's own derivative is replaced; here by one): dA = dY . deq(Wq)^T and
# dW = deq(Aq)^T . dY, with the contraction-axis scale folded into dY before dY is
# quantized (per row for dA, per column for dW).
def _unpacked(codes: np.ndarray, cols: int) -> np.ndarray:
    return oracle.unpack_codes(codes, cols)


def pin_transpose_codes():
    rng = np.random.default_rng(61)
    for (R, Cn) in [(2, 2), (6, 10), (64, 96), (34, 130)]:
        c = rng.integers(0, 16, (R, Cn)).astype(np.uint8)
        packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
        t = oracle.transpose_codes(packed, R, Cn)
        assert t.shape == (Cn, R // 2)
        assert np.array_equal(_unpacked(t, R), c.T)          # numpy's transpose of the codes
        assert np.array_equal(oracle.transpose_codes(t, Cn, R), packed)  # an involution


def pin_scaled_quant_axes():
    rng = np.random.default_rng(62)
    X = (rng.standard_normal((24, 64)) * rng.lognormal(0, 1, (24, 1))).astype(np.float32)
    X[4] = 0.0
    # power-of-two multipliers: the scaled matrix is exact, and must quantize like it
    cm = np.exp2(rng.integers(-6, 6, 64)).astype(np.float32)
    codes, scales = oracle.scaled_quant_rows(X, cm)
    _check_quantized_rows(X * cm[None, :], codes, scales)
    rm = np.exp2(rng.integers(-6, 6, 24)).astype(np.float32)
    codes, scales = oracle.scaled_quant_cols(X, rm)
    assert codes.shape == (64, 12)
    _check_quantized_rows(np.ascontiguousarray((rm[:, None] * X).T), codes, scales)
    # general multipliers: the scaled matrix is the fp32 product (numpy's IEEE multiply)
    cm = rng.uniform(0.01, 3.0, 64).astype(np.float32)
    codes, scales = oracle.scaled_quant_rows(X, cm)
    _check_quantized_rows(X * cm[None, :], codes, scales)
    rm = rng.uniform(0.01, 3.0, 24).astype(np.float32)
    codes, scales = oracle.scaled_quant_cols(X, rm)
    _check_quantized_rows(np.ascontiguousarray((rm[:, None] * X).T), codes, scales)
    # bf16 input bits give the same codes as their fp32 values
    xb = torch.from_numpy(X).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.scaled_quant_rows(bits, cm)[0], oracle.scaled_quant_rows(xb.float().numpy(), cm)[0])


def _lossless(rng, shape, axis: int, exps: np.ndarray) -> np.ndarray:
    """E2M1 values times 2^exps along `axis`, with every slice along the other axis
    reaching magnitude 6 * 2^e (so per-slice absmax quantization is lossless)."""
    c = rng.integers(0, 16, shape).astype(np.uint8)
    if axis == 0:   # one exponent per row, each row holds a +-6
        c[np.arange(shape[0]), rng.integers(0, shape[1], shape[0])] = 7
        return decode(c) * np.exp2(exps)[:, None]
    c[rng.integers(0, shape[0], shape[1]), np.arange(shape[1])] = 15
    return decode(c) * np.exp2(exps)[None, :]


def pin_backward_lossless_dA():
    # W and G = dY * sW quantize losslessly -> dA == dY @ W^T exactly (float64 matmul)
    rng = np.random.default_rng(63)
    M, K, N = 10, 64, 96
    e = rng.integers(-4, 5, N)
    f = rng.integers(-4, 5, M)
    W = _lossless(rng, (K, N), 1, e).astype(np.float32)
    u = _lossless(rng, (M, N), 0, np.zeros(M))
    dY = (u * np.exp2(f[:, None] - e[None, :])).astype(np.float32)
    A = rng.standard_normal((M, K)).astype(np.float32)
    Aq, sA = oracle.quant_rows(A)
    Wq, sW = oracle.quant_cols(W)
    assert np.array_equal(sW, np.exp2(e).astype(np.float32))
    ref = dY.astype(np.float64) @ W.astype(np.float64).T
    for d in (dY, torch.from_numpy(dY).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)):
        out = oracle.backward(d, Aq, sA, Wq, sW, K)
        assert np.array_equal(out["sG"], np.exp2(f).astype(np.float32))
        assert np.array_equal(out["dA"].astype(np.float64), ref)


def pin_backward_lossless_dW():
    # A and H = sA * dY quantize losslessly -> dW == A^T @ dY exactly
    rng = np.random.default_rng(64)
    M, K, N = 64, 32, 24
    g = rng.integers(-4, 5, M)
    h = rng.integers(-4, 5, N)
    A = _lossless(rng, (M, K), 0, g).astype(np.float32)
    u = _lossless(rng, (M, N), 1, np.zeros(N))
    dY = (u * np.exp2(h[None, :] - g[:, None])).astype(np.float32)
    W = rng.standard_normal((K, N)).astype(np.float32)
    Aq, sA = oracle.quant_rows(A)
    Wq, sW = oracle.quant_cols(W)
    assert np.array_equal(sA, np.exp2(g).astype(np.float32))
    out = oracle.backward(dY, Aq, sA, Wq, sW, K)
    assert np.array_equal(out["sH"], np.exp2(h).astype(np.float32))
    assert np.array_equal(out["dW"].astype(np.float64), A.astype(np.float64).T @ dY.astype(np.float64))


def pin_backward_decoded_operands():
    # general inputs: each output is the float64 product of the decoded, scaled operands
    # (exact there: every partial sum is a short dyadic) rounded once to fp32
    rng = np.random.default_rng(65)
    M, K, N = 32, 64, 96
    A = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    dY = (rng.standard_normal((M, N)) * 1e-3).astype(np.float32)
    Aq, sA = oracle.quant_rows(A)
    Wq, sW = oracle.quant_cols(W)
    out = oracle.backward(dY, Aq, sA, Wq, sW, K)
    g = decode(_unpacked(out["Gq"], N))
    wv = decode(_unpacked(Wq, K))          # N x K
    dA = (g @ wv) * out["sG"].astype(np.float64)[:, None]
    assert np.array_equal(out["dA"], dA.astype(np.float32))
    av = decode(_unpacked(Aq, K))          # M x K
    hv = decode(_unpacked(out["Hq"], M))   # N x M
    dW = (av.T @ hv.T) * out["sH"].astype(np.float64)[None, :]
    assert np.array_equal(out["dW"], dW.astype(np.float32))
    # and the straight-through products they approximate, to FP4 accuracy
    ref = dY.astype(np.float64) @ (wv.T * sW.astype(np.float64)[None, :]).T
    assert np.linalg.norm(out["dA"] - ref) <= 0.25 * np.linalg.norm(ref)


def pin_backward_sampled():
    # the sampled form (used at full size) on lossless inputs: dA at (m, k) pairs equals
    # the float64 dY @ W^T there, and dW at (k, n) pairs equals A^T @ dY
    rng = np.random.default_rng(66)
    M, K, N = 32, 64, 96
    e, f = rng.integers(-4, 5, N), rng.integers(-4, 5, M)
    W = _lossless(rng, (K, N), 1, e).astype(np.float32)
    dY = (_lossless(rng, (M, N), 0, np.zeros(M)) * np.exp2(f[:, None] - e[None, :])).astype(np.float32)
    A = rng.standard_normal((M, K)).astype(np.float32)
    Aq, sA = oracle.quant_rows(A)
    Wq, sW = oracle.quant_cols(W)
    mk = (rng.integers(0, M, 40), rng.integers(0, K, 40))
    kn = (rng.integers(0, K, 40), rng.integers(0, N, 40))
    out = oracle.backward_sampled(dY, Aq, sA, Wq, sW, K, mk, kn)
    ref = dY.astype(np.float64) @ W.astype(np.float64).T
    assert np.array_equal(out["dA"].astype(np.float64), ref[mk])
    g = rng.integers(-4, 5, M)
    h = rng.integers(-4, 5, N)
    A = _lossless(rng, (M, K), 0, g).astype(np.float32)
    dY = (_lossless(rng, (M, N), 1, np.zeros(N)) * np.exp2(h[None, :] - g[:, None])).astype(np.float32)
    Aq, sA = oracle.quant_rows(A)
    out = oracle.backward_sampled(dY, Aq, sA, Wq, sW, K, mk, kn)
    ref = A.astype(np.float64).T @ dY.astype(np.float64)
    assert np.array_equal(out["dW"].astype(np.float64), ref[kn])

ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
