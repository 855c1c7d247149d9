"""The C ABI on the host: the library loads, exports what include/fp4lin.h declares, and
rejects invalid arguments before any HIP call (no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

import oracle
import quantized_linear_layers_fp4_amd as fp4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4lin.h")

OK, ENULL, ESHAPE, EDTYPE, EQ, ECAP, EWS, EDEV, EHIP, EALIGN, ESCRATCH = range(11)
FAKE = C.c_void_p(0x100000)  # aligned, never dereferenced: validation fails first


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_exports():
    assert declared_symbols() == sorted(fp4.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = fp4.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name


def test_status_strings():
    L = fp4.lib()
    for s in range(10):
        assert L.fp4_status_string(s)
    assert L.fp4_status_string(99) == b"unknown status"


def test_capacity_matches_oracle():
    L = fp4.lib()
    for (M, K, q) in [(128, 256, 0.99), (8192, 2048, 0.99), (16384, 4096, 0.999), (16384, 13824, 0.99),
                      (7, 32, 0.0), (7, 32, 1.0), (1, 32, 0.5)]:
        assert L.fp4_outlier_capacity(M, K, q) == oracle.capacity(M, K, q)
    assert L.fp4_outlier_capacity(16384, 4096, 0.999) == 67109
    assert L.fp4_outlier_capacity(10, 33, 0.5) == -1          # K % 32
    assert L.fp4_outlier_capacity(10, 32, float("nan")) == -1
    assert L.fp4_outlier_capacity(10, 32, 1.5) == -1


@pytest.mark.parametrize("ydt", [fp4.FP4_BF16, fp4.FP4_F32])
def test_forward_layout_is_disjoint_and_aligned(ydt):
    """Regions in order, 256-byte aligned and disjoint; the hand-over is last and the only
    part that depends on Y's type: the escape map alone for a bf16 Y (which holds the two-byte
    accumulators itself), plus the int16 accumulators for an fp32 Y."""
    lay = fp4.WsLayout()
    L = fp4.lib()
    assert L.fp4_forward_layout(300, 512, 264, fp4.FP4_BF16, ydt, 0.99, C.byref(lay)) == OK
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    emap = up(3 * 5)  # one byte per 128 x 64 output block
    hand = emap + (up(300 * 264 * 2) if ydt == fp4.FP4_F32 else 0)
    cap = lay.capacity
    parts = [(lay.T, 4), (lay.nnz, 8), (lay.row_ptr, 301 * 4), (lay.coo_row, cap * 4), (lay.coo_col, cap * 4),
             (lay.coo_val, cap * 4), (lay.Aq, 300 * 256), (lay.sA, 300 * 4), (lay.Wq, 264 * 256),
             (lay.sW, 264 * 4), (lay.scratch, 1), (lay.handoff, hand)]
    parts.sort()
    for (a, na), (b, _) in zip(parts, parts[1:]):
        assert a % 256 == 0 and a + na <= b
    assert parts[-1][0] == lay.handoff and lay.total == lay.handoff + hand
    other = fp4.WsLayout()
    assert L.fp4_forward_layout(300, 512, 264, fp4.FP4_BF16, 1 - ydt, 0.99, C.byref(other)) == OK
    names = ("T", "nnz", "row_ptr", "coo_row", "coo_col", "coo_val", "Aq", "sA", "Wq", "sW", "handoff", "scratch")
    assert all(getattr(lay, n) == getattr(other, n) for n in names)
    assert L.fp4_forward_workspace_bytes(300, 512, 264, fp4.FP4_BF16, ydt, 0.99) == lay.total
    assert L.fp4_forward_workspace_bytes(300, 500, 264, fp4.FP4_BF16, ydt, 0.99) == 0
    assert L.fp4_forward_workspace_bytes(300, 512, 264, fp4.FP4_BF16, 2, 0.99) == 0  # FP4_Q16 is no Y type here


def test_forward_workspace_of_the_gate_up_layer():
    """With a bf16 Y the forward's hand-over is only the escape map: the workspace of the
    16384 x 4096 x 22016 layer is its codes, scales, dA list and scratch (under 0.13 GB)."""
    L = fp4.lib()
    total = L.fp4_forward_workspace_bytes(16384, 4096, 22016, fp4.FP4_BF16, fp4.FP4_BF16, 0.999)
    codes = 16384 * 2048 + 22016 * 2048
    assert codes < total < 0.13e9


@pytest.mark.parametrize("case,expect", [
    ("null_A", ENULL), ("bad_dtype", EDTYPE), ("bad_ydtype", EDTYPE), ("k_not_32", ESHAPE), ("k_too_big", ESHAPE),
    ("k_small", ESHAPE), ("n_not_8", ESHAPE), ("m_zero", ESHAPE), ("q_nan", EQ), ("q_neg", EQ), ("ws_small", EWS),
    ("misaligned", EALIGN),
])
def test_linear_forward_rejects(case, expect):
    L = fp4.lib()
    args = dict(A=FAKE, W=FAKE, dt=fp4.FP4_BF16, M=64, K=128, N=64, q=0.99, Y=FAKE, ydt=fp4.FP4_BF16,
                ws=FAKE, wsb=1 << 40)
    if case == "null_A": args["A"] = None
    if case == "bad_dtype": args["dt"] = 7
    if case == "bad_ydtype": args["ydt"] = -1
    if case == "k_not_32": args["K"] = 100
    if case == "k_too_big": args["K"] = 65536 + 32
    if case == "k_small": args["K"] = 0
    if case == "n_not_8": args["N"] = 100
    if case == "m_zero": args["M"] = 0
    if case == "q_nan": args["q"] = float("nan")
    if case == "q_neg": args["q"] = -0.01
    if case == "ws_small": args["wsb"] = 1024
    if case == "misaligned": args["Y"] = C.c_void_p(0x100004)
    st = L.fp4_linear_forward(args["A"], args["W"], args["dt"], args["M"], args["K"], args["N"], args["q"],
                              args["Y"], args["ydt"], args["ws"], args["wsb"], None)
    assert st == expect


def test_linear_forward_wq_rejects():
    """The pre-quantized-W forward checks its two extra pointers, then everything the plain
    forward checks."""
    L = fp4.lib()
    lay = fp4.WsLayout()
    assert L.fp4_forward_layout(64, 128, 64, fp4.FP4_BF16, fp4.FP4_BF16, 0.99, C.byref(lay)) == OK
    call = lambda **kw: L.fp4_linear_forward_wq(  # noqa: E731
        FAKE, FAKE, kw.get("Wq", FAKE), kw.get("sW", FAKE), fp4.FP4_BF16, 64, kw.get("K", 128), 64, 0.99, FAKE,
        fp4.FP4_BF16, FAKE, kw.get("wsb", lay.total), None)
    assert call(Wq=None) == ENULL
    assert call(sW=None) == ENULL
    assert call(Wq=C.c_void_p(0x100008)) == EALIGN
    assert call(K=100) == ESHAPE
    assert call(wsb=lay.total - 1) == EWS


def test_forward_stage_calls_reject():
    """The two stage calls of the forward check their stage mask, the pointers of the stages
    asked for, and everything the whole forward checks."""
    L = fp4.lib()
    lay = fp4.WsLayout()
    assert L.fp4_forward_layout(64, 128, 64, fp4.FP4_BF16, fp4.FP4_F32, 0.99, C.byref(lay)) == OK
    quant = lambda **kw: L.fp4_forward_quantize(  # noqa: E731
        kw.get("A", FAKE), kw.get("W", FAKE), fp4.FP4_BF16, 64, kw.get("K", 128), 64, kw.get("q", 0.99),
        kw.get("stages", 3), kw.get("ws", FAKE), kw.get("wsb", lay.total), None)
    assert quant(stages=0) == EDTYPE and quant(stages=4) == EDTYPE
    assert quant(A=None) == ENULL and quant(W=None) == ENULL
    assert quant(ws=None) == ENULL
    assert quant(K=100) == ESHAPE
    assert quant(q=1.5) == EQ
    assert quant(wsb=lay.handoff - 1) == EWS  # the quantizer stages use the part before the hand-over
    assert quant(wsb=lay.handoff) not in (EWS, OK)  # past the argument checks (no GPU here)
    assert quant(A=C.c_void_p(0x100004)) == EALIGN
    assert quant(A=C.c_void_p(0x100004), stages=fp4.FP4_STAGE_W) != EALIGN  # A unused: then the device check
    prod = lambda **kw: L.fp4_forward_product(  # noqa: E731
        kw.get("W", FAKE), fp4.FP4_BF16, 64, kw.get("K", 128), 64, 0.99, kw.get("Y", FAKE), kw.get("ydt", 1),
        FAKE, kw.get("wsb", lay.total), None)
    assert prod(W=None) == ENULL and prod(Y=None) == ENULL
    assert prod(ydt=9) == EDTYPE
    assert prod(K=100) == ESHAPE
    assert prod(wsb=16) == EWS
    # an fp32 Y needs the int16 hand-over in the workspace, a bf16 Y only the escape map
    small = L.fp4_forward_workspace_bytes(64, 128, 64, fp4.FP4_BF16, fp4.FP4_BF16, 0.99)
    assert small < lay.total and prod(ydt=0, wsb=small) == EWS and prod(ydt=1, wsb=small) != EWS
    assert prod(Y=C.c_void_p(0x100002)) == EALIGN


def test_fp8_codec_rejects():
    L = fp4.lib()
    wsb = L.fp4_fp8_workspace_bytes()
    assert wsb >= 4
    q = lambda **kw: L.fp4_fp8_quantize(kw.get("X", FAKE), kw.get("dt", 1), kw.get("n", 100), FAKE, FAKE,  # noqa
                                        kw.get("ws", FAKE), kw.get("wsb", wsb), None)
    assert q(X=None) == ENULL
    assert q(dt=2) == EDTYPE
    assert q(n=0) == ESHAPE
    assert q(n=(1 << 40) + 1) == ESHAPE
    assert q(wsb=wsb - 1) == EWS
    assert q(X=C.c_void_p(0x100004)) == EALIGN
    d = lambda **kw: L.fp4_fp8_dequantize(FAKE, kw.get("n", 100), FAKE, kw.get("Y", FAKE),  # noqa
                                          kw.get("dt", 0), None)
    assert d(Y=None) == ENULL
    assert d(dt=9) == EDTYPE
    assert d(n=-1) == ESHAPE
    assert d(Y=C.c_void_p(0x100002)) == EALIGN


def test_quantize_rejects():
    L = fp4.lib()
    c = C.c_void_p
    assert L.fp4_quantize(None, 1, 4, 64, 0, None, FAKE, FAKE, None) == ENULL
    assert L.fp4_quantize(FAKE, 1, 4, 64, 2, None, FAKE, FAKE, None) == EDTYPE
    assert L.fp4_quantize(FAKE, 1, 4, 48, 0, None, FAKE, FAKE, None) == ESHAPE   # C % 32
    assert L.fp4_quantize(FAKE, 1, 48, 64, 1, None, FAKE, FAKE, None) == ESHAPE  # R % 32 for PER_COL
    assert L.fp4_quantize(FAKE, 1, 64, 12, 1, None, FAKE, FAKE, None) == ESHAPE  # C % 8 for PER_COL
    assert L.fp4_quantize(FAKE, 1, 64, 64, 1, FAKE, FAKE, FAKE, None) == EDTYPE  # W is never clamped
    assert L.fp4_quantize(c(0x100002), 1, 4, 64, 0, None, FAKE, FAKE, None) == EALIGN


def test_outlier_clamp_rejects():
    L = fp4.lib()
    M, K, q = 64, 128, 0.99
    cap = L.fp4_outlier_capacity(M, K, q)
    wsb = L.fp4_outlier_workspace_bytes(M, K, fp4.FP4_BF16, q)
    assert wsb > 0
    call = lambda **kw: L.fp4_outlier_clamp(kw.get("A", FAKE), kw.get("dt", 1), M, K, kw.get("q", q), FAKE, FAKE,
                                            FAKE, FAKE, kw.get("cap", cap), FAKE, FAKE, FAKE, kw.get("wsb", wsb), None)
    assert call(A=None) == ENULL
    assert call(dt=3) == EDTYPE
    assert call(q=2.0) == EQ
    assert call(cap=cap - 1) == ECAP
    assert call(wsb=wsb - 1) == EWS


def test_gemm_rejects():
    L = fp4.lib()
    comp = dict(rp=FAKE, cc=FAKE, cv=FAKE, W=FAKE)
    g = lambda **kw: L.fp4_gemm(kw.get("Aq", FAKE), FAKE, FAKE, FAKE, kw.get("M", 64), kw.get("N", 64),
                                kw.get("K", 128), kw.get("rp", None), kw.get("cc", None), kw.get("cv", None), 0,
                                kw.get("W", None), 1, FAKE, kw.get("ydt", 1), None, kw.get("ws", None),
                                kw.get("wsb", 0), None)
    assert g(Aq=None) == ENULL
    assert g(rp=FAKE) == ENULL            # partial compensation arguments
    assert g(rp=FAKE, cc=FAKE) == ENULL
    assert g(rp=FAKE, cc=FAKE, cv=FAKE) == ENULL  # compensation without W
    assert g(**comp) == ENULL             # bf16 Y with compensation needs the escape map
    need = {d: L.fp4_gemm_workspace_bytes(64, 64, d, int(d != 2)) for d in (0, 1, 2)}
    assert need[1] == 256 and need[0] == 64 * 64 * 2 + 256 and need[2] == 64 * 64 * 4 + 256
    assert g(**comp, ws=FAKE, wsb=need[1] - 1) == EWS
    assert g(**comp, ws=C.c_void_p(0x100008), wsb=need[1]) == EALIGN
    assert g(**comp, ydt=0) == ENULL      # so does an fp32 Y (the int16 accumulators)
    assert g(**comp, ydt=0, ws=FAKE, wsb=need[0] - 1) == EWS
    assert g(ydt=2) == ENULL              # the two-byte accumulator output needs its escape buffer
    assert g(ydt=2, ws=FAKE, wsb=need[2] - 1) == EWS
    assert g(**comp, ydt=2, ws=FAKE, wsb=1 << 40) == EDTYPE  # and takes no dA term
    assert g(ydt=5) == EDTYPE
    assert g(K=96 + 16) == ESHAPE
    assert g(N=0) == ESHAPE
    # Wq (N x K/2) must stay below 2^31 bytes, and the compensation's W below 2^31 bytes
    assert g(N=1 << 17, K=32768) == ESHAPE
    assert g(N=1 << 15, K=32768, **comp, ws=FAKE, wsb=1 << 40) == ESHAPE


def test_gemm_workspace_bytes():
    L = fp4.lib()
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    emap = up(3 * 5)  # one byte per 128 x 64 output block: 3 x 5 blocks
    assert L.fp4_gemm_workspace_bytes(300, 264, fp4.FP4_BF16, 1) == emap  # the accumulators go through Y
    assert L.fp4_gemm_workspace_bytes(300, 264, fp4.FP4_BF16, 0) == 0
    assert L.fp4_gemm_workspace_bytes(300, 264, fp4.FP4_F32, 1) == up(300 * 264 * 2) + emap   # int16 accumulators
    assert L.fp4_gemm_workspace_bytes(300, 264, fp4.FP4_F32, 0) == 0
    assert L.fp4_gemm_workspace_bytes(300, 264, fp4.FP4_Q16, 0) == up(300 * 264 * 4) + emap   # fp32 escapes
    assert L.fp4_gemm_workspace_bytes(300, 264, fp4.FP4_Q16, 1) == 0   # no dA term on the raw hand-over
    assert L.fp4_gemm_workspace_bytes(0, 264, fp4.FP4_BF16, 1) == 0
    assert L.fp4_gemm_workspace_bytes(300, 100, fp4.FP4_BF16, 1) == 0


def test_backward_layout_is_disjoint_and_aligned():
    L = fp4.lib()
    lay = fp4.BwdLayout()
    M, K, N = 96, 160, 224
    assert L.fp4_backward_layout(M, K, N, C.byref(lay)) == OK
    parts = sorted([(lay.Gq, M * N // 2), (lay.sG, M * 4), (lay.Hq, N * M // 2), (lay.sH, N * 4),
                    (lay.WqT, K * N // 2), (lay.AqT, K * M // 2), (lay.ones, K * 4), (lay.part, 512 * N * 4)])
    for (a, na), (b, _) in zip(parts, parts[1:]):
        assert a % 256 == 0 and a + na <= b
    assert parts[-1][0] + parts[-1][1] <= lay.total
    assert L.fp4_backward_workspace_bytes(M, K, N) == lay.total
    assert L.fp4_backward_workspace_bytes(M, 100, N) == 0     # K % 32
    assert L.fp4_backward_layout(M, K, N, None) == ENULL


def test_linear_backward_rejects():
    """Checks of the backward: pointers per requested product, dtypes, each product's
    contraction (n for dA, m for dW), workspace and alignment, all before any HIP call."""
    L = fp4.lib()
    M, K, N = 64, 128, 96
    wsb = L.fp4_backward_workspace_bytes(M, K, N)
    assert wsb > 0

    def call(**kw):
        return L.fp4_linear_backward(kw.get("dY", FAKE), kw.get("dt", 1), kw.get("M", M), kw.get("K", K),
                                     kw.get("N", N), kw.get("Aq", FAKE), kw.get("sA", FAKE), kw.get("Wq", FAKE),
                                     kw.get("sW", FAKE), kw.get("dA", FAKE), kw.get("dadt", 1), kw.get("dW", FAKE),
                                     kw.get("dwdt", 0), kw.get("ws", FAKE), kw.get("wsb", wsb), None)
    assert call(dY=None) == ENULL
    assert call(dA=None, dW=None) == ENULL          # nothing asked for
    assert call(Wq=None) == ENULL                   # dA needs Wq and sW
    assert call(sW=None) == ENULL
    assert call(Aq=None) == ENULL                   # dW needs Aq and sA
    assert call(sA=None) == ENULL
    assert call(dA=None, Wq=None, sW=None, wsb=1 << 40) != ENULL  # dW alone does not
    assert call(dt=2) == EDTYPE
    assert call(dadt=3) == EDTYPE
    assert call(dwdt=-1) == EDTYPE
    assert call(N=104) == ESHAPE                    # dA contracts over n: N % 32
    assert call(N=104, dA=None, wsb=1 << 40) not in (ESHAPE, ENULL)  # dW alone: N % 8 suffices
    assert call(M=48) == ESHAPE                     # dW contracts over m: M % 32
    assert call(M=48, dW=None, wsb=1 << 40) not in (ESHAPE, ENULL)   # dA alone: any M
    assert call(M=65536 + 32, dA=None) == ESHAPE    # contraction above 65536
    assert call(K=100) == ESHAPE
    assert call(wsb=wsb - 1) == EWS
    assert call(dA=C.c_void_p(0x100004)) == EALIGN
    assert call(sA=C.c_void_p(0x100004)) == EALIGN


def test_kernel_name_queries():
    # the selection rule, exported so that a benchmark names what runs
    L = fp4.lib()
    assert L.fp4_gemm_kernel_name(16384, 22016, 4096, 256) == b"k_fp4_gemm_wide"
    assert L.fp4_gemm_kernel_name(8192, 6144, 2048, 256) == b"k_fp4_gemm_wide"   # 768 tiles: 3 per CU
    assert L.fp4_gemm_kernel_name(8192, 4096, 4096, 256) == b"k_fp4_gemm_wide"   # 512 tiles: 2 per CU
    assert L.fp4_gemm_kernel_name(8192, 4096, 4096, 257) == b"k_fp4_gemm"        # below 2 per CU
    assert L.fp4_gemm_kernel_name(16384, 22016, 4160, 256) == b"k_fp4_gemm"      # K not a multiple of 512
    assert L.fp4_gemm_kernel_name(128, 128, 256, 256) == b"k_fp4_gemm"
    assert L.fp4_gemm_kernel_name(128, 128, 256, 0) is None
    assert L.fp4_gemm_kernel_name(128, 127, 256, 256) is None
    cap = fp4.outlier_capacity(16384, 4096, 0.999)
    assert L.fp4_comp_kernel_name(16384, cap) == b"k_comp_apply"
    cap = fp4.outlier_capacity(16384, 13824, 0.99)
    assert L.fp4_comp_kernel_name(16384, cap) == b"k_comp_block64"
    assert L.fp4_comp_kernel_name(0, 1) is None


def test_outlier_clamp_noalloc_rejects():
    """The no-allocation variant checks what fp4_outlier_clamp checks, and rejects a problem
    whose scratch exceeds its fixed array with FP4_ERR_SCRATCH, before any HIP call."""
    L = fp4.lib()
    call = lambda **kw: L.fp4_outlier_clamp_noalloc(  # noqa: E731
        kw.get("A", FAKE), fp4.FP4_BF16, kw.get("M", 64), kw.get("K", 128), kw.get("q", 0.99), FAKE, FAKE, FAKE,
        FAKE, kw.get("cap", 1 << 20), kw.get("row_ptr", FAKE), FAKE, None)
    assert call(A=None) == ENULL
    assert call(K=100) == ESHAPE
    assert call(q=float("nan")) == EQ
    assert call(cap=0) == ECAP
    assert call(row_ptr=C.c_void_p(0x100004)) == EALIGN
    big_m, big_k = 65535, 65536  # q = 0.99: 1320 staging slots per row, far beyond 64 MiB
    need = L.fp4_outlier_workspace_bytes(big_m, big_k, fp4.FP4_BF16, 0.99)
    assert need > (64 << 20)
    assert call(M=big_m, K=big_k, cap=fp4.outlier_capacity(big_m, big_k, 0.99)) == ESCRATCH
    assert L.fp4_status_string(ESCRATCH) != L.fp4_status_string(99)
    # the workload shapes fit
    for (m, k, q) in [(16384, 4096, 0.999), (16384, 13824, 0.99), (8192, 11008, 0.99)]:
        assert L.fp4_outlier_workspace_bytes(m, k, fp4.FP4_BF16, q) <= (64 << 20)
