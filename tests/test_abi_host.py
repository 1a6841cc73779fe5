"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

- the shared library loads and exports every entry point include/puro_fp8.h declares;
- version / strerror;
- argument validation: every call below has at least one invalid argument (or an empty
  shape), so the library returns before making any HIP call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "puro_fp8.h")

import blockwise_scaled_fp8_quant_amd as P  # noqa: E402

OK, NULLPTR, SHAPE, ALIGN, LD, MODE, DTYPE, WORKSPACE, HIP, UNSUP = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
A16 = 0x10000          # a fake, 16-byte aligned address: never dereferenced (validation fails first)
MIS = 0x10008          # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(puro_fp8_\w+)\s*\(", src)))


def test_header_and_binding_agree():
    decl = declared_functions()
    assert len(decl) == 16
    assert sorted(P.EXPORTED_SYMBOLS) == decl


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(P.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {P.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_version_and_strerror():
    assert P.puro_fp8_version() >= 100
    for st in (OK, NULLPTR, SHAPE, ALIGN, LD, MODE, DTYPE, WORKSPACE, HIP, UNSUP):
        assert P.puro_fp8_strerror(st) and P.puro_fp8_strerror(st) != "unknown status"
    assert P.puro_fp8_strerror(12345) == "unknown status"


def q1(x=A16, M=256, K=512, ldx=512, q=A16, ldq=512, s=A16):
    return P.lib.puro_fp8_quant_act_1x128(x, M, K, ldx, q, ldq, s, None)


def test_quant_1x128_validation():
    assert q1(M=0) == OK and q1(K=0) == OK
    assert q1(M=-1) == SHAPE and q1(K=100) == SHAPE
    assert q1(x=None) == NULLPTR and q1(q=None) == NULLPTR and q1(s=None) == NULLPTR
    assert q1(x=MIS) == ALIGN and q1(q=MIS) == ALIGN and q1(s=A16 + 4) == ALIGN
    assert q1(ldx=384) == LD and q1(ldq=500) == LD and q1(ldx=516) == LD


def q128x1(x=A16, T=256, C=64, ldx=64, qT=A16, ldqT=256, sT=A16):
    return P.lib.puro_fp8_quant_act_128x1(x, T, C, ldx, qT, ldqT, sT, None)


def test_quant_128x1_validation():
    assert q128x1(T=0) == OK and q128x1(C=0) == OK
    assert q128x1(T=100) == SHAPE and q128x1(C=12) == SHAPE and q128x1(T=-128) == SHAPE
    assert q128x1(x=None) == NULLPTR and q128x1(sT=None) == NULLPTR
    assert q128x1(qT=MIS) == ALIGN
    assert q128x1(ldx=32) == LD and q128x1(ldqT=128) == LD and q128x1(ldqT=264) == LD


def qd(x=A16, T=256, C=256, ldx=256, q=A16, ldq=256, s=A16, qT=A16, ldqT=256, sT=A16):
    return P.lib.puro_fp8_quant_act_dual(x, T, C, ldx, q, ldq, s, qT, ldqT, sT, None)


def test_quant_dual_validation():
    assert qd(T=0) == OK and qd(C=0) == OK
    assert qd(T=100) == SHAPE and qd(C=64) == SHAPE and qd(T=-128) == SHAPE
    for arg in ("x", "q", "s", "qT", "sT"):
        assert qd(**{arg: None}) == NULLPTR, arg
        assert qd(**{arg: MIS}) == ALIGN, arg
    assert qd(ldx=128) == LD and qd(ldq=128) == LD and qd(ldqT=128) == LD
    assert qd(ldx=260) == LD and qd(ldq=264) == LD and qd(ldqT=264) == LD


def qw(w=A16, N=256, K=256, ldw=256, q=A16, ldq=256, s=A16, qT=A16, ldqT=256, sT=A16):
    return P.lib.puro_fp8_quant_w_128x128(w, N, K, ldw, q, ldq, s, qT, ldqT, sT, None)


def test_quant_w_validation():
    assert qw(N=0) == OK
    assert qw(N=200) == SHAPE and qw(K=64) == SHAPE
    assert qw(qT=None) == NULLPTR and qw(sT=None) == NULLPTR and qw(w=None) == NULLPTR
    assert qw(qT=MIS) == ALIGN and qw(w=MIS) == ALIGN
    assert qw(ldw=128) == LD and qw(ldqT=128) == LD and qw(ldq=264) == LD


def wjob(w=A16, N=256, K=256, ldw=256, q=A16, ldq=256, s=A16, qT=A16, ldqT=256, sT=A16):
    return P.WqJob(w, N, K, ldw, q, ldq, s, qT, ldqT, sT)


def qwb(*jobs, n=None):
    arr = (P.WqJob * max(len(jobs), 1))(*jobs)
    return P.lib.puro_fp8_quant_w_128x128_batch(arr, len(jobs) if n is None else n, None)


def test_quant_w_batch_validation():
    # every job is checked as the single-weight call checks it, before anything is launched: each
    # batch below holds at least one failing job (so no kernel runs here)
    assert P.lib.puro_fp8_quant_w_128x128_batch(None, 0, None) == OK
    assert P.lib.puro_fp8_quant_w_128x128_batch(None, 2, None) == NULLPTR
    assert qwb(wjob(), n=17) == UNSUP and qwb(wjob(), n=-1) == UNSUP
    assert qwb(wjob(N=200)) == SHAPE
    assert qwb(wjob(), wjob(K=64)) == SHAPE                       # the second job fails
    assert qwb(wjob(), wjob(), wjob(qT=None)) == NULLPTR
    assert qwb(wjob(N=0), wjob(w=MIS)) == ALIGN                   # an empty job is skipped, not accepted blindly
    assert qwb(wjob(), wjob(ldw=128)) == LD and qwb(wjob(ldq=264), wjob()) == LD
    # the same errors as one call per weight
    for bad in (dict(N=200), dict(qT=None), dict(w=MIS), dict(ldqT=128)):
        assert qwb(wjob(**bad)) == qw(**bad)


def gm(mode=0, M=256, N=256, K=256, A=A16, lda=256, sA=A16, B=A16, ldb=256, sB=A16, C=A16, ldc=256,
       dt=0, ws=None, wsb=0):
    return P.lib.puro_fp8_gemm(mode, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, dt, ws, wsb, None)


def test_gemm_validation():
    assert gm(M=0) == OK and gm(N=0) == OK
    assert gm(mode=3) == MODE and gm(mode=-1) == MODE
    assert gm(dt=2) == DTYPE
    assert gm(M=200) == SHAPE and gm(K=-128) == SHAPE and gm(N=100) == SHAPE
    assert gm(C=None) == NULLPTR and gm(A=None) == NULLPTR and gm(sB=None) == NULLPTR
    assert gm(A=MIS) == ALIGN and gm(C=MIS) == ALIGN and gm(sA=A16 + 4) == ALIGN
    assert gm(lda=128) == LD and gm(ldc=128) == LD and gm(ldb=264) == LD
    assert gm(ldc=262, dt=0) == LD       # 262 * 2 bytes is not a multiple of 16


def test_gemm_validation_fp32_ld_rule():
    # ldc * 4 must be a multiple of 16: 260 qualifies (>= N), 258 does not
    assert gm(ldc=258, dt=1) == LD


def gn(mode=0, M=256, N=256, K=256, A=A16, lda=256, sA=A16, B=A16, ldb=256, sB=A16, C=A16, ldc=256, dt=0):
    return P.lib.puro_fp8_gemm_noalloc(mode, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, dt, None)


def test_gemm_noalloc_validation():
    # the checks of puro_fp8_gemm; partials beyond the library's own buffer are refused
    assert gn(M=0) == OK and gn(N=0) == OK
    assert gn(mode=3) == MODE and gn(mode=9) == MODE and gn(dt=4) == DTYPE
    assert gn(M=200) == SHAPE and gn(C=None) == NULLPTR and gn(B=MIS) == ALIGN and gn(ldc=100) == LD
    M, N, K = 3072, 4096, 65536
    assert P.puro_fp8_gemm_workspace_size(2, M, N, K) > P.SCRATCH_BYTES
    assert gn(mode=2, M=M, N=N, K=K, lda=K, ldb=K, ldc=N, dt=1) == WORKSPACE


def test_gemm_row_stride_limit():
    # each lane's copy offset within an 8-row group, 7 ld + 127, is formed in 32 bits
    big = 1 << 29
    assert gm(lda=big + 16, K=256) == UNSUP and gm(ldb=big + 16) == UNSUP
    assert ga(lda=big + 16) == UNSUP and gq(ldb=big + 16) == UNSUP
    assert mg(lda=big + 16) == UNSUP


def test_gemm_workspace_validation():
    # a long contraction over few tiles needs a workspace; without one the call is refused
    need = P.puro_fp8_gemm_workspace_size(2, 2048, 2048, 16384)
    assert need >= 2 * 2048 * 2048 * 4
    assert gm(mode=2, M=2048, N=2048, K=16384, lda=16384, ldb=16384, ldc=2048) == WORKSPACE
    assert gm(mode=2, M=2048, N=2048, K=16384, lda=16384, ldb=16384, ldc=2048, ws=A16, wsb=need - 1) == WORKSPACE


def test_workspace_query():
    for mode in (0, 1, 2):
        assert P.puro_fp8_gemm_workspace_size(mode, 0, 128, 128) == 0
        assert P.puro_fp8_gemm_workspace_size(mode, 4096, 4096, 2048) >= 0


def ga(mode=2, M=256, N=256, K=256, A=A16, lda=256, sA=A16, B=A16, ldb=256, sB=A16, C=A16, ldc=256,
       ws=None, wsb=0):
    return P.lib.puro_fp8_gemm_accumulate(mode, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, ws, wsb, None)


def test_gemm_accumulate_validation():
    # same checks as puro_fp8_gemm with an fp32 C (ld rule in 4-byte elements)
    assert ga(M=0) == OK and ga(N=0) == OK
    assert ga(mode=5) == MODE
    assert ga(mode=3) == MODE            # the internal MX mode has no accumulating entry point
    assert ga(M=200) == SHAPE and ga(K=-128) == SHAPE
    assert ga(C=None) == NULLPTR and ga(B=None) == NULLPTR
    assert ga(C=MIS) == ALIGN and ga(sB=A16 + 8) == ALIGN
    assert ga(ldc=255) == LD and ga(ldc=258) == LD and ga(lda=100) == LD
    need = P.puro_fp8_gemm_workspace_size(2, 2048, 2048, 16384)
    assert ga(M=2048, N=2048, K=16384, lda=16384, ldb=16384, ldc=2048) == WORKSPACE
    assert ga(M=2048, N=2048, K=16384, lda=16384, ldb=16384, ldc=2048, ws=A16, wsb=need - 1) == WORKSPACE


def mq(x=A16, T=256, C=256, ldx=256, q=A16, ldq=256, xs=A16, qT=A16, ldqT=256, xsT=A16):
    return P.lib.puro_fp8_mx_quant_dual(x, T, C, ldx, q, ldq, xs, qT, ldqT, xsT, None)


def test_mx_quant_validation():
    assert mq(T=0) == OK and mq(C=0) == OK
    assert mq(T=64) == SHAPE and mq(C=96) == SHAPE and mq(T=-128) == SHAPE
    for arg in ("x", "q", "xs", "qT", "xsT"):
        assert mq(**{arg: None}) == NULLPTR, arg
        assert mq(**{arg: MIS}) == ALIGN, arg
    assert mq(ldx=128) == LD and mq(ldq=264) == LD and mq(ldqT=200) == LD


def mg(M=256, N=256, K=256, A=A16, lda=256, xa=A16, B=A16, ldb=256, xb=A16, C=A16, ldc=256, dt=1, ws=None, wsb=0):
    return P.lib.puro_fp8_mx_gemm(M, N, K, A, lda, xa, B, ldb, xb, C, ldc, dt, ws, wsb, None)


def test_mx_gemm_validation():
    assert mg(M=0) == OK and mg(N=0) == OK
    assert mg(dt=3) == DTYPE
    assert mg(K=100) == SHAPE and mg(M=-128) == SHAPE
    assert mg(A=None) == NULLPTR and mg(xb=None) == NULLPTR and mg(C=None) == NULLPTR
    assert mg(xa=MIS) == ALIGN and mg(B=MIS) == ALIGN
    assert mg(lda=128) == LD and mg(ldc=100) == LD
    need = P.puro_fp8_mx_gemm_workspace_size(2048, 2048, 16384)
    assert need > 0
    assert mg(M=2048, N=2048, K=16384, lda=16384, ldb=16384, ldc=2048) == WORKSPACE
    # the internal MX mode is not a public puro_fp8_gemm mode
    assert gm(mode=3) == MODE


def gq(mode=0, M=256, N=256, K=256, A=A16, lda=256, sA=A16, B=A16, ldb=256, sB=A16, C=A16, ldc=256,
       q=A16, ldq=256, s=A16, ws=None, wsb=0):
    return P.lib.puro_fp8_gemm_quant(mode, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, q, ldq, s, ws, wsb, None)


def test_gemm_quant_validation():
    assert gq(M=0) == OK and gq(N=0) == OK
    assert gq(mode=3) == MODE and gq(mode=7) == MODE
    assert gq(N=100) == SHAPE
    assert gq(q=None) == NULLPTR and gq(s=None) == NULLPTR and gq(C=None) == NULLPTR
    assert gq(q=MIS) == ALIGN and gq(s=A16 + 4) == ALIGN
    assert gq(ldq=128) == LD and gq(ldq=264) == LD and gq(ldc=260) == LD


def test_grid_limits_are_reported_not_launched():
    # more than 2^31 - 1 tiles: refused on the host with UNSUPPORTED (nothing is launched)
    T = 128 * (1 << 20)
    C = 128 * 4096
    assert qd(T=T, C=C, ldx=C, ldq=C, ldqT=T) == UNSUP
    assert mq(T=T, C=C, ldx=C, ldq=C, ldqT=T) == UNSUP
    assert q128x1(T=T, C=C, ldx=C, ldqT=T) == UNSUP


def test_cast_validation():
    assert P.lib.puro_fp8_cast_e4m3(A16, 0, A16, None) == OK
    assert P.lib.puro_fp8_cast_e4m3(A16, -1, A16, None) == SHAPE
    assert P.lib.puro_fp8_cast_e4m3(None, 4, A16, None) == NULLPTR
    assert P.lib.puro_fp8_cast_e4m3(MIS, 4, A16, None) == ALIGN


def test_product_path_never_imports_oracle():
    pkg = os.path.join(ROOT, "blockwise_scaled_fp8_quant_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "from oracle" not in src and "import oracle" not in src, f


def test_binding_rejects_host_tensors_before_any_call():
    """The binding checks what the C ABI cannot see (device, dtype, shape, layout) and raises before
    passing a pointer on: a host tensor never reaches the library."""
    import torch
    x = torch.zeros((128, 128), dtype=torch.bfloat16)
    q = torch.zeros((128, 128), dtype=torch.uint8)
    s = torch.zeros((1, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        P.puro_fp8_quant_act_1x128(x)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        P.puro_fp8_quant_act_dual(x)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        P.puro_fp8_quant_w_128x128(x)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        P.puro_fp8_quant_w_128x128_batch([x])
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        P.puro_fp8_gemm(P.FWD, q, s, q, torch.zeros((1, 1)))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        P.puro_fp8_mx_gemm(q, torch.zeros((1, 128, 4), dtype=torch.uint8), q, torch.zeros((1, 128, 4), dtype=torch.uint8))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        P.puro_fp8_cast_e4m3(torch.zeros(16))
    with pytest.raises(ValueError, match="2-D"):
        P.puro_fp8_quant_act_1x128(torch.zeros(128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="contraction length"):
        P.puro_fp8_gemm(P.FWD, q, s, torch.zeros((128, 256), dtype=torch.uint8), torch.zeros((1, 2)))
    with pytest.raises(ValueError, match="out_dtype"):
        P.puro_fp8_gemm(P.FWD, q, s, q, torch.zeros((1, 1)), out_dtype=7)
