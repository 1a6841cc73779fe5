"""Full-size GPU parity at the layer-sweep shapes (16384 tokens; weights qkv 4096x2048,
o 2048x2048, gate_up 12288x2048, down 2048x6144): every kernel the benchmark step launches,
at the shapes and in the launch configuration it times, checked on sampled outputs that
the oracle computes one by one.

Inputs are generated on the GPU by torch's seeded generator with the workload's
distributions: activations and gradients Student-t (nu = 3) in bf16, weights N(0, 0.02).
GEMM operands are E4M3 codes from torch's own float8_e4m3fn cast of Student-t data
scaled towards the E4M3 range, with log-uniform fp32 scales.  Only the sampled rows / token
blocks travel to the host, where the oracle computes them.

Bars: quantizers byte-identical on every sampled 128-token block (all 1x128 groups of its
rows, all 128x1 groups of its columns) and 128-row weight block; GEMMs within 1e-3
normalized error (plus the tighter 1e-4 + bf16 rounding bound) on sampled rows x columns.
"""
import numpy as np
import pytest

from gpu_util import assert_bytes_equal, host, normalized_error, say, torch
from oracle import e4m3, gemm, quant

pytestmark = pytest.mark.gpu

TOKENS = 16384
WEIGHTS = [("qkv", 4096, 2048), ("o", 2048, 2048), ("gate_up", 12288, 2048), ("down", 2048, 6144)]
TOL, TIGHT = 1e-3, 1e-4


@pytest.fixture(scope="module")
def P():
    import blockwise_scaled_fp8_quant_amd as P
    assert torch().cuda.is_available(), "GPU test run without a GPU"
    return P


def gen(seed):
    t = torch()
    g = t.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def student_t_bf16(shape, seed, scale=1.0):
    """Student-t (nu = 3) as normal / sqrt(chi2_3 / 3), chi2_3 = sum of 3 squared normals."""
    t = torch()
    g = gen(seed)
    z = t.randn(shape, generator=g, device="cuda")
    c = t.zeros(shape, device="cuda")
    for _ in range(3):
        c += t.randn(shape, generator=g, device="cuda") ** 2
    x = z / t.sqrt(c / 3.0) * scale
    return x.to(t.bfloat16)


def bits_of(x_rows):
    """bf16 device tensor -> uint16 host bits."""
    t = torch()
    return x_rows.contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def token_blocks(T, seed, n=3):
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(T // 128, size=n, replace=False).tolist())


# --------------------------------------------------------------------------- quantizers

@pytest.mark.parametrize("wname,dout,din", WEIGHTS)
def test_dual_quantizer_full_size_sampled(P, wname, dout, din):
    t = torch()
    for what, C, scale, seed in (("X", din, 1.0, 1), ("dY", dout, 1e-3, 2)):
        say(f"[fullsize dual] {wname} {what} {TOKENS}x{C}")
        x = student_t_bf16((TOKENS, C), seed * 100 + dout, scale)
        q, s, qT, sT = P.puro_fp8_quant_act_dual(x)
        t.cuda.synchronize()
        for tb in token_blocks(TOKENS, C + seed):
            rows = slice(128 * tb, 128 * tb + 128)
            xb = bits_of(x[rows])
            rq, rs = quant.quant_act_1x128(xb)
            rqT, rsT = quant.quant_act_128x1(xb)
            assert_bytes_equal(host(q[rows]), rq, f"{what} rows of block {tb}")
            assert_bytes_equal(host(s[:, rows]), rs, f"{what} row scales of block {tb}")
            assert_bytes_equal(host(qT[:, rows]), rqT, f"{what} transposed codes of block {tb}")
            assert_bytes_equal(host(sT[tb:tb + 1]), rsT, f"{what} column scales of block {tb}")


@pytest.mark.parametrize("wname,dout,din", WEIGHTS)
def test_single_quantizers_full_size_sampled(P, wname, dout, din):
    t = torch()
    say(f"[fullsize 1x128 / 128x1] {wname} X {TOKENS}x{din}")
    x = student_t_bf16((TOKENS, din), 7 + din)
    q, s = P.puro_fp8_quant_act_1x128(x)
    qT, sT = P.puro_fp8_quant_act_128x1(x)
    t.cuda.synchronize()
    for tb in token_blocks(TOKENS, din + 11):
        rows = slice(128 * tb, 128 * tb + 128)
        xb = bits_of(x[rows])
        rq, rs = quant.quant_act_1x128(xb)
        rqT, rsT = quant.quant_act_128x1(xb)
        assert_bytes_equal(host(q[rows]), rq, f"1x128 rows of block {tb}")
        assert_bytes_equal(host(s[:, rows]), rs, f"1x128 scales of block {tb}")
        assert_bytes_equal(host(qT[:, rows]), rqT, f"128x1 codes of block {tb}")
        assert_bytes_equal(host(sT[tb:tb + 1]), rsT, f"128x1 scales of block {tb}")


@pytest.mark.parametrize("wname,dout,din", WEIGHTS)
def test_weight_quantizer_full_size_sampled(P, wname, dout, din):
    t = torch()
    say(f"[fullsize 128x128] {wname} W {dout}x{din}")
    g = gen(31 + dout)
    w = (t.randn((dout, din), generator=g, device="cuda") * 0.02).to(t.bfloat16)
    q, s, qT, sT = P.puro_fp8_quant_w_128x128(w)
    t.cuda.synchronize()
    for rb in token_blocks(dout, din, n=2):
        rows = slice(128 * rb, 128 * rb + 128)
        wb = bits_of(w[rows])
        rq, rs, rqT, rsT = quant.quant_w_128x128(wb)
        assert_bytes_equal(host(q[rows]), rq, f"codes of block row {rb}")
        assert_bytes_equal(host(s[rb:rb + 1]), rs, f"scales of block row {rb}")
        assert_bytes_equal(host(qT[:, rows]), rqT, f"transposed codes of block row {rb}")
        assert_bytes_equal(host(sT[:, rb:rb + 1]), rsT, f"transposed scales of block row {rb}")


# --------------------------------------------------------------------------- GEMMs

def e4m3_codes(shape, seed):
    """Codes of Student-t data scaled so that typical tiles use the upper E4M3 range."""
    t = torch()
    x = student_t_bf16(shape, seed, scale=64.0).float().clamp(-448.0, 448.0)
    return x.to(t.float8_e4m3fn).view(t.uint8)


def log_uniform_scales(shape, seed, lo=-14, hi=-2):
    t = torch()
    g = gen(seed)
    return t.exp2(t.rand(shape, generator=g, device="cuda") * (hi - lo) + lo)


def gemm_case(mode, M, N, K, seed):
    A = e4m3_codes((M, K), seed)
    B = e4m3_codes((N, K), seed + 1)
    sA = log_uniform_scales((K // 128, M), seed + 2)
    sB = log_uniform_scales((K // 128, N) if mode == "WGRAD" else (N // 128, K // 128), seed + 3)
    return A, sA, B, sB


@pytest.mark.parametrize("mode", ["FWD", "DGRAD", "WGRAD"])
@pytest.mark.parametrize("wname,dout,din", WEIGHTS)
def test_gemm_full_size_sampled(P, wname, dout, din, mode):
    t = torch()
    M, N, K = {"FWD": (TOKENS, dout, din), "DGRAD": (TOKENS, din, dout), "WGRAD": (dout, din, TOKENS)}[mode]
    out_dtype = P.OUT_FP32 if mode == "WGRAD" else P.OUT_BF16
    say(f"[fullsize gemm] {wname} {mode} M,N,K={M},{N},{K} out={'fp32' if out_dtype else 'bf16'}")
    seed = 1000 * [w[0] for w in WEIGHTS].index(wname) + 10 * ["FWD", "DGRAD", "WGRAD"].index(mode)
    A, sA, B, sB = gemm_case(mode, M, N, K, seed)
    C = torch().empty((M, N), dtype=t.float32 if out_dtype else t.bfloat16, device="cuda")
    P.puro_fp8_gemm(getattr(P, mode), A, sA, B, sB, C=C, out_dtype=out_dtype)
    t.cuda.synchronize()
    rng = np.random.default_rng(M + N + K)
    rows = np.sort(rng.choice(M, size=96, replace=False))
    cols = np.sort(rng.choice(N, size=96, replace=False))
    rt, ct = t.from_numpy(rows).cuda(), t.from_numpy(cols).cuda()
    Ah, sAh = host(A[rt]), host(sA[:, rt])
    Bh = host(B[ct])
    sBh = host(sB[:, ct]) if mode == "WGRAD" else host(sB)
    Ad = gemm.dequant_a(Ah, sAh)
    if mode == "WGRAD":
        Bd = gemm.dequant_b(mode, Bh, sBh)
    else:
        Bd = e4m3.decode(Bh) * np.repeat(sBh[cols // 128].astype(np.float64), 128, axis=1)
    ref = Ad @ Bd.T
    sub = host(C[rt][:, ct])
    na, nb = np.sqrt((Ad * Ad).sum(1)), np.sqrt((Bd * Bd).sum(1))
    err, diff, den = normalized_error(sub, ref, na, nb)
    say(f"    max normalized error {err:.3e}")
    assert err <= TOL
    bound = TIGHT * den + (2.0 ** -8 * np.abs(ref) * (1 + 2.0 ** -7) if out_dtype == P.OUT_BF16 else 0.0)
    assert (diff <= bound).all()
    assert bool(t.isfinite(C).all())


# 8448 x 2048 tiles are 33 x 8 = 264 > one wave of 256: the library runs the first 8192 rows (one
# whole wave of tiles) without a contraction split and splits only the last 256 rows.
ROW_SPLIT = (8448, 2048, 16384)


def row_split_rows(M, seed):
    rng = np.random.default_rng(seed)
    return np.sort(np.concatenate([rng.choice(8192, size=48, replace=False),
                                   8192 + rng.choice(M - 8192, size=48, replace=False)]))


def test_gemm_row_split_sampled(P):
    """WGRAD whose leading whole wave of tiles runs unsplit and whose remaining rows are split:
    sampled rows of both parts within the GEMM bar; the accumulating variant adds C exactly once."""
    t = torch()
    M, N, K = ROW_SPLIT
    say(f"[row split gemm] WGRAD M,N,K={M},{N},{K} (unsplit rows 0..8191, split rows 8192..{M - 1})")
    assert P.puro_fp8_gemm_workspace_size(P.WGRAD, M, N, K) > 0
    A, sA, B, sB = gemm_case("WGRAD", M, N, K, 77)
    C = P.puro_fp8_gemm(P.WGRAD, A, sA, B, sB, out_dtype=P.OUT_FP32)
    C0 = t.randn((M, N), generator=gen(78), device="cuda")
    Cacc = C0.clone()
    P.puro_fp8_gemm_accumulate(P.WGRAD, A, sA, B, sB, Cacc)
    t.cuda.synchronize()
    assert bool((Cacc.view(t.int32) == (C0 + C).view(t.int32)).all()), "accumulate is not C + result"
    rows = row_split_rows(M, 79)
    cols = np.sort(np.random.default_rng(80).choice(N, size=64, replace=False))
    rt, ct = t.from_numpy(rows).cuda(), t.from_numpy(cols).cuda()
    Ad = gemm.dequant_a(host(A[rt]), host(sA[:, rt]))
    Bd = gemm.dequant_b("WGRAD", host(B[ct]), host(sB[:, ct]))
    ref = Ad @ Bd.T
    err, diff, den = normalized_error(host(C[rt][:, ct]), ref, np.sqrt((Ad * Ad).sum(1)), np.sqrt((Bd * Bd).sum(1)))
    say(f"    max normalized error {err:.3e}")
    assert (diff <= TIGHT * den).all()


def test_gemm_row_split_with_exactly_the_documented_workspace(P):
    """A shape whose remaining rows need a larger contraction split than the whole problem
    (2816 x 8192 x 32768 WGRAD: 2048 unsplit rows, then 768 rows split 8 ways): the call runs
    with a workspace of exactly puro_fp8_gemm_workspace_size bytes, and sampled rows of both
    parts are within the GEMM bar."""
    t = torch()
    M, N, K = 2816, 8192, 32768
    need = P.puro_fp8_gemm_workspace_size(P.WGRAD, M, N, K)
    say(f"[row split exact workspace] WGRAD M,N,K={M},{N},{K} workspace {need} B")
    assert need >= 8 * 768 * N * 4
    A, sA, B, sB = gemm_case("WGRAD", M, N, K, 91)
    ws = t.empty(need, dtype=t.uint8, device="cuda")
    C = P.puro_fp8_gemm(P.WGRAD, A, sA, B, sB, out_dtype=P.OUT_FP32, workspace=ws)
    t.cuda.synchronize()
    rng = np.random.default_rng(92)
    rows = np.sort(np.concatenate([rng.choice(2048, size=32, replace=False), 2048 + rng.choice(768, size=32, replace=False)]))
    cols = np.sort(rng.choice(N, size=48, replace=False))
    rt, ct = t.from_numpy(rows).cuda(), t.from_numpy(cols).cuda()
    Ad = gemm.dequant_a(host(A[rt]), host(sA[:, rt]))
    Bd = gemm.dequant_b("WGRAD", host(B[ct]), host(sB[:, ct]))
    ref = Ad @ Bd.T
    err, diff, den = normalized_error(host(C[rt][:, ct]), ref, np.sqrt((Ad * Ad).sum(1)), np.sqrt((Bd * Bd).sum(1)))
    say(f"    max normalized error {err:.3e}")
    assert (diff <= TIGHT * den).all()


def test_gemm_quant_row_split(P):
    """The fused output quantization on a two-part plan (8192 unsplit rows, 256 rows split): C, codes
    and scales equal GEMM-then-quantize everywhere, and sampled 128-row blocks of both parts equal
    the oracle's 1x128 quantizer on the bf16 C."""
    t = torch()
    M, N, K = ROW_SPLIT
    say(f"[row split gemm quant] WGRAD M,N,K={M},{N},{K}")
    A, sA, B, sB = gemm_case("WGRAD", M, N, K, 93)
    C, q, s = P.puro_fp8_gemm_quant(P.WGRAD, A, sA, B, sB)
    C2 = P.puro_fp8_gemm(P.WGRAD, A, sA, B, sB, out_dtype=P.OUT_BF16)
    q2, s2 = P.puro_fp8_quant_act_1x128(C2)
    t.cuda.synchronize()
    assert bool((C.view(t.int16) == C2.view(t.int16)).all())
    assert bool((q == q2).all())
    assert bool((s.view(t.int32) == s2.view(t.int32)).all())
    for rb in (3, 63, 64, 65):                       # blocks 64 and 65 lie in the split part
        rows = slice(128 * rb, 128 * rb + 128)
        rq, rs = quant.quant_act_1x128(bits_of(C[rows]))
        assert_bytes_equal(host(q[rows]), rq, f"codes of rows {128 * rb}..")
        assert_bytes_equal(host(s[:, rows]), rs, f"scales of rows {128 * rb}..")


def test_mx_gemm_row_split_sampled(P):
    from oracle import mx
    t = torch()
    M, N, K = ROW_SPLIT
    say(f"[row split mx gemm] M,N,K={M},{N},{K}")
    A, B = e4m3_codes((M, K), 81), e4m3_codes((N, K), 82)
    g = gen(83)
    xa = t.randint(115, 136, (K // 128, M, 4), generator=g, device="cuda", dtype=t.uint8)
    xb = t.randint(115, 136, (K // 128, N, 4), generator=g, device="cuda", dtype=t.uint8)
    C = P.puro_fp8_mx_gemm(A, xa, B, xb, out_dtype=P.OUT_FP32)
    t.cuda.synchronize()
    rows = row_split_rows(M, 84)
    cols = np.sort(np.random.default_rng(85).choice(N, size=64, replace=False))
    rt, ct = t.from_numpy(rows).cuda(), t.from_numpy(cols).cuda()
    Ad = mx.dequant(host(A[rt]), host(xa[:, rt]))
    Bd = mx.dequant(host(B[ct]), host(xb[:, ct]))
    ref = Ad @ Bd.T
    err, diff, den = normalized_error(host(C[rt][:, ct]), ref, np.sqrt((Ad * Ad).sum(1)), np.sqrt((Bd * Bd).sum(1)))
    say(f"    max normalized error {err:.3e}")
    assert (diff <= TOL * den).all()


# --------------------------------------------------------------------------- MXFP8 variant

@pytest.mark.parametrize("wname,dout,din", WEIGHTS)
def test_mx_dual_quantizer_full_size_sampled(P, wname, dout, din):
    from oracle import mx
    t = torch()
    for what, C, scale, seed in (("X", din, 1.0, 3), ("dY", dout, 1e-3, 4)):
        say(f"[fullsize mx dual] {wname} {what} {TOKENS}x{C}")
        x = student_t_bf16((TOKENS, C), seed * 100 + dout, scale)
        q, xs, qT, xsT = P.puro_fp8_mx_quant_dual(x)
        t.cuda.synchronize()
        for tb in token_blocks(TOKENS, C + seed, n=2):
            rows = slice(128 * tb, 128 * tb + 128)
            xb = bits_of(x[rows])
            rq, rxs = mx.quant_rows(xb)
            rqT, rxsT = mx.quant_cols(xb)
            assert_bytes_equal(host(q[rows]), rq, f"{what} MX rows of block {tb}")
            assert_bytes_equal(host(xs[:, rows]), rxs, f"{what} MX row scales of block {tb}")
            assert_bytes_equal(host(qT[:, rows]), rqT, f"{what} MX transposed codes of block {tb}")
            assert_bytes_equal(host(xsT[tb:tb + 1]), rxsT, f"{what} MX column scales of block {tb}")


@pytest.mark.parametrize("mode", ["FWD", "DGRAD", "WGRAD"])
@pytest.mark.parametrize("wname,dout,din", WEIGHTS)
def test_mx_gemm_full_size_sampled(P, wname, dout, din, mode):
    from oracle import mx
    t = torch()
    M, N, K = {"FWD": (TOKENS, dout, din), "DGRAD": (TOKENS, din, dout), "WGRAD": (dout, din, TOKENS)}[mode]
    out_dtype = P.OUT_FP32 if mode == "WGRAD" else P.OUT_BF16
    say(f"[fullsize mx gemm] {wname} {mode} M,N,K={M},{N},{K}")
    seed = 500 + 1000 * [w[0] for w in WEIGHTS].index(wname) + 10 * ["FWD", "DGRAD", "WGRAD"].index(mode)
    A, B = e4m3_codes((M, K), seed), e4m3_codes((N, K), seed + 1)
    g = gen(seed + 2)
    xa = t.randint(115, 136, (K // 128, M, 4), generator=g, device="cuda", dtype=t.uint8)
    xb = t.randint(115, 136, (K // 128, N, 4), generator=g, device="cuda", dtype=t.uint8)
    C = P.puro_fp8_mx_gemm(A, xa, B, xb, out_dtype=out_dtype)
    t.cuda.synchronize()
    rng = np.random.default_rng(M + N + K + 1)
    rows = np.sort(rng.choice(M, size=96, replace=False))
    cols = np.sort(rng.choice(N, size=96, replace=False))
    rt, ct = t.from_numpy(rows).cuda(), t.from_numpy(cols).cuda()
    Ad = mx.dequant(host(A[rt]), host(xa[:, rt]))
    Bd = mx.dequant(host(B[ct]), host(xb[:, ct]))
    ref = Ad @ Bd.T
    sub = host(C[rt][:, ct])
    na, nb = np.sqrt((Ad * Ad).sum(1)), np.sqrt((Bd * Bd).sum(1))
    err, diff, den = normalized_error(sub, ref, na, nb)
    say(f"    max normalized error {err:.3e}")
    rnd = 2.0 ** -8 * np.abs(ref) * (1 + 2.0 ** -7) if out_dtype == P.OUT_BF16 else 0.0
    assert (diff <= TOL * den + rnd).all()
    assert bool(t.isfinite(C).all())
