"""GPU tests of puro_fp8_gemm_quant: the GEMM with the 1x128 quantization of its bf16 output
fused into the epilogue.

Bars:
  - q, s byte-identical to the oracle's 1x128 quantizer (oracle.quant.quant_act_1x128) applied
    to the bf16 bits of the C the kernel wrote (everywhere on small shapes, on sampled 128-row
    blocks at full size): the fused epilogue quantizes the output it writes;
  - (C, q, s) byte-identical to puro_fp8_gemm's bf16 C followed by puro_fp8_quant_act_1x128(C)
    (the unfused path);
  - C within the GEMM bar against the oracle; q, s reconstruct C within the quantizer's own
    error bound.
"""
import numpy as np
import pytest

from gpu_util import assert_bytes_equal, f32_dev, host, normalized_error, say, torch, u8_dev
from oracle import e4m3, gemm, quant
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def P():
    import blockwise_scaled_fp8_quant_amd as P
    assert torch().cuda.is_available(), "GPU test run without a GPU"
    return P


def bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def operands(mode, M, N, K, seed):
    rng = np.random.default_rng(seed)
    A, sA = quant.quant_act_1x128(bits(rng.standard_t(3, (M, K))))
    if mode == "WGRAD":      # per-row B scales [K/128, N]: the layout of a 1x128 quantization
        B, sB = quant.quant_act_1x128(bits(rng.standard_t(3, (N, K))))
    else:
        B, sB, BT, sBT = quant.quant_w_128x128(bits(rng.standard_normal((N, K)) * 0.02))
    return A, sA, B, sB


def bf16_bits(c_f32: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of values that came back from a bf16 tensor (exact in fp32)."""
    return (np.ascontiguousarray(c_f32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def fused_vs_unfused(P, mode, M, N, K, seed, ldc_pad=0, ldq_pad=0, check_oracle=True):
    t = torch()
    say(f"[gemm quant] {mode} M,N,K={M},{N},{K} splits={'yes' if P.puro_fp8_gemm_workspace_size(P.MODE_NAMES[mode], M, N, K) else 'no'}")
    A, sA, B, sB = operands(mode, M, N, K, seed)
    Ad, sAd, Bd, sBd = u8_dev(A), f32_dev(sA), u8_dev(B), f32_dev(sB)
    Cb = t.full((M, N + ldc_pad), float("nan"), dtype=t.bfloat16, device="cuda")
    qb = t.full((M, N + ldq_pad), 0xA5, dtype=t.uint8, device="cuda")
    s = t.full((N // 128, M), float("nan"), dtype=t.float32, device="cuda")
    P.puro_fp8_gemm_quant(mode, Ad, sAd, Bd, sBd, C=Cb[:, :N], q=qb[:, :N], s=s)
    C2 = P.puro_fp8_gemm(mode, Ad, sAd, Bd, sBd, out_dtype=P.OUT_BF16)
    q2, s2 = P.puro_fp8_quant_act_1x128(C2)
    C, qh = host(Cb), host(qb)
    if ldq_pad:
        assert (qh[:, N:] == 0xA5).all(), "write outside a row of q"
    # the oracle's quantizer on the bf16 output the kernel wrote
    rq, rs = quant.quant_act_1x128(bf16_bits(C[:, :N]))
    assert_bytes_equal(qh[:, :N], rq, "codes vs oracle")
    assert_bytes_equal(host(s), rs, "scales vs oracle")
    assert_bytes_equal(C[:, :N], host(C2), "C")
    assert_bytes_equal(qh[:, :N], host(q2), "codes")
    assert_bytes_equal(host(s), host(s2), "scales")
    if check_oracle:
        ref = gemm.gemm(mode, A, sA, B, sB)
        na, nb = gemm.operand_norms(mode, A, sA, B, sB)
        err, diff, den = normalized_error(C[:, :N], ref, na, nb)
        assert (diff <= TOL * den + 2.0 ** -8 * np.abs(ref) * (1 + 2.0 ** -7)).all()
        # the codes reconstruct C within half an E4M3 ulp of the scaled value (plus fp32 slack)
        sc = np.repeat(host(s).T, 128, axis=1)
        v = C[:, :N] / sc
        d = e4m3.decode(qh[:, :N])
        av = np.abs(v)
        with np.errstate(divide="ignore"):
            ulp = np.where(av >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.where(av > 0, av, 1.0))) - 3), 2.0 ** -9)
        assert (np.abs(v - d) <= ulp / 2 + 2.0 ** -21 * av + 1e-30).all()
    return C


@pytest.mark.parametrize("mode,M,N,K", [("FWD", 256, 384, 512), ("FWD", 384, 256, 2048), ("DGRAD", 512, 640, 1024),
                                        ("FWD", 256, 256, 16384), ("DGRAD", 128, 128, 4096),
                                        ("WGRAD", 256, 384, 1024), ("WGRAD", 256, 256, 8192)])
def test_gemm_quant_matches_unfused(P, mode, M, N, K):
    fused_vs_unfused(P, mode, M, N, K, M + N + K)


def test_gemm_quant_strided(P):
    fused_vs_unfused(P, "FWD", 256, 384, 512, 3, ldc_pad=64, ldq_pad=48)


def test_gemm_quant_empty_contraction(P):
    t = torch()
    C, q, s = P.puro_fp8_gemm_quant("FWD", t.empty((256, 0), dtype=t.uint8, device="cuda"),
                                    t.empty((0, 256), device="cuda"), t.empty((128, 0), dtype=t.uint8, device="cuda"),
                                    t.empty((1, 0), device="cuda"))
    rq, rs = quant.quant_act_1x128(np.zeros((256, 128), np.uint16))
    assert (host(C) == 0).all()
    assert_bytes_equal(host(q), rq, "codes of zeros")
    assert_bytes_equal(host(s), rs, "scales of zeros")


@pytest.mark.parametrize("M,N,K", [(16384, 12288, 2048), (16384, 4096, 2048)])
def test_gemm_quant_full_size(P, M, N, K):
    """At the sweep's FWD shapes: fused == unfused on every byte, and the fused codes and scales of
    sampled 128-row blocks byte-identical to the oracle's quantizer on those rows of the bf16 C
    (C's own parity at these shapes is covered by the full-size sampled GEMM tests)."""
    t = torch()
    say(f"[gemm quant full size] FWD {M}x{N}x{K}")
    g = t.Generator(device="cuda")
    g.manual_seed(M + N)
    A = (t.randn((M, K), generator=g, device="cuda") * 64).clamp(-448, 448).to(t.float8_e4m3fn).view(t.uint8)
    B = (t.randn((N, K), generator=g, device="cuda") * 64).clamp(-448, 448).to(t.float8_e4m3fn).view(t.uint8)
    sA = t.exp2(t.rand((K // 128, M), generator=g, device="cuda") * 8 - 12)
    sB = t.exp2(t.rand((N // 128, K // 128), generator=g, device="cuda") * 8 - 12)
    C, q, s = P.puro_fp8_gemm_quant("FWD", A, sA, B, sB)
    C2 = P.puro_fp8_gemm("FWD", A, sA, B, sB, out_dtype=P.OUT_BF16)
    q2, s2 = P.puro_fp8_quant_act_1x128(C2)
    t.cuda.synchronize()
    assert bool((C.view(t.int16) == C2.view(t.int16)).all())
    assert bool((q == q2).all())
    assert bool((s.view(t.int32) == s2.view(t.int32)).all())
    rng = np.random.default_rng(M + N + K)
    for rb in sorted(rng.choice(M // 128, size=3, replace=False).tolist()):
        rows = slice(128 * rb, 128 * rb + 128)
        cb = C[rows].contiguous().view(t.int16).cpu().numpy().view(np.uint16)
        rq, rs = quant.quant_act_1x128(cb)
        assert_bytes_equal(q[rows].cpu().numpy(), rq, f"codes of rows {128 * rb}.. vs oracle")
        assert_bytes_equal(s[:, rows].contiguous().cpu().numpy(), rs, f"scales of rows {128 * rb}.. vs oracle")
