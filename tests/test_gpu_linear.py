"""GPU tests of the accumulating GEMM and of the autograd Fp8Linear layer.

puro_fp8_gemm_accumulate: C + P, one fp32 add per element, where P is what puro_fp8_gemm writes;
checked bit-exactly against that definition (unsplit and split contractions) and, over several
micro-batches, against the oracle's float64 sum within the GEMM tolerance.

Fp8Linear: forward and backward equal the oracle's chain (its quantizers, then its float64
GEMMs) within the GEMM bar (bf16 outputs: plus their own rounding), and stay within the FP8 quantization error of a plain fp32 PyTorch
linear layer (relative Frobenius error below 8%: E4M3 keeps 3 mantissa bits, about 5% RMS per
product of two quantized values).
"""
import numpy as np
import pytest

from gpu_util import bf16_dev, f32_dev, host, normalized_error, say, torch, u8_dev
from oracle import gemm, quant
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
TOL, TIGHT = 1e-3, 1e-4


@pytest.fixture(scope="module")
def P():
    import blockwise_scaled_fp8_quant_amd as P
    assert torch().cuda.is_available(), "GPU test run without a GPU"
    return P


def bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def quantized_case(mode, M, N, K, seed):
    """Operands from the oracle's quantizers on Student-t data (realistic codes and scales)."""
    rng = np.random.default_rng(seed)
    if mode == "WGRAD":
        A, sA = quant.quant_act_128x1(bits(rng.standard_t(3, (K, M)) * 1e-3))
        B, sB = quant.quant_act_128x1(bits(rng.standard_t(3, (K, N))))
    else:
        A, sA = quant.quant_act_1x128(bits(rng.standard_t(3, (M, K))))
        B, sB, _, _ = quant.quant_w_128x128(bits(rng.standard_normal((N, K)) * 0.02))
    return A, sA, B, sB


@pytest.mark.parametrize("mode,M,N,K", [("FWD", 256, 384, 512), ("WGRAD", 384, 256, 1024),
                                         ("WGRAD", 512, 256, 16384), ("DGRAD", 256, 256, 4096)])
def test_accumulate_is_one_fp32_add(P, mode, M, N, K):
    t = torch()
    say(f"[gemm accumulate] {mode} {M}x{N}x{K} splits={'yes' if P.puro_fp8_gemm_workspace_size(P.MODE_NAMES[mode], M, N, K) else 'no'}")
    A, sA, B, sB = quantized_case(mode, M, N, K, M + N + K)
    Ad, sAd, Bd, sBd = u8_dev(A), f32_dev(sA), u8_dev(B), f32_dev(sB)
    prod = host(P.puro_fp8_gemm(mode, Ad, sAd, Bd, sBd, out_dtype=P.OUT_FP32))
    rng = np.random.default_rng(7)
    c0 = (rng.standard_normal((M, N)) * np.abs(prod).mean()).astype(np.float32)
    C = f32_dev(c0)
    P.puro_fp8_gemm_accumulate(mode, Ad, sAd, Bd, sBd, C)
    expect = (c0 + prod).astype(np.float32)          # fp32 + fp32, rounded once
    got = host(C)
    assert (got.view(np.uint32) == expect.view(np.uint32)).all()


def test_accumulate_empty_contraction_keeps_c(P):
    t = torch()
    C = f32_dev(np.arange(256 * 128, dtype=np.float32).reshape(256, 128))
    e8 = t.empty((256, 0), dtype=t.uint8, device="cuda")
    e32 = t.empty((0, 256), dtype=t.float32, device="cuda")
    P.puro_fp8_gemm_accumulate("FWD", e8, e32, t.empty((128, 0), dtype=t.uint8, device="cuda"),
                               t.empty((1, 0), dtype=t.float32, device="cuda"), C)
    assert (host(C) == np.arange(256 * 128, dtype=np.float32).reshape(256, 128)).all()


def test_accumulate_microbatches_match_oracle_sum(P):
    """dW over 3 micro-batches of 2048 tokens, accumulated in fp32, against the float64 sum."""
    M, N, Kmb = 256, 384, 2048
    C = f32_dev(np.zeros((M, N), np.float32))
    ref = np.zeros((M, N))
    na2, nb2 = np.zeros(M), np.zeros(N)
    for mb in range(3):
        A, sA, B, sB = quantized_case("WGRAD", M, N, Kmb, 100 + mb)
        P.puro_fp8_gemm_accumulate("WGRAD", u8_dev(A), f32_dev(sA), u8_dev(B), f32_dev(sB), C)
        ref += gemm.gemm("WGRAD", A, sA, B, sB)
        na, nb = gemm.operand_norms("WGRAD", A, sA, B, sB)
        na2 += na ** 2
        nb2 += nb ** 2
    err, diff, den = normalized_error(host(C), ref, np.sqrt(na2), np.sqrt(nb2))
    say(f"    3 micro-batches: max normalized error {err:.3e}")
    assert err <= TOL and (diff <= TIGHT * den).all()


# --------------------------------------------------------------------------- Fp8Linear

def oracle_layer(xb, wb, gb):
    """The oracle's chain for Y = X W^T and its gradients (float64 results)."""
    xq, xs = quant.quant_act_1x128(xb)
    wq, ws, wqT, wsT = quant.quant_w_128x128(wb)
    y = gemm.gemm("FWD", xq, xs, wq, ws)
    ny = gemm.operand_norms("FWD", xq, xs, wq, ws)
    gq, gs = quant.quant_act_1x128(gb)
    dx = gemm.gemm("DGRAD", gq, gs, wqT, wsT)
    ndx = gemm.operand_norms("DGRAD", gq, gs, wqT, wsT)
    gqT, gsT = quant.quant_act_128x1(gb)
    xqT, xsT = quant.quant_act_128x1(xb)
    dw = gemm.gemm("WGRAD", gqT, gsT, xqT, xsT)
    ndw = gemm.operand_norms("WGRAD", gqT, gsT, xqT, xsT)
    return (y, ny), (dx, ndx), (dw, ndw)


def check_bar(got, ref_norms, what, bf16_out):
    """The GEMM bar on the fp32 result; a bf16 output may add its own rounding (at most 2^-8 |C|,
    taken on the reference with the fp32 accumulator's slack).  With a single 128-deep slice
    (Dout = 128 for dX) one product can carry a whole dot product, and that rounding alone can
    then exceed 1e-3 of the norms' product."""
    ref, (na, nb) = ref_norms
    err, diff, den = normalized_error(got, ref, na, nb)
    say(f"    {what}: max normalized error {err:.3e}")
    rnd = 2.0 ** -8 * np.abs(ref) * (1 + 2.0 ** -7) if bf16_out else 0.0
    assert (diff <= TOL * den + rnd).all(), what
    assert (diff <= TIGHT * den + rnd).all(), what


@pytest.mark.parametrize("lead,din,dout", [((256,), 384, 512), ((2, 128), 256, 640), ((4, 96), 512, 128)])
def test_fp8_linear_matches_oracle_chain(P, lead, din, dout):
    t = torch()
    from blockwise_scaled_fp8_quant_amd.linear import Fp8Linear
    say(f"[Fp8Linear] x {lead + (din,)} -> {dout}")
    rng = np.random.default_rng(din + dout)
    T = int(np.prod(lead))
    xb = bits(rng.standard_t(3, (T, din)))
    gb = bits(rng.standard_t(3, (T, dout)) * 1e-3)
    layer = Fp8Linear(din, dout, device="cuda")
    main = layer.enable_main_grad()
    wb = host(layer.weight.detach().float()).astype(np.float32)
    wb = bits(wb)                                    # exact: the weight already is bf16
    x = bf16_dev(xb).view(*lead, din).requires_grad_(True)
    y = layer(x)
    assert y.shape == (*lead, dout) and y.dtype == t.bfloat16
    y.backward(bf16_dev(gb).view(*lead, dout))
    (ry, rdx, rdw) = oracle_layer(xb, wb, gb)
    check_bar(host(y.reshape(T, dout)), ry, "Y", True)
    check_bar(host(x.grad.reshape(T, din)), rdx, "dX", True)
    check_bar(host(main), rdw, "dW (fp32 main_grad)", False)
    assert layer.weight.grad is None


def test_fp8_linear_grad_without_main_grad(P):
    t = torch()
    from blockwise_scaled_fp8_quant_amd.linear import Fp8Linear
    layer = Fp8Linear(256, 384, device="cuda")
    rng = np.random.default_rng(3)
    x = bf16_dev(bits(rng.standard_normal((256, 256)))).requires_grad_(True)
    gb = bits(rng.standard_normal((256, 384)) * 1e-2)
    layer(x).backward(bf16_dev(gb))
    # the fp32 WGRAD result, stored by autograd in the weight's dtype
    xT, xsT = quant.quant_act_128x1(host(x.detach().view(t.int16)).view(np.uint16))
    gT, gsT = quant.quant_act_128x1(gb)
    ref = gemm.gemm("WGRAD", gT, gsT, xT, xsT)
    na, nb = gemm.operand_norms("WGRAD", gT, gsT, xT, xsT)
    assert layer.weight.grad.dtype == t.bfloat16
    err, diff, den = normalized_error(host(layer.weight.grad), ref, na, nb)
    assert err <= TOL


def test_fp8_linear_close_to_fp32_linear(P):
    """Quantization error against plain fp32 PyTorch (the unquantized layer)."""
    t = torch()
    from blockwise_scaled_fp8_quant_amd.linear import Fp8Linear
    layer = Fp8Linear(1024, 768, device="cuda")
    main = layer.enable_main_grad()
    g = t.Generator(device="cuda")
    g.manual_seed(5)
    x = t.randn((512, 1024), generator=g, device="cuda").to(t.bfloat16).requires_grad_(True)
    dy = (t.randn((512, 768), generator=g, device="cuda") * 1e-2).to(t.bfloat16)
    y = layer(x)
    y.backward(dy)
    xf, wf, dyf = x.detach().float(), layer.weight.detach().float(), dy.float()
    rel = lambda a, b: float(t.linalg.norm(a.detach().float() - b) / t.linalg.norm(b))
    e_y, e_dx, e_dw = rel(y, xf @ wf.T), rel(x.grad, dyf @ wf), rel(main, dyf.T @ xf)
    say(f"    relative Frobenius error vs fp32: Y {e_y:.4f}  dX {e_dx:.4f}  dW {e_dw:.4f}")
    assert e_y < 0.08 and e_dx < 0.08 and e_dw < 0.08


def test_fp8_linear_accumulates_microbatches(P):
    t = torch()
    from blockwise_scaled_fp8_quant_amd.linear import Fp8Linear
    layer = Fp8Linear(256, 256, device="cuda")
    main = layer.enable_main_grad()
    rng = np.random.default_rng(9)
    grads = []
    for mb in range(2):
        x = bf16_dev(bits(rng.standard_normal((128, 256))))
        gb = bf16_dev(bits(rng.standard_normal((128, 256)) * 1e-2))
        layer(x).backward(gb)
        grads.append(host(P.puro_fp8_gemm("WGRAD", *P.puro_fp8_quant_act_128x1(gb), *P.puro_fp8_quant_act_128x1(x),
                                          out_dtype=P.OUT_FP32)))
    expect = (np.float32(0) + grads[0]).astype(np.float32) + grads[1]
    assert (host(main).view(np.uint32) == expect.astype(np.float32).view(np.uint32)).all()


def test_fp8_linear_rejects_ragged_tokens(P):
    from blockwise_scaled_fp8_quant_amd.linear import Fp8Linear
    layer = Fp8Linear(256, 256, device="cuda")
    x = torch().zeros((100, 256), dtype=torch().bfloat16, device="cuda")
    with pytest.raises(P.PuroError):
        layer(x)
