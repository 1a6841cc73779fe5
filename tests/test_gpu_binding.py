"""GPU tests of the Python binding's argument checks: what the C ABI cannot see from a pointer
(element type, shape, row layout of a device tensor) is rejected before anything is launched,
and the outputs the caller passed are left untouched."""
import pytest

from gpu_util import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import blockwise_scaled_fp8_quant_amd as P
    assert torch().cuda.is_available(), "GPU test run without a GPU"
    return P


def test_wrong_dtype_shape_and_layout_are_rejected(P):
    t = torch()
    x = t.randn((256, 512), device="cuda").to(t.bfloat16)
    with pytest.raises(TypeError, match="dtype"):
        P.puro_fp8_quant_act_1x128(x.float())
    with pytest.raises(ValueError, match="shape"):
        P.puro_fp8_quant_act_1x128(x, s=t.empty((4, 128), device="cuda"))
    with pytest.raises(ValueError, match="unit element stride"):
        P.puro_fp8_quant_act_1x128(x.t().contiguous().t())           # column-major view
    with pytest.raises(ValueError, match="contiguous"):
        P.puro_fp8_quant_act_1x128(x, s=t.empty((256, 4), device="cuda").t())
    q = t.full((256, 512), 0x5A, dtype=t.uint8, device="cuda")
    with pytest.raises(ValueError, match="shape"):
        P.puro_fp8_quant_act_dual(x, q=q, s=t.empty((4, 256), device="cuda"), qT=t.empty((256, 512), dtype=t.uint8,
                                                                                        device="cuda"))
    t.cuda.synchronize()
    assert bool((q == 0x5A).all()), "a rejected call wrote its output"


def test_gemm_operand_checks(P):
    t = torch()
    A = t.zeros((256, 256), dtype=t.uint8, device="cuda")
    B = t.zeros((384, 256), dtype=t.uint8, device="cuda")
    sA = t.ones((2, 256), device="cuda")
    sB = t.ones((3, 2), device="cuda")
    C = P.puro_fp8_gemm(P.FWD, A, sA, B, sB)                          # valid: zeros
    t.cuda.synchronize()
    assert C.shape == (256, 384) and bool((C == 0).all())
    with pytest.raises(ValueError, match="sB"):
        P.puro_fp8_gemm(P.WGRAD, A, sA, B, sB)                       # WGRAD wants sB [K/128, N]
    with pytest.raises(TypeError, match="C"):
        P.puro_fp8_gemm(P.FWD, A, sA, B, sB, C=t.empty((256, 384), device="cuda"), out_dtype=P.OUT_BF16)
    with pytest.raises(TypeError, match="dtype"):
        P.puro_fp8_gemm(P.FWD, A.to(t.int8), sA, B, sB)
    with pytest.raises(ValueError, match="shape"):
        P.puro_fp8_mx_gemm(A, t.zeros((2, 256, 2), dtype=t.uint8, device="cuda"),
                           B, t.zeros((2, 384, 4), dtype=t.uint8, device="cuda"))
    with pytest.raises(ValueError, match="needs the fp32 tensor"):
        P.puro_fp8_gemm_accumulate(P.WGRAD, A, sA, B, t.ones((2, 384), device="cuda"), None)
