"""GPU test of puro_fp8_gemm_noalloc, the GEMM entry point that allocates nothing (its contraction
split keeps partial sums in the library's own per-device buffer): called through the C ABI, its
output must equal puro_fp8_gemm's for the same arguments bit for bit (same kernels, same plan, and
the split-K reduction runs in a fixed order), on calls in a row whose second problem is smaller
than the first, so the second reads a buffer that still holds the first call's partials.  Every
case is also held to the GEMM parity bar against the oracle on sampled outputs."""
import numpy as np
import pytest

from gpu_util import host, normalized_error, say, torch
from oracle import gemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import blockwise_scaled_fp8_quant_amd as P
    assert torch().cuda.is_available(), "GPU test run without a GPU"
    return P


def case(mode, M, N, K, seed):
    t = torch()
    g = t.Generator(device="cuda")
    g.manual_seed(seed)
    A = (t.randn((M, K), generator=g, device="cuda") * 48).clamp(-448, 448).to(t.float8_e4m3fn).view(t.uint8)
    B = (t.randn((N, K), generator=g, device="cuda") * 48).clamp(-448, 448).to(t.float8_e4m3fn).view(t.uint8)
    sA = t.exp2(t.rand((K // 128, M), generator=g, device="cuda") * 8 - 12)
    sB = t.exp2(t.rand((K // 128, N) if mode == "WGRAD" else (N // 128, K // 128), generator=g, device="cuda") * 8 - 12)
    return A, sA, B, sB


def run_pair(P, mode, M, N, K, out_dtype, seed):
    t = torch()
    ws = P.puro_fp8_gemm_workspace_size(P.MODE_NAMES[mode], M, N, K)
    say(f"[noalloc] {mode} M,N,K={M},{N},{K} out={'bf16' if out_dtype == P.OUT_BF16 else 'fp32'} "
        f"partials {ws} B (buffer {P.SCRATCH_BYTES} B)")
    assert ws <= P.SCRATCH_BYTES
    A, sA, B, sB = case(mode, M, N, K, seed)
    dt = t.bfloat16 if out_dtype == P.OUT_BF16 else t.float32
    C = t.full((M, N), float("nan"), dtype=dt, device="cuda")
    P.puro_fp8_gemm_noalloc(mode, A, sA, B, sB, C, out_dtype=out_dtype)
    ref = P.puro_fp8_gemm(mode, A, sA, B, sB, out_dtype=out_dtype)
    t.cuda.synchronize()
    same = (C.view(t.int16) == ref.view(t.int16)) if dt == t.bfloat16 else (C.view(t.int32) == ref.view(t.int32))
    assert bool(same.all()), f"{mode} {M}x{N}x{K}: allocation-free output differs from puro_fp8_gemm"
    # the GEMM bar against the oracle on sampled outputs
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, size=32, replace=False))
    cols = np.sort(rng.choice(N, size=32, replace=False))
    rt, ct = t.from_numpy(rows).cuda(), t.from_numpy(cols).cuda()
    Ad = gemm.dequant_a(host(A[rt]), host(sA[:, rt]))
    if mode == "WGRAD":
        Bd = gemm.dequant_b(mode, host(B[ct]), host(sB[:, ct]))
    else:
        from oracle import e4m3
        Bd = e4m3.decode(host(B[ct])) * np.repeat(host(sB[t.from_numpy(cols // 128).cuda()]).astype(np.float64), 128, 1)
    r = Ad @ Bd.T
    err, diff, den = normalized_error(host(C[rt][:, ct]), r, np.sqrt((Ad * Ad).sum(1)), np.sqrt((Bd * Bd).sum(1)))
    rnd = 2.0 ** -8 * np.abs(r) * (1 + 2.0 ** -7) if dt == t.bfloat16 else 0.0
    assert (diff <= 1e-3 * den + rnd).all(), err


def test_noalloc_matches_gemm_on_consecutive_calls(P):
    # split contractions (the buffer is used): a large one, then a smaller one in a row
    run_pair(P, "WGRAD", 2048, 2048, 16384, P.OUT_FP32, 1)   # 4 splits of 2048 x 2048: the whole buffer
    run_pair(P, "WGRAD", 1024, 512, 8192, P.OUT_FP32, 2)     # smaller: reads a buffer holding old partials
    run_pair(P, "FWD", 256, 512, 16384, P.OUT_BF16, 3)
    run_pair(P, "DGRAD", 128, 256, 4096, P.OUT_BF16, 4)
    # a problem without a split (the buffer is not touched)
    assert P.puro_fp8_gemm_workspace_size(P.FWD, 4096, 4096, 2048) == 0
    run_pair(P, "FWD", 4096, 4096, 2048, P.OUT_BF16, 5)


def test_noalloc_refuses_partials_larger_than_its_buffer(P):
    t = torch()
    M, N, K = 3072, 4096, 65536
    assert P.puro_fp8_gemm_workspace_size(P.WGRAD, M, N, K) > P.SCRATCH_BYTES
    lib = P.lib
    rc = lib.puro_fp8_gemm_noalloc(2, M, N, K, 16, K, 16, 16, K, 16, 16, N, 1, None)
    assert rc == -7, rc                                      # PURO_ERR_WORKSPACE, nothing launched
    t.cuda.synchronize()
