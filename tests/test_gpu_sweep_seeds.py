"""GPU parity on the full-layer sweep's own seeded inputs (16384 tokens, seeds 0..3), through
exactly the calls the benchmark step makes.

For each seed the workload is drawn by ``workloads.draw("layer_sweep_s{seed}")`` (the tensors the
bench times for seed 0), and for each of the four weights (qkv 4096x2048, o 2048x2048, gate_up
12288x2048, down 2048x6144) the step's calls run in the step's order and launch configuration:
W 128x128 with its transposed copy; the dual quantizer on X; FWD (bf16); the dual quantizer on
dY; DGRAD (bf16); WGRAD (fp32).

Bars:
  - quantizers byte-identical to the oracle: two sampled 128-row blocks of W (q, s, qT, sT), and
    two sampled 128-token blocks of X and of dY (all four dual outputs);
  - GEMMs on sampled rows x columns, against the oracle's float64 product of the GPU's quantized
    operands: |C - C_ref| <= 1e-3 (||A^_i|| ||B^_j||), and the tight 1e-4 bound (plus one bf16
    rounding of C_ref for bf16 outputs).
Token counts: four of the pages' 4096-token sequences (agihunt digest, section 方法, training
layout).
"""
import numpy as np
import pytest

from gpu_util import assert_bytes_equal, bf16_dev, host, normalized_error, say, torch
from oracle import e4m3, gemm, quant
from workloads import SWEEP_WEIGHTS, draw

pytestmark = pytest.mark.gpu
TOL, TIGHT = 1e-3, 1e-4


@pytest.fixture(scope="module")
def P():
    import blockwise_scaled_fp8_quant_amd as P
    assert torch().cuda.is_available(), "GPU test run without a GPU"
    return P


def check_gemm(P, mode, A, sA, B, sB, C, seed, bf16):
    t = torch()
    M, N = C.shape
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, size=64, replace=False))
    cols = np.sort(rng.choice(N, size=64, replace=False))
    rt, ct = t.from_numpy(rows).cuda(), t.from_numpy(cols).cuda()
    Ad = gemm.dequant_a(host(A[rt]), host(sA[:, rt]))
    if mode == "WGRAD":
        Bd = gemm.dequant_b(mode, host(B[ct]), host(sB[:, ct]))
    else:
        # each sampled column j takes the scales of its 128-row weight block, sB[j / 128][kb]
        sBb = host(sB[t.from_numpy(cols // 128).cuda()])    # [cols][K/128]
        Bd = e4m3.decode(host(B[ct])) * np.repeat(sBb.astype(np.float64), 128, axis=1)
    ref = Ad @ Bd.T
    na, nb = np.sqrt((Ad * Ad).sum(1)), np.sqrt((Bd * Bd).sum(1))
    err, diff, den = normalized_error(host(C[rt][:, ct]), ref, na, nb)
    rnd = 2.0 ** -8 * np.abs(ref) * (1 + 2.0 ** -7) if bf16 else 0.0
    say(f"    {mode}: max normalized error {err:.3e}")
    assert (diff <= TOL * den + rnd).all()
    assert (diff <= TIGHT * den + rnd).all()


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_layer_sweep_seed(P, seed):
    t = torch()
    say(f"[sweep seed {seed}] drawing layer_sweep_s{seed} (16384 tokens)")
    d = draw(f"layer_sweep_s{seed}")
    rng = np.random.default_rng(1000 + seed)
    for wname, (dout, din) in SWEEP_WEIGHTS:
        say(f"[sweep seed {seed}] {wname} W {dout}x{din}, X 16384x{din}, dY 16384x{dout}")
        X, W, dY = bf16_dev(d[f"X_{wname}"]), bf16_dev(d[f"W_{wname}"]), bf16_dev(d[f"dY_{wname}"])
        T = X.shape[0]
        Wq, Ws, WqT, WsT = P.puro_fp8_quant_w_128x128(W)
        Xq, Xs, XqT, XsT = P.puro_fp8_quant_act_dual(X)
        Y = P.puro_fp8_gemm(P.FWD, Xq, Xs, Wq, Ws, out_dtype=P.OUT_BF16)
        Gq, Gs, GqT, GsT = P.puro_fp8_quant_act_dual(dY)
        dX = P.puro_fp8_gemm(P.DGRAD, Gq, Gs, WqT, WsT, out_dtype=P.OUT_BF16)
        dW = P.puro_fp8_gemm(P.WGRAD, GqT, GsT, XqT, XsT, out_dtype=P.OUT_FP32)
        t.cuda.synchronize()

        for rb in sorted(rng.choice(dout // 128, size=2, replace=False).tolist()):
            rows = slice(128 * rb, 128 * rb + 128)
            rq, rs, rqT, rsT = quant.quant_w_128x128(d[f"W_{wname}"][rows])
            assert_bytes_equal(host(Wq[rows]), rq, f"W codes, block row {rb}")
            assert_bytes_equal(host(Ws[rb:rb + 1]), rs, f"W scales, block row {rb}")
            assert_bytes_equal(host(WqT[:, rows]), rqT, f"W^T codes, block row {rb}")
            assert_bytes_equal(host(WsT[:, rb:rb + 1]), rsT, f"W^T scales, block row {rb}")
        for name, bits, (q, s, qT, sT) in (("X", d[f"X_{wname}"], (Xq, Xs, XqT, XsT)),
                                           ("dY", d[f"dY_{wname}"], (Gq, Gs, GqT, GsT))):
            for tb in sorted(rng.choice(T // 128, size=2, replace=False).tolist()):
                rows = slice(128 * tb, 128 * tb + 128)
                rq, rs = quant.quant_act_1x128(bits[rows])
                rqT, rsT = quant.quant_act_128x1(bits[rows])
                assert_bytes_equal(host(q[rows]), rq, f"{name} 1x128 codes, token block {tb}")
                assert_bytes_equal(host(s[:, rows]), rs, f"{name} 1x128 scales, token block {tb}")
                assert_bytes_equal(host(qT[:, rows]), rqT, f"{name} 128x1 codes, token block {tb}")
                assert_bytes_equal(host(sT[tb:tb + 1]), rsT, f"{name} 128x1 scales, token block {tb}")

        base = 100 * seed + 10 * [w for w, _ in SWEEP_WEIGHTS].index(wname)
        check_gemm(P, "FWD", Xq, Xs, Wq, Ws, Y, base + 1, True)
        check_gemm(P, "DGRAD", Gq, Gs, WqT, WsT, dX, base + 2, True)
        check_gemm(P, "WGRAD", GqT, GsT, XqT, XsT, dW, base + 3, False)
        del X, W, dY, Wq, Ws, WqT, WsT, Xq, Xs, XqT, XsT, Y, Gq, Gs, GqT, GsT, dX, dW
    del d
