"""GPU tests of puro_fp8_quant_w_128x128_batch: several 128x128 weight quantizations in one launch.

Bar: every job's codes and scales (both orientations) byte-identical to one
puro_fp8_quant_w_128x128 call on the same weight (whose bytes are pinned against the oracle by
test_gpu_quant.py), and, for the small weight, to the oracle directly.
"""
import numpy as np
import pytest

from gpu_util import assert_bytes_equal, bf16_dev, host, say, torch
from oracle import quant
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import blockwise_scaled_fp8_quant_amd as P
    assert torch().cuda.is_available(), "GPU test run without a GPU"
    return P


def weight(N, K, seed, scale=0.02):
    t = torch()
    g = t.Generator(device="cuda")
    g.manual_seed(seed)
    return (t.randn((N, K), generator=g, device="cuda") * scale).to(t.bfloat16)


def check_batch(P, ws, transposed=True):
    res = P.puro_fp8_quant_w_128x128_batch(ws, transposed=transposed)
    for i, (w, got) in enumerate(zip(ws, res)):
        ref = P.puro_fp8_quant_w_128x128(w, transposed=transposed)
        for name, a, b in zip(("q", "s", "qT", "sT"), got, ref):
            if b is None:
                assert a is None
                continue
            assert_bytes_equal(host(a), host(b), f"job {i} ({tuple(w.shape)}) {name}")
    return res


def test_batch_sweep_weights(P):
    """The 4 weights of the layer sweep (qkv, o, gate_up, down) in one launch."""
    shapes = [(4096, 2048), (2048, 2048), (12288, 2048), (2048, 6144)]
    say(f"[quant_w batch] {shapes}")
    check_batch(P, [weight(n, k, 10 + i) for i, (n, k) in enumerate(shapes)])


def test_batch_mixed_shapes_oracle_and_no_transpose(P):
    rng = np.random.default_rng(5)
    small = f32_to_bf16_bits(rng.standard_normal((384, 512)).astype(np.float32) * np.float32(0.02))
    ws = [bf16_dev(small), weight(128, 128, 1), weight(1280, 384, 2, scale=3.0)]
    say("[quant_w batch] 384x512, 128x128, 1280x384 without transposed copies")
    res = check_batch(P, ws, transposed=False)
    rq, rs, _, _ = quant.quant_w_128x128(small)
    assert_bytes_equal(host(res[0][0]), rq, "codes vs oracle")
    assert_bytes_equal(host(res[0][1]), rs, "scales vs oracle")
    say("[quant_w batch] the same with transposed copies")
    res = check_batch(P, ws, transposed=True)
    _, _, rqT, rsT = quant.quant_w_128x128(small)
    assert_bytes_equal(host(res[0][2]), rqT, "transposed codes vs oracle")
    assert_bytes_equal(host(res[0][3]), rsT, "transposed scales vs oracle")


def test_batch_empty_strided_and_sixteen_jobs(P):
    t = torch()
    say("[quant_w batch] an empty weight, a strided weight, 16 jobs")
    wide = weight(256, 640, 3)
    strided = wide[:, :512]                                       # ldw 640 > K 512
    empty = t.empty((0, 256), dtype=t.bfloat16, device="cuda")
    ws = [strided, empty] + [weight(128 * (1 + i % 3), 256, 20 + i) for i in range(14)]
    assert len(ws) == 16
    res = P.puro_fp8_quant_w_128x128_batch(ws)
    ref = P.puro_fp8_quant_w_128x128(strided)
    for name, a, b in zip(("q", "s", "qT", "sT"), res[0], ref):
        assert_bytes_equal(host(a), host(b), f"strided {name}")
    for i in range(2, 16):
        ref = P.puro_fp8_quant_w_128x128(ws[i])
        for name, a, b in zip(("q", "s", "qT", "sT"), res[i], ref):
            assert_bytes_equal(host(a), host(b), f"job {i} {name}")
