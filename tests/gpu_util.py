"""Helpers shared by the GPU parity tests: host <-> device marshalling and error metrics.

Expected values always come from the oracle (``oracle/``) run on the same seeded
inputs; nothing here computes a quantization or a GEMM.
"""
import sys

import numpy as np

DEV = "cuda:0"


def torch():
    import torch as _t
    return _t


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(t.bfloat16)


def u8_dev(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def f32_dev(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t) -> np.ndarray:
    tt = torch()
    torch().cuda.synchronize()
    if t.dtype == tt.bfloat16:
        return (t.contiguous().view(tt.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return t.contiguous().cpu().numpy()


def assert_bytes_equal(gpu: np.ndarray, ref: np.ndarray, what: str):
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if gpu.dtype == np.float32:
        g, r = gpu.view(np.uint32), ref.view(np.uint32)
    else:
        g, r = gpu, ref
    bad = np.argwhere(g != r)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: gpu {g[tuple(bad[0])]!r} ref {r[tuple(bad[0])]!r}"


def normalized_error(c_gpu: np.ndarray, c_ref: np.ndarray, na: np.ndarray, nb: np.ndarray):
    """max |C_gpu - C_ref| / (||A^_i|| ||B^_j||) over all entries; where a norm is 0, C must be 0."""
    den = np.outer(na, nb)
    diff = np.abs(c_gpu.astype(np.float64) - c_ref)
    zero = den == 0
    assert (c_gpu[zero] == 0).all(), "nonzero output where an operand row is zero"
    den = np.where(zero, 1.0, den)
    return float((diff / den).max()), diff, den
