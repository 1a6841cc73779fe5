"""Seeded synthetic inputs shared by the GPU tests, the bench and the oracle checks.

This module only *draws* tensors: it holds none of the quantization or GEMM
arithmetic.  Every tensor is drawn as float32 from NumPy's PCG64 generator
(``numpy.random.default_rng(seed)``) in a fixed order, then rounded to bfloat16
by round-to-nearest-even on the bit pattern.  The result is returned as the raw
``uint16`` bf16 bit pattern, which is exactly what the GPU receives (as
``torch.bfloat16``) and what the oracle widens on its own.

Shapes follow one GPU's share of the Puro-2B workload: 4096-token sequences
(agihunt digest "清华用消费级 5090 花 6890 美元从零训 2B…", section 方法/Method,
first paragraph) and a ~2B dense layer built on the Qwen3-1.7B shape
(hidden 2048, fused QKV 4096 rows, gate+up 12288 rows, intermediate 6144).
The hidden sizes are not printed on the pages; they are the public Qwen3-1.7B
dimensions.  Distributions (normal sigmas, Student-t with 3 degrees of freedom,
0.5% outliers scaled by 20) are the synthetic recipe of each named workload.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Tuple

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "Tensor",
    "Workload",
    "WORKLOADS",
    "draw",
    "normal_bf16",
    "student_t_bf16",
    "SWEEP_WEIGHTS",
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even) and return the uint16 bits.

    NaN inputs map to a quiet NaN with the same sign.  This is input preparation
    (how the synthetic bf16 tensors are made), not part of the quantizer.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16), rounded)
    return rounded


def normal_bf16(rng: np.random.Generator, shape: Tuple[int, int], sigma: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


def student_t_bf16(rng: np.random.Generator, shape: Tuple[int, int], scale: float, df: float = 3.0) -> np.ndarray:
    x = rng.standard_t(df, size=shape).astype(np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return f32_to_bf16_bits(x)


def normal_with_outliers_bf16(rng: np.random.Generator, shape: Tuple[int, int], sigma: float,
                              frac: float, factor: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(sigma)
    n = x.size
    k = int(round(frac * n))
    idx = rng.choice(n, size=k, replace=False)
    flat = x.reshape(-1)
    flat[idx] *= np.float32(factor)
    return f32_to_bf16_bits(x)


@dataclass(frozen=True)
class Tensor:
    """One drawn tensor: name, [rows, cols], distribution tag and its parameters."""
    name: str
    shape: Tuple[int, int]
    dist: str                 # "normal" | "t3" | "normal_outliers"
    scale: float
    extra: Tuple = ()


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload: tensors in draw order plus the GEMMs run on them.

    ``gemms`` entries are (mode, A-tensor, B-tensor, out dtype):
      FWD   Y[T,Dout]   = X[T,Din]  . W[Dout,Din]^T   A=X  (1x128), B=W (128x128)
      DGRAD dX[T,Din]   = dY[T,Dout] . W[Dout,Din]    A=dY (1x128), B=W^T (128x128 copy)
      WGRAD dW[Dout,Din]= dY^T . X                    A=dY (128x1), B=X (128x1)
    """
    name: str
    seed: int
    tensors: Tuple[Tensor, ...]
    gemms: Tuple[Tuple[str, str, str, str], ...]
    note: str = ""


def _sweep_tensors(T: int) -> Tuple[Tensor, ...]:
    out: List[Tensor] = []
    for wname, (dout, din) in SWEEP_WEIGHTS:
        out.append(Tensor(f"X_{wname}", (T, din), "t3", 1.0))
        out.append(Tensor(f"W_{wname}", (dout, din), "normal", 0.02))
        out.append(Tensor(f"dY_{wname}", (T, dout), "t3", 1e-3))
    return tuple(out)


def _sweep_gemms() -> Tuple[Tuple[str, str, str, str], ...]:
    g = []
    for wname, _ in SWEEP_WEIGHTS:
        g.append(("FWD", f"X_{wname}", f"W_{wname}", "bf16"))
        g.append(("DGRAD", f"dY_{wname}", f"W_{wname}", "bf16"))
        g.append(("WGRAD", f"dY_{wname}", f"X_{wname}", "fp32"))
    return tuple(g)


# The four linear weights of one ~2B-scale layer, [Dout, Din].
SWEEP_WEIGHTS: Tuple[Tuple[str, Tuple[int, int]], ...] = (
    ("qkv", (4096, 2048)),
    ("o", (2048, 2048)),
    ("gate_up", (12288, 2048)),
    ("down", (2048, 6144)),
)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", 0,
        (Tensor("X", (256, 512), "normal_outliers", 1.0, (0.005, 20.0)),
         Tensor("W", (384, 512), "normal", 0.02)),
        (("FWD", "X", "W", "fp32"),),
        "X ~ N(0,1) with 0.5% of entries (655, without replacement) multiplied by 20; W ~ N(0,0.02)"),
    "qkv_fwd": Workload(
        "qkv_fwd", 0,
        (Tensor("X", (4096, 2048), "normal", 1.0),
         Tensor("W", (4096, 2048), "normal", 0.02)),
        (("FWD", "X", "W", "bf16"),),
        "attention QKV projection forward, 4096 tokens"),
    "mlp_fwd": Workload(
        "mlp_fwd", 0,
        (Tensor("X", (8192, 2048), "normal", 1.0),
         Tensor("W_gu", (12288, 2048), "normal", 0.02),
         Tensor("H", (8192, 6144), "normal", 0.5),
         Tensor("W_d", (2048, 6144), "normal", 0.02)),
        (("FWD", "X", "W_gu", "bf16"), ("FWD", "H", "W_d", "bf16")),
        "MLP forward, 8192 tokens: gate+up then down projection"),
    "down_bwd": Workload(
        "down_bwd", 0,
        (Tensor("dY", (8192, 2048), "normal", 1e-3),
         Tensor("W_d", (2048, 6144), "normal", 0.02),
         Tensor("H", (8192, 6144), "normal", 0.5)),
        (("DGRAD", "dY", "W_d", "bf16"), ("WGRAD", "dY", "H", "fp32")),
        "MLP down-projection backward, 8192 tokens"),
}
for _s in range(4):
    WORKLOADS[f"layer_sweep_s{_s}"] = Workload(
        f"layer_sweep_s{_s}", _s, _sweep_tensors(16384), _sweep_gemms(),
        "all four linear weights of one layer at 16384 tokens, fwd+dgrad+wgrad; "
        "activations Student-t(3), dY = 1e-3 * Student-t(3)")


def _draw_one(rng: np.random.Generator, t: Tensor, shape: Tuple[int, int]) -> np.ndarray:
    if t.dist == "normal":
        return normal_bf16(rng, shape, t.scale)
    if t.dist == "t3":
        return student_t_bf16(rng, shape, t.scale)
    if t.dist == "normal_outliers":
        frac, factor = t.extra
        return normal_with_outliers_bf16(rng, shape, t.scale, frac, factor)
    raise ValueError(f"unknown distribution {t.dist}")


def draw(workload: str | Workload) -> Dict[str, np.ndarray]:
    """Draw every tensor of a workload in its fixed order; returns name -> uint16 bf16 bits."""
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    rng = np.random.default_rng(wl.seed)
    out: Dict[str, np.ndarray] = {}
    for t in wl.tensors:
        out[t.name] = _draw_one(rng, t, t.shape)
    return out
