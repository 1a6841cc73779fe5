"""Python binding of libpuro_fp8 (blockwise-scaled FP8 linear layer for MI355X / gfx950).

Argument marshalling only: every function takes torch tensors that already live on the
GPU, passes their device pointers, sizes and the current HIP stream to the C ABI
(``include/puro_fp8.h``), allocates missing outputs with torch (device memory is all
torch is used for), and raises ``PuroError`` on a non-zero status.  Before any pointer is
passed on, every tensor is checked for what the C ABI cannot see: that it lives on the
current GPU, has the element type and shape the entry point expects, and has rows of unit
element stride (scale arrays, which the ABI takes without a leading dimension, must be
contiguous); a mismatch raises TypeError or ValueError and launches nothing.  Every step of the
computation runs in the library's HIP kernels; there is no fallback of any kind, and
importing this package fails loudly when the shared library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "LIB_PATH", "lib", "PuroError", "FWD", "DGRAD", "WGRAD", "OUT_BF16", "OUT_FP32",
    "puro_fp8_quant_act_1x128", "puro_fp8_quant_act_128x1", "puro_fp8_quant_act_dual",
    "puro_fp8_quant_w_128x128", "puro_fp8_gemm", "puro_fp8_gemm_accumulate", "puro_fp8_gemm_workspace_size",
    "puro_fp8_cast_e4m3", "puro_fp8_strerror", "puro_fp8_version", "EXPORTED_SYMBOLS",
    "puro_fp8_mx_quant_dual", "puro_fp8_mx_gemm", "puro_fp8_mx_gemm_workspace_size", "puro_fp8_gemm_quant",
    "puro_fp8_quant_w_128x128_batch", "puro_fp8_gemm_noalloc", "SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpuro_fp8.so")

FWD, DGRAD, WGRAD = 0, 1, 2
SCRATCH_BYTES = 64 * 1024 * 1024   # PURO_FP8_SCRATCH_BYTES: the allocation-free GEMM's own buffer
OUT_BF16, OUT_FP32 = 0, 1
MODE_NAMES = {"FWD": FWD, "DGRAD": DGRAD, "WGRAD": WGRAD}

EXPORTED_SYMBOLS = (
    "puro_fp8_quant_act_1x128", "puro_fp8_quant_act_128x1", "puro_fp8_quant_act_dual", "puro_fp8_quant_w_128x128",
    "puro_fp8_gemm", "puro_fp8_gemm_accumulate", "puro_fp8_gemm_workspace_size", "puro_fp8_cast_e4m3",
    "puro_fp8_strerror", "puro_fp8_version",
    "puro_fp8_mx_quant_dual", "puro_fp8_mx_gemm", "puro_fp8_mx_gemm_workspace_size", "puro_fp8_gemm_quant",
    "puro_fp8_quant_w_128x128_batch", "puro_fp8_gemm_noalloc",
)

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python blockwise_scaled_fp8_quant_amd/build.py "
        f"or __graft_entry__.build()); there is no non-HIP implementation")

# torch ships its own HIP runtime (same SONAME, libamdhip64.so.7).  It must be loaded
# before the library so that the library's NEEDED entry binds to it: device pointers and
# streams from torch are only valid in torch's runtime instance.
import torch as _torch_runtime  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
        return {os.path.realpath(p) for p in paths}
    except OSError:
        return set()


if len(_hip_runtimes_mapped()) > 1:
    raise ImportError(f"two HIP runtimes are mapped in this process ({sorted(_hip_runtimes_mapped())}); "
                      "import torch before any other HIP library")

_i64, _p, _int, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
lib.puro_fp8_quant_act_1x128.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _p]
lib.puro_fp8_quant_act_128x1.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _p]
lib.puro_fp8_quant_act_dual.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p]
lib.puro_fp8_quant_w_128x128.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p]


class WqJob(ctypes.Structure):
    """puro_fp8_wq_job (include/puro_fp8.h): the arguments of one 128x128 weight quantization."""
    _fields_ = [("w", _p), ("N", _i64), ("K", _i64), ("ldw", _i64), ("q", _p), ("ldq", _i64), ("s", _p),
                ("qT", _p), ("ldqT", _i64), ("sT", _p)]


lib.puro_fp8_quant_w_128x128_batch.argtypes = [ctypes.POINTER(WqJob), _int, _p]
lib.puro_fp8_gemm.argtypes = [_int, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p, _i64, _int, _p, _sz, _p]
lib.puro_fp8_gemm_accumulate.argtypes = [_int, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p, _i64, _p, _sz, _p]
lib.puro_fp8_gemm_noalloc.argtypes = [_int, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p, _i64, _int, _p]
lib.puro_fp8_gemm_quant.argtypes = [_int, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p, _i64, _p, _i64, _p, _p, _sz, _p]
lib.puro_fp8_mx_quant_dual.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p]
lib.puro_fp8_mx_gemm.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p, _i64, _int, _p, _sz, _p]
lib.puro_fp8_mx_gemm_workspace_size.argtypes = [_i64, _i64, _i64]
lib.puro_fp8_mx_gemm_workspace_size.restype = _sz
lib.puro_fp8_gemm_workspace_size.argtypes = [_int, _i64, _i64, _i64]
lib.puro_fp8_gemm_workspace_size.restype = _sz
lib.puro_fp8_cast_e4m3.argtypes = [_p, _i64, _p, _p]
lib.puro_fp8_strerror.argtypes = [_int]
lib.puro_fp8_strerror.restype = ctypes.c_char_p
lib.puro_fp8_version.argtypes = []
for _f in ("puro_fp8_quant_act_1x128", "puro_fp8_quant_act_128x1", "puro_fp8_quant_act_dual",
           "puro_fp8_quant_w_128x128", "puro_fp8_quant_w_128x128_batch", "puro_fp8_gemm",
           "puro_fp8_gemm_accumulate", "puro_fp8_gemm_quant", "puro_fp8_gemm_noalloc", "puro_fp8_mx_quant_dual",
           "puro_fp8_mx_gemm",
           "puro_fp8_cast_e4m3", "puro_fp8_version"):
    getattr(lib, _f).restype = _int


class PuroError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.puro_fp8_strerror(status).decode()} (status {status})")


def puro_fp8_strerror(status: int) -> str:
    return lib.puro_fp8_strerror(status).decode()


def puro_fp8_version() -> int:
    return lib.puro_fp8_version()


def _torch():
    import torch
    return torch


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    return _torch().cuda.current_stream().cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(status: int, where: str):
    if status != 0:
        raise PuroError(status, where)


def _ld(t) -> int:
    return t.stride(0) if t.dim() == 2 else t.shape[-1]


def _need(t, what: str, dtype, shape, whole: bool = False):
    """Check tensor argument `what` before its pointer goes to the library (the C ABI sees only
    the pointer): a torch tensor on the current GPU, of `dtype` and `shape`, whose rows have
    unit element stride -- or, with `whole`, fully contiguous (scale arrays and buffers the ABI
    takes without a leading dimension)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: must be a GPU tensor, not on {t.device}")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{what}: must live on the current GPU (cuda:{torch.cuda.current_device()}), "
                         f"not on {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.numel() > 1:
        if whole and not t.is_contiguous():
            raise ValueError(f"{what}: must be contiguous")
        if t.stride(-1) != 1:
            raise ValueError(f"{what}: rows must have unit element stride (got strides {t.stride()})")
    return t


def _2d(t, what: str):
    """The (rows, columns) of a 2-D tensor argument."""
    if getattr(t, "dim", None) is None or t.dim() != 2:
        raise ValueError(f"{what}: expected a 2-D tensor")
    return t.shape


def puro_fp8_quant_act_1x128(x, q=None, s=None, stream=None) -> Tuple[object, object]:
    """x bf16 [M, K] -> (q uint8 [M, K], s fp32 [K/128, M])."""
    torch = _torch()
    M, K = _2d(x, "x")
    _need(x, "x", torch.bfloat16, (M, K))
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    _need(q, "q", torch.uint8, (M, K))
    _need(s, "s", torch.float32, (K // 128, M), whole=True)
    _check(lib.puro_fp8_quant_act_1x128(_ptr(x), M, K, _ld(x), _ptr(q), _ld(q), _ptr(s), _stream(stream)),
           "puro_fp8_quant_act_1x128")
    return q, s


def puro_fp8_quant_act_128x1(x, qT=None, sT=None, stream=None) -> Tuple[object, object]:
    """x bf16 [T, C] -> (qT uint8 [C, T], sT fp32 [T/128, C])."""
    torch = _torch()
    T, C = _2d(x, "x")
    _need(x, "x", torch.bfloat16, (T, C))
    if qT is None:
        qT = torch.empty((C, T), dtype=torch.uint8, device=x.device)
    if sT is None:
        sT = torch.empty((T // 128, C), dtype=torch.float32, device=x.device)
    _need(qT, "qT", torch.uint8, (C, T))
    _need(sT, "sT", torch.float32, (T // 128, C), whole=True)
    _check(lib.puro_fp8_quant_act_128x1(_ptr(x), T, C, _ld(x), _ptr(qT), _ld(qT), _ptr(sT), _stream(stream)),
           "puro_fp8_quant_act_128x1")
    return qT, sT


def puro_fp8_quant_act_dual(x, q=None, s=None, qT=None, sT=None, stream=None):
    """x bf16 [T, C] -> (q [T, C], s [C/128, T], qT [C, T], sT [T/128, C]): the outputs of
    puro_fp8_quant_act_1x128 and puro_fp8_quant_act_128x1 from one read of x."""
    torch = _torch()
    T, C = _2d(x, "x")
    _need(x, "x", torch.bfloat16, (T, C))
    if q is None:
        q = torch.empty((T, C), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((C // 128, T), dtype=torch.float32, device=x.device)
    if qT is None:
        qT = torch.empty((C, T), dtype=torch.uint8, device=x.device)
    if sT is None:
        sT = torch.empty((T // 128, C), dtype=torch.float32, device=x.device)
    _need(q, "q", torch.uint8, (T, C))
    _need(s, "s", torch.float32, (C // 128, T), whole=True)
    _need(qT, "qT", torch.uint8, (C, T))
    _need(sT, "sT", torch.float32, (T // 128, C), whole=True)
    _check(lib.puro_fp8_quant_act_dual(_ptr(x), T, C, _ld(x), _ptr(q), _ld(q), _ptr(s), _ptr(qT), _ld(qT),
                                       _ptr(sT), _stream(stream)), "puro_fp8_quant_act_dual")
    return q, s, qT, sT


def _weight_outs(w, q, s, qT, sT, transposed: bool, what: str):
    """Allocate the missing outputs of one 128x128 weight quantization and check all of them."""
    torch = _torch()
    N, K = _2d(w, what)
    _need(w, what, torch.bfloat16, (N, K))
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    if transposed:
        if qT is None:
            qT = torch.empty((K, N), dtype=torch.uint8, device=w.device)
        if sT is None:
            sT = torch.empty((K // 128, N // 128), dtype=torch.float32, device=w.device)
    _need(q, f"{what} codes", torch.uint8, (N, K))
    _need(s, f"{what} scales", torch.float32, (N // 128, K // 128), whole=True)
    if qT is not None:
        _need(qT, f"{what} transposed codes", torch.uint8, (K, N))
    if sT is not None:
        _need(sT, f"{what} transposed scales", torch.float32, (K // 128, N // 128), whole=True)
    return N, K, q, s, qT, sT


def puro_fp8_quant_w_128x128(w, q=None, s=None, qT=None, sT=None, transposed: bool = True, stream=None):
    """w bf16 [N, K] -> (q [N, K], s [N/128, K/128], qT [K, N] or None, sT [K/128, N/128] or None)."""
    N, K, q, s, qT, sT = _weight_outs(w, q, s, qT, sT, transposed, "w")
    ldqT = _ld(qT) if qT is not None else 0
    _check(lib.puro_fp8_quant_w_128x128(_ptr(w), N, K, _ld(w), _ptr(q), _ld(q), _ptr(s), _ptr(qT), ldqT,
                                        _ptr(sT), _stream(stream)), "puro_fp8_quant_w_128x128")
    return q, s, qT, sT


def puro_fp8_quant_w_128x128_batch(weights, outs=None, transposed: bool = True, stream=None):
    """Several weights in one launch: weights = [w bf16 [N, K], ...]; outs (optional) = [(q, s, qT, sT),
    ...] as puro_fp8_quant_w_128x128 takes them.  Returns [(q, s, qT, sT), ...], the same bytes as one
    puro_fp8_quant_w_128x128 call per weight."""
    res = []
    jobs = (WqJob * max(len(weights), 1))()
    for i, w in enumerate(weights):
        q, s, qT, sT = outs[i] if outs is not None else (None, None, None, None)
        N, K, q, s, qT, sT = _weight_outs(w, q, s, qT, sT, transposed, f"weights[{i}]")
        jobs[i] = WqJob(_ptr(w), N, K, _ld(w), _ptr(q), _ld(q), _ptr(s), _ptr(qT),
                        _ld(qT) if qT is not None else 0, _ptr(sT))
        res.append((q, s, qT, sT))
    _check(lib.puro_fp8_quant_w_128x128_batch(jobs, len(weights), _stream(stream)), "puro_fp8_quant_w_128x128_batch")
    return res


def puro_fp8_gemm_workspace_size(mode: int, M: int, N: int, K: int) -> int:
    return lib.puro_fp8_gemm_workspace_size(mode, M, N, K)


def _gemm_args(mode, A, sA, B, sB, C, c_dtype, workspace, need_fn):
    """Shapes, checks and the workspace of one GEMM call (blockwise when mode is given, else MX)."""
    torch = _torch()
    M, K = _2d(A, "A")
    N, KB = _2d(B, "B")
    if KB != K:
        raise ValueError(f"A [{M}, {K}] and B [{N}, {KB}] differ in the contraction length")
    _need(A, "A", torch.uint8, (M, K))
    _need(B, "B", torch.uint8, (N, K))
    if K == 0 and sA is None and sB is None:
        pass                                         # empty contraction: no scales, as the C ABI allows
    elif mode is None:                               # MX: E8M0 bytes [K/128, rows, 4]
        _need(sA, "xa", torch.uint8, (K // 128, M, 4), whole=True)
        _need(sB, "xb", torch.uint8, (K // 128, N, 4), whole=True)
    else:
        _need(sA, "sA", torch.float32, (K // 128, M), whole=True)
        _need(sB, "sB", torch.float32, (K // 128, N) if mode == WGRAD else (N // 128, K // 128), whole=True)
    if C is None:
        C = torch.empty((M, N), dtype=c_dtype, device=A.device)
    _need(C, "C", c_dtype, (M, N))
    need = need_fn(M, N, K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
    if workspace is not None:
        _need(workspace, "workspace", workspace.dtype, None, whole=True)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return M, N, K, C, workspace, wbytes


def _mode(mode) -> int:
    return MODE_NAMES[mode] if isinstance(mode, str) else mode


def _out_dtype(out_dtype):
    torch = _torch()
    if out_dtype not in (OUT_BF16, OUT_FP32):
        raise ValueError(f"out_dtype {out_dtype}: expected OUT_BF16 or OUT_FP32")
    return torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32


def puro_fp8_gemm(mode, A, sA, B, sB, C=None, out_dtype: int = OUT_BF16, workspace=None, stream=None):
    """C [M, N] = blockwise-scaled FP8 product of A [M, K] and B [N, K] (see puro_fp8.h)."""
    mode = _mode(mode)
    M, N, K, C, workspace, wbytes = _gemm_args(mode, A, sA, B, sB, C, _out_dtype(out_dtype), workspace,
                                               lambda m, n, k: lib.puro_fp8_gemm_workspace_size(mode, m, n, k))
    _check(lib.puro_fp8_gemm(mode, M, N, K, _ptr(A), _ld(A), _ptr(sA), _ptr(B), _ld(B), _ptr(sB), _ptr(C), _ld(C),
                             out_dtype, _ptr(workspace), wbytes, _stream(stream)), "puro_fp8_gemm")
    return C


def puro_fp8_gemm_noalloc(mode, A, sA, B, sB, C, out_dtype: int = OUT_BF16, stream=None):
    """puro_fp8_gemm into the caller's C without a workspace: a contraction split keeps its partial
    sums in the library's own device buffer (SCRATCH_BYTES per device, shared by every call on the
    device).  Neither this function nor the library allocates anything."""
    mode = _mode(mode)
    if C is None:
        raise ValueError("C: the allocation-free GEMM writes into a tensor the caller provides")
    M, N, K, C, _, _ = _gemm_args(mode, A, sA, B, sB, C, _out_dtype(out_dtype), None, lambda m, n, k: 0)
    _check(lib.puro_fp8_gemm_noalloc(mode, M, N, K, _ptr(A), _ld(A), _ptr(sA), _ptr(B), _ld(B), _ptr(sB), _ptr(C),
                                     _ld(C), out_dtype, _stream(stream)), "puro_fp8_gemm_noalloc")
    return C


def puro_fp8_gemm_quant(mode, A, sA, B, sB, C=None, q=None, s=None, workspace=None, stream=None):
    """(C bf16 [M, N], q uint8 [M, N], s fp32 [N/128, M]): the GEMM and the 1x128 quantization of
    its bf16 output along N, in one launch (two when the contraction is split)."""
    torch = _torch()
    mode = _mode(mode)
    M, N, K, C, workspace, wbytes = _gemm_args(mode, A, sA, B, sB, C, torch.bfloat16, workspace,
                                               lambda m, n, k: lib.puro_fp8_gemm_workspace_size(mode, m, n, k))
    if q is None:
        q = torch.empty((M, N), dtype=torch.uint8, device=A.device)
    if s is None:
        s = torch.empty((N // 128, M), dtype=torch.float32, device=A.device)
    _need(q, "q", torch.uint8, (M, N))
    _need(s, "s", torch.float32, (N // 128, M), whole=True)
    _check(lib.puro_fp8_gemm_quant(mode, M, N, K, _ptr(A), _ld(A), _ptr(sA), _ptr(B), _ld(B), _ptr(sB), _ptr(C),
                                   _ld(C), _ptr(q), _ld(q), _ptr(s), _ptr(workspace), wbytes, _stream(stream)),
           "puro_fp8_gemm_quant")
    return C, q, s


def puro_fp8_gemm_accumulate(mode, A, sA, B, sB, C, workspace=None, stream=None):
    """C [M, N] fp32 += blockwise-scaled FP8 product of A [M, K] and B [N, K] (see puro_fp8.h)."""
    torch = _torch()
    mode = _mode(mode)
    if C is None:
        raise ValueError("C: the accumulating GEMM needs the fp32 tensor it adds into")
    M, N, K, C, workspace, wbytes = _gemm_args(mode, A, sA, B, sB, C, torch.float32, workspace,
                                               lambda m, n, k: lib.puro_fp8_gemm_workspace_size(mode, m, n, k))
    _check(lib.puro_fp8_gemm_accumulate(mode, M, N, K, _ptr(A), _ld(A), _ptr(sA), _ptr(B), _ld(B), _ptr(sB), _ptr(C),
                                        _ld(C), _ptr(workspace), wbytes, _stream(stream)), "puro_fp8_gemm_accumulate")
    return C


def puro_fp8_mx_quant_dual(x, q=None, xs=None, qT=None, xsT=None, stream=None):
    """x bf16 [T, C] -> (q [T, C], xs uint8 [C/128, T, 4], qT [C, T], xsT uint8 [T/128, C, 4]): MXFP8
    codes and E8M0 block scales along C and, transposed, along T."""
    torch = _torch()
    T, C = _2d(x, "x")
    _need(x, "x", torch.bfloat16, (T, C))
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=x.device)
    q = u8(T, C) if q is None else q
    xs = u8(C // 128, T, 4) if xs is None else xs
    qT = u8(C, T) if qT is None else qT
    xsT = u8(T // 128, C, 4) if xsT is None else xsT
    _need(q, "q", torch.uint8, (T, C))
    _need(xs, "xs", torch.uint8, (C // 128, T, 4), whole=True)
    _need(qT, "qT", torch.uint8, (C, T))
    _need(xsT, "xsT", torch.uint8, (T // 128, C, 4), whole=True)
    _check(lib.puro_fp8_mx_quant_dual(_ptr(x), T, C, _ld(x), _ptr(q), _ld(q), _ptr(xs), _ptr(qT), _ld(qT),
                                      _ptr(xsT), _stream(stream)), "puro_fp8_mx_quant_dual")
    return q, xs, qT, xsT


def puro_fp8_mx_gemm(A, xa, B, xb, C=None, out_dtype: int = OUT_BF16, workspace=None, stream=None):
    """C [M, N] = MXFP8 product of A [M, K] (scales xa [K/128, M, 4]) and B [N, K] (xb [K/128, N, 4])."""
    M, N, K, C, workspace, wbytes = _gemm_args(None, A, xa, B, xb, C, _out_dtype(out_dtype), workspace,
                                               lambda m, n, k: lib.puro_fp8_mx_gemm_workspace_size(m, n, k))
    _check(lib.puro_fp8_mx_gemm(M, N, K, _ptr(A), _ld(A), _ptr(xa), _ptr(B), _ld(B), _ptr(xb), _ptr(C), _ld(C),
                                out_dtype, _ptr(workspace), wbytes, _stream(stream)), "puro_fp8_mx_gemm")
    return C


def puro_fp8_mx_gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib.puro_fp8_mx_gemm_workspace_size(M, N, K))


def puro_fp8_cast_e4m3(v, q=None, stream=None):
    """v fp32 (any shape, contiguous) -> q uint8 codes of the same shape."""
    torch = _torch()
    _need(v, "v", torch.float32, None, whole=True)
    if q is None:
        q = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _need(q, "q", torch.uint8, tuple(v.shape), whole=True)
    _check(lib.puro_fp8_cast_e4m3(_ptr(v), v.numel(), _ptr(q), _stream(stream)), "puro_fp8_cast_e4m3")
    return q
