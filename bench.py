"""Benchmark of the blockwise-scaled FP8 linear-layer hot path on one MI355X.

One step = one pass of the whole path over the full-layer workload at 16384 tokens
(4 sequences of 4096), seed 0, on the 4 linear weights of one ~2B-scale layer
(qkv 4096x2048, o 2048x2048, gate+up 12288x2048, down 2048x6144):
    quantize all 4 W 128x128 (+ transposed copies) in one launch;
  then for each weight:
    quantize X  1x128 and 128x1 in one pass (dual quantizer);  FWD   Y  = X  W^T  (bf16 out)
    quantize dY 1x128 and 128x1 in one pass (dual quantizer);  DGRAD dX = dY W    (bf16 out)
                                                                WGRAD dW = dY^T X  (fp32 out)
Inputs are seeded synthetic bf16 tensors already resident in HBM when timing starts.
Prints ONE JSON line.  `value` = GEMM TFLOP/s of the whole step (all 12 GEMMs' flops
divided by the step time, quantizers included in the time), timed with HIP events around the
K steps only.  The per-kernel durations (`kernels`, `roofline`) come from K more steps right
after, with an event pair around every launch (these add idle time between kernels, so that
pass's step time, `ms_per_step_instrumented`, is longer).  After the timed steps the
standalone 1x128 and 128x1 quantizers and the FWD GEMM with its output's 1x128 quantization
fused into the epilogue are timed on the same tensors (reported under `kernels` with
"in_step": false; not part of `value`), and so is the MXFP8 variant of the
whole step (`mx_variant`: blocks of 32 with E8M0 scales; W, X and dY through the MX dual
quantizer, then the three GEMMs).  `configs` times the other named configurations (the tiny
outlier case, the QKV projection FWD at 4096 tokens, the MLP FWD and the down-projection
backward at 8192 tokens) op by op on their own seeded inputs, each launch reading from HBM.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

HBM traffic of each kernel comes from two rocprofv3 counter runs of this script (FETCH_SIZE,
then WRITE_SIZE), both scaled by what the same counter reads for a plain copy of known size
that every run performs once, untimed, before the steps:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_fetch -o pmc -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-configs
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_write -o pmc -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-configs
    python bench.py --summarize-pmc OUT/pmc_fetch OUT/pmc_write   # writes TRAFFIC_FILE

The summary records a hash of the kernel sources; once they change, `traffic` reads null
until the counters are taken again.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
WORKLOAD = "layer_sweep_s0"
METRIC = "FP8 blockwise GEMM TFLOP/s fwd/dgrad/wgrad (% FP8 MFMA peak); quant GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_layer_sweep_16384.txt")
CSRC = os.path.join(ROOT, "blockwise_scaled_fp8_quant_amd", "csrc")
COPY_BYTES = 256 << 20          # calibration copy: 256 MiB read + 256 MiB written


def kernel_source_hash() -> str:
    """Hash of the code of the kernels and their launch plans (the HIP sources and the headers and
    generated sequences they include; the host-only C ABI layer is left out): comments and blank
    space are ignored, so that an edit of a comment keeps the traffic counters taken on the same
    code."""
    import re
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp", ".inc")):
            with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
                text = fh.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(f.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def op_of_kernel(name: str):
    """Map a dispatched kernel's name to the bench op it belongs to (None: not a path kernel)."""
    if "mx_quant_dual" in name:
        return "mx_quant_dual"
    if "gemm_kernel<3" in name or "gemm_w4mx_kernel" in name:
        return "mx_gemm"
    if "gemm_kernel<0, true, true>" in name or "gemm_w4_kernel<true, true>" in name:
        return "gemm_fwd_quant_out"
    if "gemm_kernel<0" in name:
        return "gemm_fwd"
    if "gemm_kernel<1" in name:
        return "gemm_dgrad"
    if "gemm_kernel<2" in name:
        return "gemm_wgrad"
    if "quant_dual" in name:
        return "quant_act_dual"
    if "quant_1x128" in name:
        return "quant_act_1x128"
    if "quant_128x128" in name:
        return "quant_w_128x128"
    if "quant_128x1" in name:
        return "quant_act_128x1"
    if "neg" in name:
        return "copy"
    return None


def read_counter_csv(d: str, counter: str):
    """Per-dispatch (kernel name, value in KiB) from one rocprofv3 --pmc csv run, in dispatch order."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = int(r["Dispatch_Id"])
                name, v = per.get(key, (r["Kernel_Name"], 0.0))
                per[key] = (name, v + float(r["Counter_Value"]))
    return [per[k] for k in sorted(per)]


def summarize_pmc(fetch_dir: str, write_dir: str):
    """Turn the two counter runs into per-op HBM bytes per launch; writes TRAFFIC_FILE."""
    res = {}
    factors = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = read_counter_csv(d, counter)
        copies = [v for n, v in rows if op_of_kernel(n) == "copy"]
        if not copies:
            raise SystemExit(f"{counter}: the calibration copy was not found")
        factors[counter] = (COPY_BYTES, copies[0] * 1024.0)
        scale = COPY_BYTES / (copies[0] * 1024.0)
        # One op can be several dispatches: a split GEMM's reduce kernel runs right after the GEMM
        # kernel, and a GEMM whose leading rows run unsplit is two launches of the same GEMM kernel
        # in a row (no GEMM op of the bench follows another of the same kernel).  FWD and DGRAD both
        # run the four-wave kernel and alternate in the step (X's FWD, then dY's DGRAD, per weight);
        # its fused-quantization instance is the standalone FWD with the output quantized.
        last, prev, w4_ops = None, None, 0
        for n, v in rows:
            gemm = "gemm_kernel" in n or "gemm_w4_kernel" in n or "gemm_w4mx_kernel" in n
            cont = "split_reduce" in n or (gemm and n == prev)
            if "split_reduce" in n or cont:
                op = last
            elif "gemm_w4_kernel" in n and op_of_kernel(n) is None:
                op = "gemm_fwd" if w4_ops % 2 == 0 else "gemm_dgrad"
                w4_ops += 1
            else:
                op = op_of_kernel(n)
            prev = n
            if op is None or op == "copy":
                continue
            if gemm:
                last = op
            e = res.setdefault(op, {"FETCH_SIZE": 0.0, "WRITE_SIZE": 0.0, "launches": 0})
            e[counter] += v * 1024.0 * scale
            if counter == "FETCH_SIZE" and not cont:
                e["launches"] += 1
    lines = ["# HBM traffic per launch: layer sweep, 16384 tokens, seed 0 (bench step)",
             "# rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_fetch -o pmc -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-configs",
             "# rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_write -o pmc -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-configs",
             "# python bench.py --summarize-pmc OUT/pmc_fetch OUT/pmc_write   (OUT: the counter runs' output directory)",
             "# counters are scaled so that the calibration copy (256 MiB read + 256 MiB written) reads its own size;",
             "# a GEMM op includes its split-K reduce kernel and both launches of a row-split GEMM",
             f"kernel_source_hash {kernel_source_hash()}"]
    for c, (b, measured) in factors.items():
        lines.append(f"calibration {c} copy_bytes {b} counter_bytes {measured:.0f} factor {b / measured:.4f}")
    for op in sorted(res):
        e = res[op]
        n = max(e["launches"], 1)
        lines.append(f"op {op} launches {e['launches']} fetch_bytes_per_launch {e['FETCH_SIZE'] / n:.0f} "
                     f"write_bytes_per_launch {e['WRITE_SIZE'] / n:.0f} "
                     f"traffic_bytes_per_launch {(e['FETCH_SIZE'] + e['WRITE_SIZE']) / n:.0f}")
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def load_traffic():
    """op -> HBM bytes per launch, or {} when missing or taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return {}
    out, src = {}, None
    for ln in lines:
        f = ln.split()
        if f and f[0] == "kernel_source_hash":
            src = f[1]
        elif f and f[0] == "op":
            out[f[1]] = float(f[f.index("traffic_bytes_per_launch") + 1])
    return out if src == kernel_source_hash() else {}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_step(P, torch, d):
    """Allocate every buffer once; return the step's (kernel name, launch thunk, work dict,
    weight) list, the standalone single-quantizer list timed after the step, and the buffers."""
    from workloads import SWEEP_WEIGHTS
    dev = "cuda:0"
    ops, single, mxops = [], [], []

    def bf16(b):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    keep = []
    wjobs, wouts, wbytes = [], [], 0
    for wname, (dout, din) in SWEEP_WEIGHTS:
        X, W, dY = bf16(d[f"X_{wname}"]), bf16(d[f"W_{wname}"]), bf16(d[f"dY_{wname}"])
        T = X.shape[0]
        Wq, Ws, WqT, WsT = u8(dout, din), f32(dout // 128, din // 128), u8(din, dout), f32(din // 128, dout // 128)
        Xq, Xs = u8(T, din), f32(din // 128, T)
        Gq, Gs = u8(T, dout), f32(dout // 128, T)
        GqT, GsT = u8(dout, T), f32(T // 128, dout)
        XqT, XsT = u8(din, T), f32(T // 128, din)
        Y = torch.empty((T, dout), dtype=torch.bfloat16, device=dev)
        dX = torch.empty((T, din), dtype=torch.bfloat16, device=dev)
        dW = f32(dout, din)
        keep += [X, W, dY, Wq, Ws, WqT, WsT, Xq, Xs, Gq, Gs, GqT, GsT, XqT, XsT, Y, dX, dW]
        qb = lambda n: {"kind": "quant", "bytes": 2 * n + n + 4 * (n // 128)}
        qdb = lambda n: {"kind": "quant", "bytes": 2 * n + 2 * n + 2 * 4 * (n // 128)}
        qwb = {"kind": "quant", "bytes": 2 * dout * din + 2 * dout * din + 2 * 4 * (dout // 128) * (din // 128)}
        gf = lambda m, n, k, ob: {"kind": "gemm", "flops": 2 * m * n * k, "bytes": m * k + n * k + 4 * (m + n) * (k // 128) + ob * m * n}
        wjobs.append(W)
        wouts.append((Wq, Ws, WqT, WsT))
        wbytes += qwb["bytes"]
        ops += [
            ("quant_act_dual", lambda X=X, Xq=Xq, Xs=Xs, XqT=XqT, XsT=XsT: P.puro_fp8_quant_act_dual(X, Xq, Xs, XqT, XsT), qdb(T * din), wname),
            ("gemm_fwd", lambda Xq=Xq, Xs=Xs, Wq=Wq, Ws=Ws, Y=Y: P.puro_fp8_gemm(P.FWD, Xq, Xs, Wq, Ws, C=Y, out_dtype=P.OUT_BF16), gf(T, dout, din, 2), wname),
            ("quant_act_dual", lambda dY=dY, Gq=Gq, Gs=Gs, GqT=GqT, GsT=GsT: P.puro_fp8_quant_act_dual(dY, Gq, Gs, GqT, GsT), qdb(T * dout), wname),
            ("gemm_dgrad", lambda Gq=Gq, Gs=Gs, WqT=WqT, WsT=WsT, dX=dX: P.puro_fp8_gemm(P.DGRAD, Gq, Gs, WqT, WsT, C=dX, out_dtype=P.OUT_BF16), gf(T, din, dout, 2), wname),
            ("gemm_wgrad", lambda GqT=GqT, GsT=GsT, XqT=XqT, XsT=XsT, dW=dW: P.puro_fp8_gemm(P.WGRAD, GqT, GsT, XqT, XsT, C=dW, out_dtype=P.OUT_FP32), gf(dout, din, T, 4), wname),
        ]
        # MXFP8 variant of the same step (blocks of 32, E8M0 scales): W, X, dY each through the
        # MX dual quantizer (both orientations), then the three GEMMs on the MX operands
        mWq, mWx, mWqT, mWxT = u8(dout, din), u8(din // 128, dout, 4), u8(din, dout), u8(dout // 128, din, 4)
        mXq, mXx, mXqT, mXxT = u8(T, din), u8(din // 128, T, 4), u8(din, T), u8(T // 128, din, 4)
        mGq, mGx, mGqT, mGxT = u8(T, dout), u8(dout // 128, T, 4), u8(dout, T), u8(T // 128, dout, 4)
        keep += [mWq, mWx, mWqT, mWxT, mXq, mXx, mXqT, mXxT, mGq, mGx, mGqT, mGxT]
        mqb = lambda n: {"kind": "quant", "bytes": 2 * n + 2 * n + 2 * (n // 32)}
        mxops += [
            ("mx_quant_dual", lambda W=W, a=mWq, b=mWx, c=mWqT, e=mWxT: P.puro_fp8_mx_quant_dual(W, a, b, c, e), mqb(dout * din), wname),
            ("mx_quant_dual", lambda X=X, a=mXq, b=mXx, c=mXqT, e=mXxT: P.puro_fp8_mx_quant_dual(X, a, b, c, e), mqb(T * din), wname),
            ("mx_gemm_fwd", lambda a=mXq, b=mXx, c=mWq, e=mWx, Y=Y: P.puro_fp8_mx_gemm(a, b, c, e, C=Y, out_dtype=P.OUT_BF16), gf(T, dout, din, 2), wname),
            ("mx_quant_dual", lambda dY=dY, a=mGq, b=mGx, c=mGqT, e=mGxT: P.puro_fp8_mx_quant_dual(dY, a, b, c, e), mqb(T * dout), wname),
            ("mx_gemm_dgrad", lambda a=mGq, b=mGx, c=mWqT, e=mWxT, dX=dX: P.puro_fp8_mx_gemm(a, b, c, e, C=dX, out_dtype=P.OUT_BF16), gf(T, din, dout, 2), wname),
            ("mx_gemm_wgrad", lambda a=mGqT, b=mGxT, c=mXqT, e=mXxT, dW=dW: P.puro_fp8_mx_gemm(a, b, c, e, C=dW, out_dtype=P.OUT_FP32), gf(dout, din, T, 4), wname),
        ]
        Yq, Ys = u8(T, dout), f32(dout // 128, T)
        keep += [Yq, Ys]
        single += [
            ("gemm_fwd_quant_out", lambda Xq=Xq, Xs=Xs, Wq=Wq, Ws=Ws, Y=Y, Yq=Yq, Ys=Ys:
                P.puro_fp8_gemm_quant(P.FWD, Xq, Xs, Wq, Ws, C=Y, q=Yq, s=Ys), gf(T, dout, din, 2), wname),
            ("quant_act_1x128", lambda X=X, Xq=Xq, Xs=Xs: P.puro_fp8_quant_act_1x128(X, Xq, Xs), qb(T * din), wname),
            ("quant_act_1x128", lambda dY=dY, Gq=Gq, Gs=Gs: P.puro_fp8_quant_act_1x128(dY, Gq, Gs), qb(T * dout), wname),
            ("quant_act_128x1", lambda dY=dY, GqT=GqT, GsT=GsT: P.puro_fp8_quant_act_128x1(dY, GqT, GsT), qb(T * dout), wname),
            ("quant_act_128x1", lambda X=X, XqT=XqT, XsT=XsT: P.puro_fp8_quant_act_128x1(X, XqT, XsT), qb(T * din), wname),
        ]
    # the four weights are quantized anew once per step (after an optimizer step), in one launch
    ops.insert(0, ("quant_w_128x128", lambda: P.puro_fp8_quant_w_128x128_batch(wjobs, wouts),
                   {"kind": "quant", "bytes": wbytes}, "all"))
    return ops, single, mxops, keep


def config_ops(P, torch, name, d):
    """The ops of one named configuration, on its own seeded inputs: [(op name, thunk, work)]."""
    dev = "cuda:0"

    def bf16(b):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

    qb = lambda n: {"kind": "quant", "bytes": 3 * n + 4 * (n // 128)}
    qdb = lambda n: {"kind": "quant", "bytes": 4 * n + 8 * (n // 128)}
    qwb = lambda n, t: {"kind": "quant", "bytes": (4 if t else 3) * n + (8 if t else 4) * (n // 16384)}
    gf = lambda m, n, k, ob: {"kind": "gemm", "flops": 2 * m * n * k, "bytes": m * k + n * k + ob * m * n}
    ops = []
    if name in ("tiny", "qkv_fwd"):
        X, W = bf16(d["X"]), bf16(d["W"])
        (T, K), N = X.shape, W.shape[0]
        Xq, Xs = P.puro_fp8_quant_act_1x128(X)
        Wq, Ws, _, _ = P.puro_fp8_quant_w_128x128(W, transposed=False)
        out = P.OUT_FP32 if name == "tiny" else P.OUT_BF16
        Y = torch.empty((T, N), dtype=torch.float32 if name == "tiny" else torch.bfloat16, device=dev)
        ops += [("quant_act_1x128 X", lambda: P.puro_fp8_quant_act_1x128(X, Xq, Xs), qb(T * K)),
                ("quant_w_128x128 W", lambda: P.puro_fp8_quant_w_128x128(W, Wq, Ws, transposed=False), qwb(N * K, False)),
                ("gemm_fwd", lambda: P.puro_fp8_gemm(P.FWD, Xq, Xs, Wq, Ws, C=Y, out_dtype=out),
                 gf(T, N, K, 4 if name == "tiny" else 2))]
    elif name == "mlp_fwd":
        X, Wg, H, Wd = bf16(d["X"]), bf16(d["W_gu"]), bf16(d["H"]), bf16(d["W_d"])
        Xq, Xs = P.puro_fp8_quant_act_1x128(X)
        Hq, Hs = P.puro_fp8_quant_act_1x128(H)
        Wgq, Wgs, _, _ = P.puro_fp8_quant_w_128x128(Wg, transposed=False)
        Wdq, Wds, _, _ = P.puro_fp8_quant_w_128x128(Wd, transposed=False)
        G = torch.empty((X.shape[0], Wg.shape[0]), dtype=torch.bfloat16, device=dev)
        Y = torch.empty((H.shape[0], Wd.shape[0]), dtype=torch.bfloat16, device=dev)
        ops += [("quant_act_1x128 X", lambda: P.puro_fp8_quant_act_1x128(X, Xq, Xs), qb(X.numel())),
                ("quant_w_128x128 W_gu", lambda: P.puro_fp8_quant_w_128x128(Wg, Wgq, Wgs, transposed=False), qwb(Wg.numel(), False)),
                ("gemm_fwd gate_up", lambda: P.puro_fp8_gemm(P.FWD, Xq, Xs, Wgq, Wgs, C=G, out_dtype=P.OUT_BF16),
                 gf(X.shape[0], Wg.shape[0], X.shape[1], 2)),
                ("quant_act_1x128 H", lambda: P.puro_fp8_quant_act_1x128(H, Hq, Hs), qb(H.numel())),
                ("quant_w_128x128 W_d", lambda: P.puro_fp8_quant_w_128x128(Wd, Wdq, Wds, transposed=False), qwb(Wd.numel(), False)),
                ("gemm_fwd down", lambda: P.puro_fp8_gemm(P.FWD, Hq, Hs, Wdq, Wds, C=Y, out_dtype=P.OUT_BF16),
                 gf(H.shape[0], Wd.shape[0], H.shape[1], 2))]
    elif name == "down_bwd":
        dY, Wd, H = bf16(d["dY"]), bf16(d["W_d"]), bf16(d["H"])
        T, Dout = dY.shape
        Din = Wd.shape[1]
        Gq, Gs, GqT, GsT = P.puro_fp8_quant_act_dual(dY)
        Wq, Ws, WqT, WsT = P.puro_fp8_quant_w_128x128(Wd)
        HqT, HsT = P.puro_fp8_quant_act_128x1(H)
        dX = torch.empty((T, Din), dtype=torch.bfloat16, device=dev)
        dW = torch.empty((Dout, Din), dtype=torch.float32, device=dev)
        ws = torch.empty(max(P.puro_fp8_gemm_workspace_size(P.WGRAD, Dout, Din, T), 1), dtype=torch.uint8, device=dev)
        ops += [("quant_act_dual dY", lambda: P.puro_fp8_quant_act_dual(dY, Gq, Gs, GqT, GsT), qdb(dY.numel())),
                ("quant_w_128x128 W_d (+T)", lambda: P.puro_fp8_quant_w_128x128(Wd, Wq, Ws, WqT, WsT), qwb(Wd.numel(), True)),
                ("quant_act_128x1 H", lambda: P.puro_fp8_quant_act_128x1(H, HqT, HsT), qb(H.numel())),
                ("gemm_dgrad", lambda: P.puro_fp8_gemm(P.DGRAD, Gq, Gs, WqT, WsT, C=dX, out_dtype=P.OUT_BF16),
                 gf(T, Din, Dout, 2)),
                ("gemm_wgrad", lambda: P.puro_fp8_gemm(P.WGRAD, GqT, GsT, HqT, HsT, C=dW, out_dtype=P.OUT_FP32, workspace=ws),
                 gf(Dout, Din, T, 4))]
    return ops


def bench_configs(P, torch, iters: int):
    """Every named configuration besides the step's (the tiny outlier case, the QKV projection FWD at
    4096 tokens, the MLP FWD and the down-projection backward at 8192 tokens), on its own seeded
    inputs: per op, the median over `iters` launches of its HIP-event duration, each launch after a
    512 MiB write that evicts L2 and the memory-side cache (the op reads its inputs from HBM)."""
    from workloads import WORKLOADS, draw
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    out = {}
    for name in ("tiny", "qkv_fwd", "mlp_fwd", "down_bwd"):
        d = draw(name)
        ops = config_ops(P, torch, name, d)
        rows = {}
        total_us = 0.0
        for op, fn, work in ops:
            fn()
            ms = []
            for _ in range(iters):
                flush.fill_(1)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                e1.synchronize()
                ms.append(e0.elapsed_time(e1))
            us = 1000 * statistics.median(ms)
            total_us += us
            row = {"median_us": round(us, 2)}
            if work["kind"] == "gemm":
                tf = work["flops"] / (us / 1e6) / 1e12
                row.update({"gflop": round(work["flops"] / 1e9, 2), "TFLOP/s": round(tf, 1),
                            "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)})
            else:
                gbs = work["bytes"] / (us / 1e6) / 1e9
                row.update({"alg_bytes": work["bytes"], "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
            rows[op] = row
        out[name] = {"workload": WORKLOADS[name].note, "ops": rows, "total_us": round(total_us, 2)}
        del ops, d
    del flush
    return out


def cpu_model() -> str:
    """The host CPU's model name (Linux), for the oracle timing's record."""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(d, tokens: int):
    """The oracle, as it stands, on the first `tokens` tokens of the same step (all 4 weights)."""
    import numpy as np
    from oracle import gemm, quant
    from workloads import SWEEP_WEIGHTS
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    flops = 0
    t0 = time.perf_counter()
    for wname, (dout, din) in SWEEP_WEIGHTS:
        X = d[f"X_{wname}"][:tokens]
        W = d[f"W_{wname}"]
        dY = d[f"dY_{wname}"][:tokens]
        Wq, Ws, WqT, WsT = quant.quant_w_128x128(W)
        Xq, Xs = quant.quant_act_1x128(X)
        gemm.gemm("FWD", Xq, Xs, Wq, Ws)
        Gq, Gs = quant.quant_act_1x128(dY)
        gemm.gemm("DGRAD", Gq, Gs, WqT, WsT)
        GqT, GsT = quant.quant_act_128x1(dY)
        XqT, XsT = quant.quant_act_128x1(X)
        gemm.gemm("WGRAD", GqT, GsT, XqT, XsT)
        flops += 3 * 2 * tokens * dout * din
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {tokens} of 16384 tokens of the same step (all 4 weights: full 128x128 weight "
                      f"quantization, 1x128 and 128x1 activation/gradient quantization, float64 FWD/DGRAD/WGRAD); "
                      f"{dt:.1f} s on {os.cpu_count()} host cpus ({cpu_model()})",
            "seconds": dt}


def smi_sampler(samples, stop):
    """Poll amd-smi for socket power (W) and the mean GFX clock (MHz) until `stop` is set;
    appends (time, watts, mhz) to `samples`."""
    import re
    import subprocess
    smi = "/opt/rocm/bin/amd-smi"
    while not stop.is_set():
        try:
            out = subprocess.run([smi, "metric", "-p", "-c"], capture_output=True, text=True, timeout=10).stdout
        except (OSError, subprocess.TimeoutExpired):
            return
        t = time.time()
        w = re.search(r"SOCKET_POWER: (\d+) W", out)
        clks = [int(x) for x in re.findall(r"GFX_\d+:\s+CLK: (\d+) MHz", out)]
        if w and clks:
            samples.append((t, int(w.group(1)), sum(clks) / len(clks)))
        stop.wait(0.05)


def power_phases(ops, mxops, torch, secs):
    """Board power and GFX clock while the step, the MX step and each of the step's op kinds run
    back to back for `secs` seconds each (amd-smi samples; the first second of a phase is
    skipped).  Prints one JSON line per phase: median socket power, median clock, achieved rate."""
    import threading
    samples, stop = [], threading.Event()
    th = threading.Thread(target=smi_sampler, args=(samples, stop), daemon=True)
    th.start()
    phases = [("idle", [], 3.0), ("step", ops, secs), ("mx_step", mxops, secs)]
    for kind in ("gemm_fwd", "gemm_dgrad", "gemm_wgrad", "quant_act_dual", "quant_w_128x128"):
        phases.append((kind, [o for o in ops if o[0] == kind], secs))
    for name, sel, dur in phases:
        torch.cuda.synchronize()
        t0, n = time.time(), 0
        if not sel:
            time.sleep(dur)
        while sel and time.time() - t0 < dur:
            for _ in range(10):
                for o in sel:
                    o[1]()
            torch.cuda.synchronize()
            n += 10
        t1 = time.time()
        got = [x for x in samples if t0 + 1.0 <= x[0] <= t1]
        flops = sum(o[2].get("flops", 0.0) for o in sel) * n
        nbytes = sum(o[2].get("bytes", 0.0) for o in sel if o[2].get("kind") == "quant") * n
        print(json.dumps({
            "phase": name, "seconds": round(t1 - t0, 2), "passes": n, "smi_samples": len(got),
            "socket_power_w": statistics.median([x[1] for x in got]) if got else None,
            "gfx_clock_mhz": round(statistics.median([x[2] for x in got])) if got else None,
            "TFLOP/s": round(flops / (t1 - t0) / 1e12, 1) if flops else None,
            "GB/s": round(nbytes / (t1 - t0) / 1e9, 1) if nbytes else None}), flush=True)
    stop.set()
    th.join(timeout=15)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other named configurations")
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--power-phases", type=float, metavar="SECONDS",
                    help="instead of timing: board power and clock per phase (needs amd-smi)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(data-parallel ranks would each run this same step on their own tokens)", file=sys.stderr)
        sys.exit(2)

    import torch
    import blockwise_scaled_fp8_quant_amd as P
    from workloads import draw
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    log("drawing inputs (layer sweep, 16384 tokens, seed 0) ...")
    t0 = time.time()
    d = draw(WORKLOAD)
    log(f"  drawn in {time.time() - t0:.1f} s")
    ops, single, mxops, keep = build_step(P, torch, d)
    stream = torch.cuda.current_stream()
    if args.power_phases:
        power_phases(ops, mxops, torch, args.power_phases)
        return

    # calibration copy for the HBM-traffic counters (untimed; reads and writes COPY_BYTES)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst

    def run(op_list, events=None):
        for i, (_, fn, _, _) in enumerate(op_list):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    def events(n_ops, iters):
        """Start/stop HIP events for every op of `iters` passes, each recorded once here so that
        the device event exists before timing starts (torch creates it at the first record):
        building them between the warm-up and the timed passes leaves the GPU idle long enough
        for its clocks to drop, and the first timed steps then run slower."""
        ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(n_ops)]
              for _ in range(iters)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for e in [start, stop] + [x for row in ev for pair in row for x in pair]:
            e.record(stream)
        return start, stop, ev

    def timed(op_list, iters, warmup):
        """`warmup` untimed passes; `iters` timed passes with HIP events only around the whole
        run (the step time: an event pair around every op adds ~7 us of idle GPU per op); then
        `iters` more passes with an event pair around every op, for the per-kernel durations.
        Returns (ms of the uninstrumented passes, ms of the instrumented ones, per-op stats)."""
        start, stop, _ = events(0, 0)
        start2, stop2, ev = events(len(op_list), iters)
        for _ in range(warmup):
            run(op_list)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(iters):
            run(op_list)
        stop.record(stream)
        torch.cuda.synchronize()
        start2.record(stream)
        for k in range(iters):
            run(op_list, ev[k])
        stop2.record(stream)
        torch.cuda.synchronize()
        per = {}
        for k in range(iters):
            for i, (name, _, work, _) in enumerate(op_list):
                e = per.setdefault(name, {"ms": [], "flops": 0, "bytes": 0, "launches": 0, "kind": work["kind"]})
                e["ms"].append(ev[k][i][0].elapsed_time(ev[k][i][1]))
                e["launches"] += 1
                e["flops"] += work.get("flops", 0)
                e["bytes"] += work.get("bytes", 0)
        return start.elapsed_time(stop), start2.elapsed_time(stop2), per

    hbm = load_traffic()

    def rows(per, total_ms, iters, in_step):
        out = {}
        for name, e in per.items():
            tot = sum(e["ms"])
            row = {"in_step": in_step, "launches_per_step": e["launches"] // iters,
                   "avg_us": round(1000 * tot / len(e["ms"]), 2),
                   "median_us": round(1000 * statistics.median(e["ms"]), 2)}
            if in_step:
                row["share_of_step"] = round(tot / total_ms, 4)
            if e["kind"] == "gemm":
                tf = e["flops"] / (tot / 1e3) / 1e12
                row.update({"TFLOP/s": round(tf, 1), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)})
            else:
                gbs = e["bytes"] / (tot / 1e3) / 1e9
                row.update({"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
            row["alg_bytes_per_launch"] = e["bytes"] // e["launches"]
            row["hbm_bytes_per_launch"] = round(hbm[name]) if name in hbm else None
            out[name] = row
        return out

    log(f"{args.warmup} warm-up steps, then {args.steps} timed steps")
    total_ms, inst_ms, per = timed(ops, args.steps, args.warmup)
    ms_per_step = total_ms / args.steps
    kernels = rows(per, inst_ms, args.steps, True)

    # standalone single quantizers on the same tensors (outside the step)
    _, single_ms, single_per = timed(single, args.steps, 1)
    kernels.update(rows(single_per, single_ms, args.steps, False))

    # the MXFP8 variant of the step, timed the same way (not part of `value`)
    mx_ms, mx_inst_ms, mx_per = timed(mxops, args.steps, args.warmup)
    mx_step_ms = mx_ms / args.steps
    mx_variant = {"ms_per_step": round(mx_step_ms, 4),
                  "gemm_TFLOP/s_per_step": round(sum(w.get("flops", 0) for _, _, w, _ in mxops) / (mx_step_ms / 1e3) / 1e12, 2),
                  "ms_per_step_instrumented": round(mx_inst_ms / args.steps, 4),
                  "kernels": rows(mx_per, mx_inst_ms, args.steps, True)}

    configs = None
    if not args.no_configs:
        log("timing the other named configurations ...")
        configs = bench_configs(P, torch, max(args.steps, 10))

    gemm_flops = sum(w.get("flops", 0) for _, _, w, _ in ops)
    value = gemm_flops / (ms_per_step / 1e3) / 1e12
    dom = max(per, key=lambda n: sum(per[n]["ms"]))
    de = per[dom]
    traffic = hbm.get(dom)
    traffic = None if traffic is None else round(traffic)
    avg_ms = sum(de["ms"]) / len(de["ms"])
    if de["kind"] == "gemm":
        achieved = (de["flops"] / de["launches"]) / (avg_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": traffic, "kernel": dom,
                "avg_launch_us": round(1000 * avg_ms, 2)}
    else:
        achieved = (de["bytes"] / de["launches"]) / (avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                "avg_launch_us": round(1000 * avg_ms, 2)}

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the oracle on {args.cpu_tokens} tokens ...")
        cpu = cpu_baseline(d, args.cpu_tokens)
        log(f"  oracle sample took {cpu['seconds']:.1f} s")
        cpu.pop("seconds")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_instrumented": round(inst_ms / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3xfp8e4m3->fp32", "data": "synthetic",
        "config": {"workload": "layer_sweep: 16384 tokens, seed 0, weights qkv 4096x2048, o 2048x2048, "
                               "gate_up 12288x2048, down 2048x6144; per weight: W 128x128 (+T), X and dY dual "
                               "1x128+128x1 quantization, fwd+dgrad+wgrad",
                   "tokens": 16384, "gemm_gflop_per_step": round(gemm_flops / 1e9, 1),
                   "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels, "configs": configs, "mx_variant": mx_variant,
    }
    print(json.dumps(out), flush=True)
    del keep


if __name__ == "__main__":
    main()
