#!/usr/bin/env python3
"""Benchmark: affine group-quantized qmv, 4-bit codes, group 64,
W [14336, 4096], batch 1, on one MI355X.

One step = one qmv call (stage x, stream the packed weight, unpack, dot,
fold scales/biases, reduce, store) over one set of device-resident inputs.
Steps rotate over enough distinct weight copies (>= 512 MB in total) that the
256 MB last-level cache cannot serve a repeat.  Time is taken with HIP events
on the stream the kernel runs on, around the K timed launches.

Prints ONE JSON line.  Extra modes for profiling runs:
  --no-cpu-baseline   skip the CPU oracle timing
  --copy-calibration  time a plain device copy of known size (for counter
                      scaling) instead of the qmv workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "qmv GB/s & % of HBM peak, 4-bit g64 N=14336 K=4096 batch 1"
HBM_PEAK_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "qmv_b4_g64_14336x4096_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_affine_quantized_amd", "csrc", f)
                  for f in ("qmv_device.h", "qmv_kernels.h", "qmv_api.hip")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(N, K, bits, g, M) -> int:
    """Packed W + bf16 scales and biases + bf16 x + bf16 y, each once."""
    return N * K * bits // 8 + 2 * 2 * N * (K // g) + 2 * M * K + 2 * M * N


def read_traffic(src_hash: str):
    """HBM bytes per launch from the committed counter summary, or None if
    the summary is missing or was taken on different kernel sources."""
    try:
        text = open(PROFILE_TRAFFIC).read()
    except OSError:
        return None
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != src_hash:
        return None
    return float(m_val.group(1))


def cpu_baseline(N, K, bits, g, M, budget_s=10.0):
    """The oracle (plain C, fp64, one thread) on the same workload shape."""
    import numpy as np

    import oracle
    import synth

    w = synth.weight((N, K))
    w_q, s, b = oracle.quantize_pack(w, g, bits)
    x = synth.activation_bf16((M, K))
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.qmv(x, w_q, s, b, g, bits)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / reps
    return {"value": algorithmic_bytes(N, K, bits, g, M) / per / 1e9,
            "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"full {N}x{K} b{bits} g{g} M={M} qmv, {reps} runs "
                      f"({el:.1f} s), fp64 dequant-and-dot, 1 thread",
            "ms_per_call": per * 1e3}


def copy_calibration(steps: int):
    import torch
    n = 256 * 1024 * 1024
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n,
                      "copy_calibration_bytes_written": n, "launches": steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} "
              "is not supported (the qmv path has no multi-GPU leg here)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_affine_quantized_amd as q
    import synth

    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    cfg = synth.HEADLINE
    N, K, bits, g, M = cfg["N"], cfg["K"], cfg["bits"], cfg["group"], cfg["M"]
    dev = torch.device("cuda:0")
    nbytes = algorithmic_bytes(N, K, bits, g, M)
    sets = max(2, math.ceil(512e6 / nbytes))

    # device-resident inputs: quantize once on the device, replicate
    w = torch.from_numpy(synth.weight((N, K))).to(dev)
    w_q, s, b = q.qmv_pack(w, g, bits)
    del w
    x_bits = synth.activation_bf16((M, K))
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    bufs = []
    for _ in range(sets):
        bufs.append((x.clone(), w_q.clone(), s.clone(), b.clone(),
                     torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(i):
        xb, wb, sb, bb, yb = bufs[i % sets]
        q.qmv(xb, wb, sb, bb, group_size=g, bits=bits, y=yb, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9

    result = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "N": N, "K": K, "bits": bits,
                   "group_size": g, "batch": M, "transpose": True,
                   "bytes_per_step": nbytes, "weight_sets_rotated": sets,
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)},
    }
    traffic = read_traffic(kernel_source_hash())
    result["roofline"] = {"bound": "hbm", "achieved": round(gbs, 2),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbs / HBM_PEAK_GBS, 4),
                          "traffic": traffic}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(N, K, bits, g, M)
        cb.pop("ms_per_call", None)
        cb["value"] = round(cb["value"], 4)
        result["cpu_baseline"] = cb
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
