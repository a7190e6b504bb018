#!/usr/bin/env python3
"""Benchmark the affine group-quantized matvec kernels on one MI355X.

Default: the 4-bit, group-64 qmv of W [14336, 4096] at batch 1 (the headline
workload), one JSON line on stdout.  `--workload NAME` times another
workload, `--all` prints one line per workload, `--list` names them.

One step = one call of the workload's entry point(s) on one set of
device-resident inputs (for the FFN step: the gate/up launch and the fused
down-projection launch).  Steps rotate over enough distinct copies of the
inputs (>= 512 MB in total) that the 256 MB last-level cache cannot serve a
repeat.  The K timed steps are captured into one HIP graph and replayed, so
the host's per-launch cost (several microseconds through Python) does not
starve the GPU; time is taken with HIP events on the replay stream.  The
eager (host-launched) time per step is reported beside it.  Bytes are
algorithmic: packed weights, bf16 scales and biases, activations and
outputs, each counted once per step.

Other modes (profiling aids):
  --no-cpu-baseline   skip the CPU oracle timing
  --copy-calibration  run a plain 256 MiB device copy (counter scaling)
  --copy-reference    time a plain device copy of the workload's byte count
  --eager             time host-launched steps instead of a graph replay
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
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_affine_quantized_amd", "csrc", f)
                  for f in ("qmv_device.h", "qmv_kernels.h", "qmv_api.hip", "pack_kernels.h",
                            "qvm_kernels.h", "qmm_kernels.h")]
ROTATE_BYTES = 512e6


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def qbytes(N, K, bits, g):
    """Packed weight + bf16 scales + bf16 biases."""
    return N * K * bits // 8 + 2 * 2 * N * (K // g)


def read_traffic(workload: str, src_hash: str):
    """HBM bytes per launch from the committed counter summary for this
    workload, or None if absent or taken on different kernel sources."""
    path = os.path.join(PROFILE_DIR, f"traffic_{workload}.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != src_hash:
        return None
    return float(m_val.group(1))


# --------------------------------------------------------------- workloads
class Workload:
    """name, algorithmic bytes per step, and setup(dev) -> (step(i), check)."""

    def __init__(self, name, nbytes, setup, launches=1, oracle_fn=None):
        self.name, self.nbytes, self.setup = name, nbytes, setup
        self.launches, self.oracle_fn = launches, oracle_fn


def _dev_bf16(torch, a, dev):
    import numpy as np
    return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)


def make_qmv(N, K, bits, g, M, name):
    nbytes = qbytes(N, K, bits, g) + 2 * M * K + 2 * M * N

    def setup(dev):
        import torch
        import bit_affine_quantized_amd as q
        import synth
        w = torch.from_numpy(synth.weight((N, K))).to(dev)
        w_q, s, b = q.qmv_pack(w, g, bits)
        del w
        x = _dev_bf16(torch, synth.activation_bf16((M, K)), dev)
        sets = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [(x.clone(), w_q.clone(), s.clone(), b.clone(),
                 torch.empty((M, N), dtype=torch.bfloat16, device=dev))
                for _ in range(sets)]

        def step(i, stream):
            xb, wb, sb, bb, yb = bufs[i % sets]
            q.qmv(xb, wb, sb, bb, group_size=g, bits=bits, y=yb, stream=stream)
        return step, sets

    def cpu(budget_s):
        import oracle
        import synth
        w_q, s, b = oracle.quantize_pack(synth.weight((N, K)), g, bits)
        x = synth.activation_bf16((M, K))
        return lambda: oracle.qmv(x, w_q, s, b, g, bits), \
            f"full {N}x{K} b{bits} g{g} M={M} qmv"
    return Workload(name, nbytes, setup, 1, cpu)


def make_qvm(K, N, bits, g, M, name):
    """transpose = 0: y [M, N] = x [M, K] @ W_hat with W packed [K, N] along
    N.  Algorithmic bytes: packed W, scales and biases, x and y once (the
    split-K partial sums are not counted)."""
    nbytes = qbytes(K, N, bits, g) + 2 * M * K + 2 * M * N

    def setup(dev):
        import torch
        import bit_affine_quantized_amd as q
        import synth
        w = torch.from_numpy(synth.weight((K, N))).to(dev)
        w_q, s, b = q.qmv_pack(w, g, bits)
        del w
        x = _dev_bf16(torch, synth.activation_bf16((M, K)), dev)
        sets = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [(x.clone(), w_q.clone(), s.clone(), b.clone(),
                 torch.empty((M, N), dtype=torch.bfloat16, device=dev))
                for _ in range(sets)]

        def step(i, stream):
            xb, wb, sb, bb, yb = bufs[i % sets]
            q.qmv(xb, wb, sb, bb, transpose=False, group_size=g, bits=bits,
                  y=yb, stream=stream)
        return step, sets

    def cpu(budget_s):
        import oracle
        import synth
        w_q, s, b = oracle.quantize_pack(synth.weight((K, N)), g, bits)
        x = synth.activation_bf16((M, K))
        return lambda: oracle.qvm(x, w_q, s, b, N, g, bits), \
            f"full {K}x{N} b{bits} g{g} M={M} qvm"
    return Workload(name, nbytes, setup, 1, cpu)


def make_dequant(N, K, bits, g, name):
    """Device dequantize to bf16 [N, K]: reads the packed weight, writes
    2 bytes per weight."""
    nbytes = qbytes(N, K, bits, g) + 2 * N * K

    def setup(dev):
        import torch
        import bit_affine_quantized_amd as q
        import synth
        w = torch.from_numpy(synth.weight((N, K))).to(dev)
        w_q, s, b = q.qmv_pack(w, g, bits)
        del w
        sets = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [(w_q.clone(), s.clone(), b.clone(),
                 torch.empty((N, K), dtype=torch.bfloat16, device=dev))
                for _ in range(sets)]

        def step(i, stream):
            wb, sb, bb, ob = bufs[i % sets]
            q.qmv_dequantize(wb, sb, bb, g, bits, out=ob, stream=stream)
        return step, sets

    def cpu(budget_s):
        import oracle
        import synth
        w_q, s, b = oracle.quantize_pack(synth.weight((N, K)), g, bits)
        return lambda: oracle.dequantize(w_q, s, b, K, g, bits), \
            f"full {N}x{K} b{bits} g{g} dequantize"
    return Workload(name, nbytes, setup, 1, cpu)


def make_gate_up(N, K, bits, g, name):
    nbytes = 2 * qbytes(N, K, bits, g) + 2 * K + 2 * 2 * N

    def setup(dev):
        import torch
        import bit_affine_quantized_amd as q
        import synth
        packs = []
        for seed in (synth.SEED_W, synth.SEED_UP):
            w = torch.from_numpy(synth.weight((N, K), seed)).to(dev)
            packs.append(q.qmv_pack(w, g, bits))
            del w
        x = _dev_bf16(torch, synth.activation_bf16((K,)), dev)
        sets = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [(x.clone(), tuple(t.clone() for t in packs[0]),
                 tuple(t.clone() for t in packs[1]),
                 torch.empty(N, dtype=torch.bfloat16, device=dev),
                 torch.empty(N, dtype=torch.bfloat16, device=dev))
                for _ in range(sets)]

        def step(i, stream):
            xb, gw, uw, gy, uy = bufs[i % sets]
            q.qmv_gate_up(xb, gw, uw, group_size=g, bits=bits, gate_y=gy,
                          up_y=uy, stream=stream)
        return step, sets
    return Workload(name, nbytes, setup, 1)


def make_silu_down(N, K, bits, g, name):
    """W_down [N, K]: gate/up [K], residual and y [N]."""
    nbytes = qbytes(N, K, bits, g) + 2 * 2 * K + 2 * 2 * N

    def setup(dev):
        import torch
        import bit_affine_quantized_amd as q
        import synth
        w = torch.from_numpy(synth.weight((N, K), synth.SEED_DOWN)).to(dev)
        pack = q.qmv_pack(w, g, bits)
        del w
        gate = _dev_bf16(torch, synth.activation_bf16((K,), 1), dev)
        up = _dev_bf16(torch, synth.activation_bf16((K,), 2), dev)
        xr = _dev_bf16(torch, synth.activation_bf16((N,), synth.SEED_XRESID),
                       dev)
        sets = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [(gate.clone(), up.clone(), xr.clone(),
                 tuple(t.clone() for t in pack),
                 torch.empty(N, dtype=torch.bfloat16, device=dev))
                for _ in range(sets)]

        def step(i, stream):
            gb, ub, rb, wd, yb = bufs[i % sets]
            q.qmv_silu_gate_resid(gb, ub, rb, *wd, group_size=g, bits=bits,
                                  y=yb, stream=stream)
        return step, sets
    return Workload(name, nbytes, setup, 1)


def make_ffn(N, K, bits, g, name):
    """gate/up [N, K] in one launch, then down [K, N] with silu and residual."""
    nbytes = (2 * qbytes(N, K, bits, g) + 2 * K + 2 * 2 * N) + \
        (qbytes(K, N, bits, g) + 2 * 2 * N + 2 * 2 * K)

    def setup(dev):
        import torch
        import bit_affine_quantized_amd as q
        import synth
        packs = []
        for seed, shape in ((synth.SEED_W, (N, K)), (synth.SEED_UP, (N, K)),
                            (synth.SEED_DOWN, (K, N))):
            w = torch.from_numpy(synth.weight(shape, seed)).to(dev)
            packs.append(q.qmv_pack(w, g, bits))
            del w
        x = _dev_bf16(torch, synth.activation_bf16((K,)), dev)
        xr = _dev_bf16(torch, synth.activation_bf16((K,), synth.SEED_XRESID),
                       dev)
        sets = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [(x.clone(), xr.clone(),
                 [tuple(t.clone() for t in p) for p in packs],
                 torch.empty(N, dtype=torch.bfloat16, device=dev),
                 torch.empty(N, dtype=torch.bfloat16, device=dev),
                 torch.empty(K, dtype=torch.bfloat16, device=dev))
                for _ in range(sets)]

        def step(i, stream):
            xb, rb, (gw, uw, dw), gy, uy, yb = bufs[i % sets]
            q.qmv_gate_up(xb, gw, uw, group_size=g, bits=bits, gate_y=gy,
                          up_y=uy, stream=stream)
            q.qmv_silu_gate_resid(gy, uy, rb, *dw, group_size=g, bits=bits,
                                  y=yb, stream=stream)
        return step, sets
    return Workload(name, nbytes, setup, 2)


def make_moe(E, N, K, bits, g, T, top, sorted_idx, name):
    import numpy as np
    import synth
    lhs, rhs = synth.moe_indices(T, top, E)
    used = len(np.unique(rhs))
    P = T * top
    # distinct experts' weights once, x, y, indices
    nbytes = used * qbytes(N, K, bits, g) + 2 * T * K + 2 * P * N + 2 * 4 * P

    def setup(dev):
        import torch
        import bit_affine_quantized_amd as q
        ws, ss, bs = [], [], []
        for e in range(E):
            w = torch.from_numpy(synth.weight((N, K), 1000 + e)).to(dev)
            a, b_, c = q.qmv_pack(w, g, bits)
            ws.append(a), ss.append(b_), bs.append(c)
            del w
        w_q, s, b = torch.stack(ws), torch.stack(ss), torch.stack(bs)
        del ws, ss, bs
        x = _dev_bf16(torch, synth.activation_bf16((T, 1, K)), dev)
        l_np, r_np = lhs.ravel(), rhs.ravel()
        if sorted_idx:
            perm = np.argsort(r_np, kind="stable")
            l_np, r_np = l_np[perm], r_np[perm]
        li = torch.from_numpy(l_np.astype(np.int32)).to(dev)
        ri = torch.from_numpy(r_np.astype(np.int32)).to(dev)
        full = E * qbytes(N, K, bits, g)
        sets = max(2, math.ceil(ROTATE_BYTES / full))
        bufs = [(x.clone(), w_q.clone(), s.clone(), b.clone(), li.clone(),
                 ri.clone(), torch.empty((P, 1, N), dtype=torch.bfloat16,
                                         device=dev)) for _ in range(sets)]

        def step(i, stream):
            xb, wb, sb, bb, lb, rb, yb = bufs[i % sets]
            q.gather_qmv(xb, wb, sb, bb, lb, rb, group_size=g, bits=bits,
                         sorted_indices=sorted_idx, y=yb, stream=stream)
        return step, sets
    return Workload(name, nbytes, setup, 1)


def workloads():
    import synth
    W = {}
    h = synth.HEADLINE
    W[h["name"]] = make_qmv(h["N"], h["K"], h["bits"], h["group"], 1, h["name"])
    t = synth.TINY
    W[t["name"]] = make_qmv(t["N"], t["K"], t["bits"], t["group"], 1, t["name"])
    for M in (1, 4):
        n = f"decode_qmv_4096x4096_b4_g64_m{M}"
        W[n] = make_qmv(4096, 4096, 4, 64, M, n)
    for bits in (2, 3, 5, 6, 8):
        for g in (32, 64, 128):
            n = f"qmv_14336x4096_b{bits}_g{g}_m1"
            W[n] = make_qmv(14336, 4096, bits, g, 1, n)
    W["ffn_gate_up_14336x4096_b8_g64"] = make_gate_up(
        14336, 4096, 8, 64, "ffn_gate_up_14336x4096_b8_g64")
    W["ffn_down_silu_resid_4096x14336_b8_g64"] = make_silu_down(
        4096, 14336, 8, 64, "ffn_down_silu_resid_4096x14336_b8_g64")
    W["ffn_step_14336x4096_b8_g64"] = make_ffn(
        14336, 4096, 8, 64, "ffn_step_14336x4096_b8_g64")
    for M in (8, 16, 64):
        n = f"qmm_4096x4096_b4_g64_m{M}"
        W[n] = make_qmv(4096, 4096, 4, 64, M, n)
    for M in (1, 4):
        n = f"qvm_4096x4096_b4_g64_m{M}"
        W[n] = make_qvm(4096, 4096, 4, 64, M, n)
    W["dequant_14336x4096_b4_g64"] = make_dequant(14336, 4096, 4, 64,
                                                  "dequant_14336x4096_b4_g64")
    m = synth.MOE
    for srt in (False, True):
        n = f"moe_gather_64x2048x2048_b4_g64_t16_top8_{'sorted' if srt else 'unsorted'}"
        W[n] = make_moe(m["E"], m["N"], m["K"], m["bits"], m["group"],
                        m["tokens"], m["top_k"], srt, n)
    # larger routings (8 and 64 vectors per expert): the matrix-core gather
    for T in (64, 512):
        n = f"moe_gather_64x2048x2048_b4_g64_t{T}_top8_unsorted"
        W[n] = make_moe(m["E"], m["N"], m["K"], m["bits"], m["group"], T, m["top_k"], False, n)
    return W


def cpu_baseline(wl: Workload, budget_s=10.0):
    fn, what = wl.oracle_fn(budget_s)
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / reps
    return {"value": round(wl.nbytes / per / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{what}, {reps} runs in {el:.1f} s (plain C, fp64 "
                      "dequant-and-dot, 1 thread)"}


def _time_eager(step, steps, stream):
    import torch
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        step(i, stream)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def _time_graph(step, steps, warmup):
    """Capture `steps` steps into one HIP graph and time a replay: the GPU
    runs the launches back to back with no host launch cost in between."""
    import torch
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):        # per-stream set-up happens outside capture
        step(0, side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        cs = torch.cuda.current_stream()
        for i in range(steps):
            step(i, cs)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    graph.replay()                       # warm replay
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del graph
    return ms


def run_workload(wl: Workload, steps: int, warmup: int, want_cpu: bool,
                 use_graph: bool = True):
    import torch
    dev = torch.device("cuda:0")
    step, sets = wl.setup(dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i, stream)
    torch.cuda.synchronize()
    ms_eager = _time_eager(step, steps, stream)
    ms = _time_graph(step, steps, warmup) if use_graph else ms_eager
    gbs = wl.nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC if wl.name.startswith("qmv_14336x4096_b4_g64_m1")
        else f"{wl.name} GB/s & % of HBM peak",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "bytes_per_step": wl.nbytes,
                   "launches_per_step": wl.launches,
                   "input_sets_rotated": sets,
                   "timing": "hip_graph_replay" if use_graph else "eager",
                   "eager_ms_per_step": round(ms_eager, 6),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)},
    }
    res["roofline"] = {"bound": "hbm", "achieved": round(gbs, 2),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 4),
                       "traffic": read_traffic(wl.name, kernel_source_hash())}
    res["cpu_baseline"] = cpu_baseline(wl) if (want_cpu and wl.oracle_fn) \
        else None
    del step
    torch.cuda.empty_cache()
    return res


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


def copy_reference(nbytes: int, steps: int):
    """A plain device copy of `nbytes` (read + write), rotated over >= 512 MB
    and timed like the workloads: what a streaming kernel of this size
    achieves on this machine, for context beside the roofline."""
    import torch
    n = (nbytes // 4096) * 4096
    sets = max(2, math.ceil(ROTATE_BYTES / (2 * n)))
    bufs = [(torch.ones(n, dtype=torch.uint8, device="cuda"),
             torch.empty(n, dtype=torch.uint8, device="cuda"))
            for _ in range(sets)]
    torch.cuda.synchronize()

    def step(i, stream):
        a, b = bufs[i % sets]
        b.copy_(a)
    for i in range(20):
        step(i, None)
    ms = _time_graph(step, steps, 0)
    return {"copy_bytes": n, "ms_per_copy": round(ms, 6),
            "read_plus_write_GBs": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "frac_of_8TBs": round(2 * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--list", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--copy-reference", action="store_true",
                    help="time a plain device copy of the workload's size")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of a graph replay")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} "
              "is not supported (the qmv path has no multi-GPU leg here)",
              file=sys.stderr)
        sys.exit(2)

    W = workloads()
    if args.list:
        for n, w in W.items():
            print(n, w.nbytes)
        return
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    import synth
    if args.copy_reference:
        n = args.workload or synth.HEADLINE["name"]
        print(json.dumps({"workload": n, **copy_reference(W[n].nbytes,
                                                          args.steps)}))
        return
    names = list(W) if args.all else [args.workload or synth.HEADLINE["name"]]
    for n in names:
        if n not in W:
            print(f"unknown workload {n}; --list shows them", file=sys.stderr)
            sys.exit(2)
        want_cpu = not args.no_cpu_baseline and (n == synth.HEADLINE["name"])
        print(json.dumps(run_workload(W[n], args.steps, args.warmup,
                                      want_cpu, not args.eager)), flush=True)


if __name__ == "__main__":
    main()
