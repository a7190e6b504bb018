#!/usr/bin/env python3
"""Benchmark the affine group-quantized matvec kernels on one MI355X.

Default: the 4-bit, group-64 qmv of W [14336, 4096] at batch 1 (the headline
workload), one JSON line on stdout.  `--workload NAME` times another
workload, `--all` prints one line per workload, `--list` names them.

One step = one call of the workload's entry point(s) on one set of
device-resident inputs (for the FFN step: the gate/up launch and the fused
down-projection launch).  Steps rotate over enough distinct copies of the
inputs (>= 512 MB in total) that the 256 MB last-level cache cannot serve a
repeat.  The K timed steps are launched eagerly behind a bounded device spin that
holds the stream while the host enqueues them, so the timed region (HIP
events on the stream) holds only the K launches back to back: neither the
host's per-launch cost (several microseconds through Python) nor a graph
launch falls inside it.  The time of one HIP-graph replay of the K steps and
the unqueued eager time are reported beside it.  Bytes are
algorithmic: packed weights, bf16 scales and biases, activations and
outputs, each counted once per step.

Other modes (profiling aids):
  --no-cpu-baseline   skip the CPU oracle timing
  --copy-calibration  run a plain 256 MiB device copy (counter scaling)
  --copy-reference    time a plain device copy of the workload's byte count
  --read-reference    time the streaming-read reference (libqmv_bench.so) at
                      the workload's byte count, alone and with y's stores
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
CSRC = os.path.join(ROOT, "bit_affine_quantized_amd", "csrc")
# the sources whose code a workload's kernels run: the launch logic and the
# device helpers always, then its kernel family's headers
COMMON_SOURCES = ("qmv_api.hip", "qmv_device.h")
FAMILY_SOURCES = {
    "qmv": ("qmv_kernels.h", "qmv_line_kernels.h"),
    "qmm": ("qmm_kernels.h", "qvm_kernels.h", "qmf_kernels.h"),   # matrix cores (split-K or one pass)
    "ffn": ("qmv_kernels.h", "qmv_line_kernels.h"),   # gate/up runs the line kernel
    "moe": ("qmv_kernels.h", "qmm_kernels.h"),
    "qvm": ("qvm_kernels.h",),
    "pack": ("pack_kernels.h",),
}
ROTATE_BYTES = 512e6


def kernel_sources(workload: str = ""):
    rows_of_x = int(workload.rsplit("_m", 1)[1]) if re.search(r"_m\d+$", workload) else 1
    fam = ("pack" if workload.startswith(("pack_", "dequant_")) else
           "qvm" if workload.startswith("qvm_") else
           "qmm" if rows_of_x >= 5 else
           "ffn" if workload.startswith("ffn_") else
           "moe" if workload.startswith("moe_") else "qmv")
    return [os.path.join(CSRC, f) for f in COMMON_SOURCES + FAMILY_SOURCES[fam]]


def kernel_source_hash(workload: str = "") -> str:
    """Hash of the sources the workload's kernels are built from: a traffic
    summary taken on other sources is not used."""
    h = hashlib.sha256()
    for p in kernel_sources(workload):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def qbytes(N, K, bits, g):
    """Packed weight + bf16 scales + bf16 biases."""
    return N * K * bits // 8 + 2 * 2 * N * (K // g)


def read_traffic(workload: str, src_hash: str):
    """HBM bytes per launch from the committed counter summary for this
    workload, or None if absent or taken on different kernel sources."""
    path = os.path.join(PROFILE_DIR, f"{workload}.md")
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

    def __init__(self, name, nbytes, setup, launches=1, oracle_fn=None, dtype="bf16"):
        self.name, self.nbytes, self.setup = name, nbytes, setup
        self.launches, self.oracle_fn = launches, oracle_fn
        self.dtype = dtype


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
        # split-K calls (5 or more rows of x) get a caller-owned workspace
        nws = q.qmv_workspace_bytes(M, N, K, g, bits, True)
        bufs = [(x.clone(), w_q.clone(), s.clone(), b.clone(),
                 torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                 torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None)
                for _ in range(sets)]

        def step(i, stream):
            xb, wb, sb, bb, yb, ws = bufs[i % sets]
            q.qmv(xb, wb, sb, bb, group_size=g, bits=bits, y=yb, stream=stream,
                  workspace=ws)
        return step, sets

    def cpu():
        import oracle
        import synth
        w_q, s, b = oracle.quantize_pack(synth.weight((N, K)), g, bits)
        x = synth.activation_bf16((M, K))

        def blocks(T):
            edges = [N * i // T for i in range(T + 1)]
            return [(lambda r0=r0, r1=r1: oracle.qmv(
                x, w_q[r0:r1], s[r0:r1], b[r0:r1], g, bits))
                for r0, r1 in zip(edges[:-1], edges[1:]) if r1 > r0]
        return (lambda: oracle.qmv(x, w_q, s, b, g, bits),
                f"{N}x{K} b{bits} g{g} M={M} qmv", blocks)
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
        nws = q.qmv_workspace_bytes(M, N, K, g, bits, False)
        bufs = [(x.clone(), w_q.clone(), s.clone(), b.clone(),
                 torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                 torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None)
                for _ in range(sets)]

        def step(i, stream):
            xb, wb, sb, bb, yb, ws = bufs[i % sets]
            q.qmv(xb, wb, sb, bb, transpose=False, group_size=g, bits=bits,
                  y=yb, stream=stream, workspace=ws)
        return step, sets

    def cpu():
        import oracle
        import synth
        w_q, s, b = oracle.quantize_pack(synth.weight((K, N)), g, bits)
        x = synth.activation_bf16((M, K))

        def blocks(T):
            # K-row blocks give partial products; the split is summed after
            edges = [K * i // T for i in range(T + 1)]
            return [(lambda r0=r0, r1=r1: oracle.qvm(
                x[:, r0:r1], w_q[r0:r1], s[r0:r1], b[r0:r1], N, g, bits))
                for r0, r1 in zip(edges[:-1], edges[1:]) if r1 > r0]
        return (lambda: oracle.qvm(x, w_q, s, b, N, g, bits),
                f"{K}x{N} b{bits} g{g} M={M} qvm", blocks)
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

    def cpu():
        import oracle
        import synth
        w_q, s, b = oracle.quantize_pack(synth.weight((N, K)), g, bits)

        def blocks(T):
            edges = [N * i // T for i in range(T + 1)]
            return [(lambda r0=r0, r1=r1: oracle.dequantize(
                w_q[r0:r1], s[r0:r1], b[r0:r1], K, g, bits))
                for r0, r1 in zip(edges[:-1], edges[1:]) if r1 > r0]
        return (lambda: oracle.dequantize(w_q, s, b, K, g, bits),
                f"{N}x{K} b{bits} g{g} dequantize", blocks)
    return Workload(name, nbytes, setup, 1, cpu)


def make_pack(N, K, bits, g, name):
    """Device quantize + pack of an fp32 [N, K] weight: reads 4 bytes per
    weight, writes the packed codes, scales and biases."""
    nbytes = 4 * N * K + qbytes(N, K, bits, g)

    def setup(dev):
        import torch
        import bit_affine_quantized_amd as q
        import synth
        w = torch.from_numpy(synth.weight((N, K))).to(dev)
        sets = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [(w.clone(), torch.empty((N, K * bits // 32), dtype=torch.int32, device=dev),
                 torch.empty((N, K // g), dtype=torch.bfloat16, device=dev),
                 torch.empty((N, K // g), dtype=torch.bfloat16, device=dev))
                for _ in range(sets)]
        del w

        def step(i, stream):
            wb, wq, sb, bb = bufs[i % sets]
            q.qmv_pack(wb, g, bits, stream=stream, out=(wq, sb, bb))
        return step, sets
    return Workload(name, nbytes, setup, 1, dtype="f32")


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
    # 5 rows of x: the first size on the matrix cores (QMV_QMM_MIN_M=6 in
    # the environment times the same shape on 4-row slabs)
    for M in (1, 4, 5):
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
    W["pack_14336x4096_b4_g64"] = make_pack(14336, 4096, 4, 64, "pack_14336x4096_b4_g64")
    m = synth.MOE
    for srt in (False, True):
        n = f"moe_gather_64x2048x2048_b4_g64_t16_top8_{'sorted' if srt else 'unsorted'}"
        W[n] = make_moe(m["E"], m["N"], m["K"], m["bits"], m["group"],
                        m["tokens"], m["top_k"], srt, n)
    # larger routings: 4 and 5 vectors per expert on either side of the
    # matrix-core threshold (QMV_GATHER_QMM_MIN in the environment moves it),
    # and 8 and 64 per expert on the matrix cores
    for T in (32, 40, 64, 512):
        n = f"moe_gather_64x2048x2048_b4_g64_t{T}_top8_unsorted"
        W[n] = make_moe(m["E"], m["N"], m["K"], m["bits"], m["group"], T, m["top_k"], False, n)
    return W


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Threads for the multi-threaded oracle run: the CPUs this process may
    run on, capped by OMP_NUM_THREADS when the environment sets it (a shared
    host gives each GPU a share of its cores)."""
    t = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        t = min(t, int(cap))
    return max(1, t)


def _median_seconds(fn, runs):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    ts.sort()
    return ts[len(ts) // 2], ts


def cpu_baseline(wl: Workload, runs: int = 5):
    """The oracle (plain C, fp64 dequant-and-dot, untuned) on the workload's
    full inputs: median of `runs` runs at 1 thread and at T threads.  The T
    threads take contiguous row blocks of W, each calling the oracle on its
    block (ctypes releases the interpreter lock during the call)."""
    from concurrent.futures import ThreadPoolExecutor
    one, what, rows_fn = wl.oracle_fn()
    T = cpu_threads()
    t1, all1 = _median_seconds(one, runs)
    pool = ThreadPoolExecutor(max_workers=T)
    try:
        blocks = rows_fn(T)

        def many():
            list(pool.map(lambda f: f(), blocks))
        many()                                  # warm the pool
        tT, allT = _median_seconds(many, runs)
    finally:
        pool.shutdown()
    return {"value": round(wl.nbytes / tT / 1e9, 4), "unit": "GB/s",
            "cores": T, "kind": "oracle",
            "value_1_thread": round(wl.nbytes / t1 / 1e9, 4),
            "median_s": {"1": round(t1, 4), str(T): round(tT, 4)},
            "runs": runs, "cpu_model": cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{what}: the whole workload, median of {runs} runs at "
                      f"1 and at {T} threads (row blocks); plain C oracle, "
                      "fp64 dequant-and-dot"}


def _time_queued(step, steps, stream, info=None, lead_ms=2.0):
    """K eager launches queued behind a bounded device spin, timed by events.

    The spin (a few times the measured host enqueue time) holds the stream
    while the host enqueues some untimed lead steps, the start event, the K
    steps and the end event, so the timed region holds only the K launches
    running back to back; neither the host's per-launch cost nor a graph
    launch falls inside it.  The lead steps (at least `lead_ms` of GPU work)
    run between the spin and the start event, so the timed steps start on a
    GPU that has been busy with the same work, not idle behind a one-wave
    spin.  If the host took longer than the spin to enqueue, the queue may
    have drained and the time is pessimistic; `queue_drained` says so."""
    import torch
    torch.cuda.synchronize()
    probe = min(steps, 20)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    e0.record(stream)
    for i in range(probe):
        step(i, stream)
    e1.record(stream)
    host_per_step = (time.perf_counter() - h0) / probe
    torch.cuda.synchronize()
    gpu_per_step = e0.elapsed_time(e1) / probe
    lead = int(min(max(math.ceil(lead_ms / max(gpu_per_step, 1e-4)), 1), 20000))
    spin_ms = min(max(1.0, 3e3 * host_per_step * (lead + steps)), 3000.0)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(spin_ms * _spin_cycles_per_ms()))
    h0 = time.perf_counter()
    for i in range(lead):
        step(steps + i, stream)
    t0.record(stream)
    for i in range(steps):
        step(i, stream)
    t1.record(stream)
    enqueue_ms = (time.perf_counter() - h0) * 1e3
    torch.cuda.synchronize()
    if info is not None:
        info["spin_ms"] = round(spin_ms, 3)
        info["lead_steps"] = lead
        info["host_enqueue_ms"] = round(enqueue_ms, 3)
        info["queue_drained"] = enqueue_ms > spin_ms
    return t0.elapsed_time(t1) / steps


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


_SPIN_CYCLES_PER_MS = None


def _spin_cycles_per_ms():
    """Cycles of torch's device sleep kernel per millisecond on this GPU."""
    global _SPIN_CYCLES_PER_MS
    if _SPIN_CYCLES_PER_MS is None:
        import torch
        st = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record(st)
        torch.cuda._sleep(2_000_000)
        e1.record(st)
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS = 2_000_000 / max(e0.elapsed_time(e1), 1e-3)
    return _SPIN_CYCLES_PER_MS


def _time_graph(step, steps, warmup, info=None):
    """Capture `steps` steps into one HIP graph and time a replay: the GPU
    runs the launches back to back with no host launch cost in between.

    The start event would otherwise be reached while the host is still
    submitting the graph, and that submission latency would count as kernel
    time.  So a bounded device spin (a few times the measured submission
    time) is queued first: the start event, the replay and the end event are
    all enqueued while the GPU spins, and the timed region holds only the
    replayed launches."""
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
    h0 = time.perf_counter()
    graph.replay()                       # warm replay; its host submission time sizes the spin
    h1 = time.perf_counter()
    torch.cuda.synchronize()
    submit_ms = (h1 - h0) * 1e3
    spin_ms = min(max(1.0, 4.0 * submit_ms), 200.0)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(spin_ms * _spin_cycles_per_ms()))
    t0.record(stream)
    graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    if info is not None:
        info["graph_host_submit_ms"] = round(submit_ms, 3)
        info["graph_spin_ms"] = round(spin_ms, 3)
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
    qinfo, ginfo = {}, {}
    ms_queued = _time_queued(step, steps, stream, qinfo)
    ms_graph = _time_graph(step, steps, warmup, ginfo) if use_graph else None
    ms = ms_queued
    gbs = wl.nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC if wl.name.startswith("qmv_14336x4096_b4_g64_m1")
        else f"{wl.name} GB/s & % of HBM peak",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "bytes_per_step": wl.nbytes,
                   "launches_per_step": wl.launches,
                   "input_sets_rotated": sets,
                   "timing": "eager launches queued behind a device spin, HIP events",
                   **qinfo,
                   "graph_ms_per_step": None if ms_graph is None else round(ms_graph, 6),
                   **ginfo,
                   "unqueued_eager_ms_per_step": round(ms_eager, 6),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)},
    }
    res["roofline"] = {"bound": "hbm", "achieved": round(gbs, 2),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 4),
                       "traffic": read_traffic(wl.name, kernel_source_hash(wl.name))}
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


def read_reference(nbytes: int, rows: int, steps: int, split=None):
    """The streaming-read reference (libqmv_bench.so, qmv_bench_read) over
    `nbytes` bytes, rotated over >= 512 MB and timed like the workloads:
    alone, and writing one bf16 per row-sized span as a matvec writes y.
    With `split` = (weight bytes, bytes of each of scales and biases) also
    the three-array read a matvec must do (qmv_bench_read3), with y."""
    import ctypes
    import torch
    from bit_affine_quantized_amd import _build
    L = ctypes.CDLL(_build.BENCH_LIB)
    L.qmv_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                 ctypes.c_uint64, ctypes.c_void_p]
    L.qmv_bench_read.restype = ctypes.c_int
    L.qmv_bench_read3.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    L.qmv_bench_read3.restype = ctypes.c_int
    n = (nbytes // 16) * 16
    every = max(16, (n // rows) // 16 * 16)
    sets = max(2, math.ceil(ROTATE_BYTES / n))
    bufs = [(torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda"),
             torch.empty(n // every + 1, dtype=torch.int16, device="cuda"))
            for _ in range(sets)]
    torch.cuda.synchronize()
    out = {"read_bytes": n, "input_sets_rotated": sets}
    for label, store in (("read", 0), ("read_and_store", every)):
        def step(i, stream, store=store):
            a, y = bufs[i % sets]
            rc = L.qmv_bench_read(ctypes.c_void_p(a.data_ptr()), n,
                                  ctypes.c_void_p(y.data_ptr()), store,
                                  ctypes.c_void_p(stream.cuda_stream))
            if rc:
                raise RuntimeError(f"qmv_bench_read failed: {rc}")
        stream = torch.cuda.current_stream()
        for i in range(20):
            step(i, stream)
        info = {}
        ms = _time_queued(step, steps, stream, info)
        ms_graph = _time_graph(step, steps, 0)
        out[label] = {"ms_per_launch": round(ms, 6),
                      "GBs": round(n / (ms * 1e-3) / 1e9, 1),
                      "frac_of_8TBs": round(n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "graph_ms_per_launch": round(ms_graph, 6),
                      "queue_drained": info.get("queue_drained")}
        if store:
            out[label]["outputs"] = n // every
    if split is not None:
        wb, sbb = split
        sets3 = max(2, math.ceil(ROTATE_BYTES / (wb + 2 * sbb)))
        bufs3 = [(torch.randint(0, 255, (wb,), dtype=torch.uint8, device="cuda"),
                  torch.randint(0, 255, (sbb,), dtype=torch.uint8, device="cuda"),
                  torch.randint(0, 255, (sbb,), dtype=torch.uint8, device="cuda"),
                  torch.empty(rows, dtype=torch.int16, device="cuda")) for _ in range(sets3)]
        torch.cuda.synchronize()

        def step3(i, stream):
            w, sc, bi, y = bufs3[i % sets3]
            rc = L.qmv_bench_read3(ctypes.c_void_p(w.data_ptr()), wb, ctypes.c_void_p(sc.data_ptr()),
                                   ctypes.c_void_p(bi.data_ptr()), sbb, rows,
                                   ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
            if rc:
                raise RuntimeError(f"qmv_bench_read3 failed: {rc}")
        stream = torch.cuda.current_stream()
        for i in range(20):
            step3(i, stream)
        info = {}
        ms = _time_queued(step3, steps, stream, info)
        tot = wb + 2 * sbb
        out["read3_and_store"] = {"weight_bytes": wb, "scale_bytes": sbb, "bias_bytes": sbb,
                                  "ms_per_launch": round(ms, 6),
                                  "GBs": round(tot / (ms * 1e-3) / 1e9, 1),
                                  "frac_of_8TBs": round(tot / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "graph_ms_per_launch": round(_time_graph(step3, steps, 0), 6),
                                  "queue_drained": info.get("queue_drained"), "outputs": rows}
    return out


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
    ap.add_argument("--read-reference", action="store_true",
                    help="time the streaming-read reference at the workload's byte count")
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
    if args.read_reference:
        n = args.workload or synth.HEADLINE["name"]
        rows = synth.HEADLINE["N"] if n == synth.HEADLINE["name"] else 4096
        split = None
        mq = re.match(r"(?:decode_)?qmv_(\d+)x(\d+)_b(\d+)_g(\d+)_m1$", n)
        if mq:                                  # one-vector matvec: W, scales, biases
            N_, K_, b_, g_ = (int(v) for v in mq.groups())
            split = (N_ * K_ * b_ // 8, 2 * N_ * (K_ // g_))
        print(json.dumps({"workload": n, **read_reference(W[n].nbytes, rows,
                                                          args.steps, split)}))
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
