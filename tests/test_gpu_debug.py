"""QMV_DEBUG: gather_qmv checks lhs < Bx and rhs < E on the device before
running, refuses out-of-range indices with QMV_EINVAL, and otherwise gives
the same bits as without the check.  Under graph capture the check is
skipped (it must wait for the device)."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import bf16_to_np_bits, to_dev_bf16, to_dev_u32

pytestmark = pytest.mark.gpu


def _case(dev):
    import torch
    E, N, K, g, bits, Bx, P = 5, 128, 256, 64, 4, 3, 9
    ws, ss, bs = [], [], []
    for e in range(E):
        w_q, s, b = oracle.quantize_pack(synth.weight((N, K), 600 + e), g, bits)
        ws.append(w_q), ss.append(s), bs.append(b)
    x = synth.activation_bf16((Bx, 1, K), 61)
    rng = np.random.default_rng(62)
    lhs = rng.integers(0, Bx, P).astype(np.uint32)
    rhs = rng.integers(0, E, P).astype(np.uint32)
    d = dict(x=to_dev_bf16(x, dev), w=to_dev_u32(np.stack(ws), dev), s=to_dev_bf16(np.stack(ss), dev),
             b=to_dev_bf16(np.stack(bs), dev), g=g, bits=bits, E=E, Bx=Bx, lhs=lhs, rhs=rhs)
    return d, torch


def _gather(q, d, torch, lhs, rhs, dev):
    li = torch.from_numpy(lhs.astype(np.int32)).to(dev)
    ri = torch.from_numpy(rhs.astype(np.int32)).to(dev)
    return q.gather_qmv(d["x"], d["w"], d["s"], d["b"], li, ri, group_size=d["g"], bits=d["bits"])


def test_debug_check_passes_good_indices_and_refuses_bad_ones(dev, monkeypatch):
    import bit_affine_quantized_amd as q
    d, torch = _case(dev)
    monkeypatch.delenv("QMV_DEBUG", raising=False)
    want = bf16_to_np_bits(_gather(q, d, torch, d["lhs"], d["rhs"], dev))
    monkeypatch.setenv("QMV_DEBUG", "1")
    got = bf16_to_np_bits(_gather(q, d, torch, d["lhs"], d["rhs"], dev))
    np.testing.assert_array_equal(got, want)
    bad_rhs = d["rhs"].copy()
    bad_rhs[4] = d["E"]
    with pytest.raises(q.QmvError, match="out of range"):
        _gather(q, d, torch, d["lhs"], bad_rhs, dev)
    bad_lhs = d["lhs"].copy()
    bad_lhs[7] = d["Bx"] + 5
    with pytest.raises(q.QmvError, match="out of range"):
        _gather(q, d, torch, bad_lhs, d["rhs"], dev)
    monkeypatch.setenv("QMV_DEBUG", "0")                  # "0" turns it off
    np.testing.assert_array_equal(bf16_to_np_bits(_gather(q, d, torch, d["lhs"], d["rhs"], dev)), want)


def test_debug_check_is_skipped_under_graph_capture(dev, monkeypatch):
    import bit_affine_quantized_amd as q
    d, torch = _case(dev)
    monkeypatch.setenv("QMV_DEBUG", "1")
    li = torch.from_numpy(d["lhs"].astype(np.int32)).to(dev)
    ri = torch.from_numpy(d["rhs"].astype(np.int32)).to(dev)
    want = bf16_to_np_bits(q.gather_qmv(d["x"], d["w"], d["s"], d["b"], li, ri, group_size=d["g"],
                                        bits=d["bits"]))
    y = torch.empty((len(d["lhs"]), 1, 128), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):                          # warm-up on the capture stream
        q.gather_qmv(d["x"], d["w"], d["s"], d["b"], li, ri, group_size=d["g"], bits=d["bits"], y=y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        q.gather_qmv(d["x"], d["w"], d["s"], d["b"], li, ri, group_size=d["g"], bits=d["bits"], y=y)
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_to_np_bits(y), want, err_msg=f"replay {rep}")
