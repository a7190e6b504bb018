"""The kernels under HIP graph capture: every replay must give the same bits
as the eager call.  Replays are interleaved with eager work and host
synchronizations, and each replay's output is checked on its own."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import bf16_to_np_bits, to_dev_bf16, to_dev_u32

pytestmark = pytest.mark.gpu


def _packed(N, K, bits, g, dev, seed=0):
    w_q, s, b = oracle.quantize_pack(synth.weight((N, K), seed), g, bits)
    return to_dev_u32(w_q, dev), to_dev_bf16(s, dev), to_dev_bf16(b, dev)


@pytest.mark.parametrize("bits", (4, 8, 3))
def test_qmv_graph_replays_match_eager(dev, bits):
    import torch

    import bit_affine_quantized_amd as q
    N, K, g = 1000, 2048, 64
    w = _packed(N, K, bits, g, dev)
    x = to_dev_bf16(synth.activation_bf16((1, K), 5), dev)
    y_eager = bf16_to_np_bits(q.qmv(x, *w, group_size=g, bits=bits))
    y = torch.zeros((1, N), dtype=torch.bfloat16, device=dev)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=side):
        q.qmv(x, *w, group_size=g, bits=bits, y=y)
    torch.cuda.synchronize()
    for rep in range(4):
        y.zero_()                                  # eager work between replays
        junk = q.qmv(x, *w, group_size=g, bits=bits)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_to_np_bits(y), y_eager,
                                      err_msg=f"replay {rep}")
        del junk


def test_ffn_graph_replays_match_eager(dev):
    import torch

    import bit_affine_quantized_amd as q
    N, K, g, bits = 2048, 1024, 64, 8
    wg, wu = _packed(N, K, bits, g, dev, 0), _packed(N, K, bits, g, dev, 1)
    wd = _packed(K, N, bits, g, dev, 2)
    x = to_dev_bf16(synth.activation_bf16((K,), 5), dev)
    xr = to_dev_bf16(synth.activation_bf16((K,), 6), dev)
    gy, uy = q.qmv_gate_up(x, wg, wu, group_size=g, bits=bits)
    y_eager = bf16_to_np_bits(q.qmv_silu_gate_resid(gy, uy, xr, *wd,
                                                    group_size=g, bits=bits))
    gy2 = torch.empty_like(gy)
    uy2 = torch.empty_like(uy)
    y = torch.empty((K,), dtype=torch.bfloat16, device=dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        q.qmv_gate_up(x, wg, wu, group_size=g, bits=bits, gate_y=gy2, up_y=uy2)
        q.qmv_silu_gate_resid(gy2, uy2, xr, *wd, group_size=g, bits=bits, y=y)
    for rep in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_to_np_bits(y), y_eager,
                                      err_msg=f"replay {rep}")


def test_qvm_graph_replays_match_eager(dev):
    """transpose = 0 (split K) under capture: the call's stream-ordered
    workspace becomes part of the graph, and every replay must reproduce the
    eager bits."""
    import torch

    import bit_affine_quantized_amd as q
    K, N, g, bits = 4096, 2048, 64, 4
    w_q, s, b = oracle.quantize_pack(synth.weight((K, N), 0), g, bits)
    w = (to_dev_u32(w_q, dev), to_dev_bf16(s, dev), to_dev_bf16(b, dev))
    x = to_dev_bf16(synth.activation_bf16((1, K), 5), dev)
    side = torch.cuda.Stream()
    y = torch.zeros((1, N), dtype=torch.bfloat16, device=dev)
    with torch.cuda.stream(side):
        q.qmv(x, *w, transpose=False, group_size=g, bits=bits, y=y)   # warm-up
    torch.cuda.synchronize()
    y_eager = bf16_to_np_bits(y)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        q.qmv(x, *w, transpose=False, group_size=g, bits=bits, y=y)
    torch.cuda.synchronize()
    for rep in range(4):
        y.zero_()
        junk = q.qmv(x, *w, transpose=False, group_size=g, bits=bits)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_to_np_bits(y), y_eager, err_msg=f"replay {rep}")
        del junk


def test_qmm_graph_replays_match_eager(dev):
    """The split-K matrix-core path (M = 32 rows of x) under capture: replays
    alternate with eager calls on the capture stream and on another stream,
    and every replay must reproduce the eager bits."""
    import torch

    import bit_affine_quantized_amd as q
    M, N, K, g, bits = 32, 1024, 2048, 64, 4
    w = _packed(N, K, bits, g, dev, seed=3)
    x = to_dev_bf16(synth.activation_bf16((M, K), 7), dev)
    side = torch.cuda.Stream()
    y = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
    with torch.cuda.stream(side):
        q.qmv(x, *w, group_size=g, bits=bits, y=y)                       # warm-up
    torch.cuda.synchronize()
    y_eager = bf16_to_np_bits(y)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        q.qmv(x, *w, group_size=g, bits=bits, y=y)
    torch.cuda.synchronize()
    for rep in range(4):
        y.zero_()
        junk = q.qmv(x, *w, group_size=g, bits=bits)                     # default stream
        with torch.cuda.stream(side):
            junk2 = q.qmv(x, *w, group_size=g, bits=bits)                # capture stream
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_to_np_bits(junk2), y_eager, err_msg=f"eager {rep}")
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_to_np_bits(y), y_eager, err_msg=f"replay {rep}")
        del junk, junk2


def _split_k_cases(dev):
    """Two split-K calls with different inputs: transpose = 0 (qvm) and 32
    rows of x on the matrix cores."""
    K, N, g, bits = 2048, 1024, 64, 4
    wv = oracle.quantize_pack(synth.weight((K, N), 11), g, bits)
    wm = oracle.quantize_pack(synth.weight((N, K), 12), g, bits)
    xv = synth.activation_bf16((2, K), 21)
    xm = synth.activation_bf16((32, K), 22)
    cases = [
        dict(x=xv, w=wv, transpose=False, M=2, ref=oracle.qvm(xv, *wv, N, g, bits)),
        dict(x=xm, w=wm, transpose=True, M=32, ref=oracle.qmv(xm, *wm, g, bits)),
    ]
    for c in cases:
        c["xd"] = to_dev_bf16(c["x"], dev)
        c["wd"] = tuple(f(a, dev) for f, a in zip((to_dev_u32, to_dev_bf16, to_dev_bf16), c["w"]))
    return cases, K, N, g, bits


@pytest.mark.parametrize("own_workspace", (True, False))
def test_split_k_graphs_replayed_concurrently_on_two_streams(dev, own_workspace):
    """Two graphs captured on ONE stream, each holding a split-K call, are
    replayed on two different streams with no synchronization between them.
    Each must match the oracle (T2): a workspace shared between the two
    would mix their partial sums.  With own_workspace each call gets a
    caller-owned workspace; otherwise qmv's stream-ordered allocation is
    captured into each graph."""
    import torch

    import bit_affine_quantized_amd as q
    from tests.parity import check_t2
    cases, K, N, g, bits = _split_k_cases(dev)
    side = torch.cuda.Stream()
    graphs = []
    for c in cases:
        c["y"] = torch.zeros((c["M"], N), dtype=torch.float32, device=dev)
        ws = None
        if own_workspace:
            nb = q.qmv_workspace_bytes(c["M"], N, K, g, bits, c["transpose"])
            assert nb > 0
            ws = torch.empty(nb, dtype=torch.uint8, device=dev)
            c["ws"] = ws
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            q.qmv(c["xd"], *c["wd"], transpose=c["transpose"], group_size=g, bits=bits,
                  out_dtype=torch.float32, y=c["y"], workspace=ws)
        graphs.append(gr)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(5):
        for c in cases:
            c["y"].fill_(-1.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            graphs[0].replay()
        with torch.cuda.stream(s2):
            graphs[1].replay()
        with torch.cuda.stream(s1):
            graphs[0].replay()
        torch.cuda.synchronize()
        for i, c in enumerate(cases):
            check_t2(c["y"].cpu().numpy(), c["ref"], f"graph {i} replay {rep}")


def test_with_workspace_is_bit_identical_to_qmv(dev):
    """qmv_with_workspace and qmv run the same kernels in the same order."""
    import torch

    import bit_affine_quantized_amd as q
    cases, K, N, g, bits = _split_k_cases(dev)
    for c in cases:
        y0 = q.qmv(c["xd"], *c["wd"], transpose=c["transpose"], group_size=g, bits=bits)
        nb = q.qmv_workspace_bytes(c["M"], N, K, g, bits, c["transpose"])
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        y1 = q.qmv(c["xd"], *c["wd"], transpose=c["transpose"], group_size=g, bits=bits,
                   workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_to_np_bits(y0), bf16_to_np_bits(y1))


def test_with_workspace_too_small_raises(dev):
    import torch

    import bit_affine_quantized_amd as q
    cases, K, N, g, bits = _split_k_cases(dev)
    c = cases[0]
    nb = q.qmv_workspace_bytes(c["M"], N, K, g, bits, c["transpose"])
    ws = torch.empty(nb - 64, dtype=torch.uint8, device=dev)
    with pytest.raises(q.QmvError, match="workspace"):
        q.qmv(c["xd"], *c["wd"], transpose=c["transpose"], group_size=g, bits=bits, workspace=ws)
