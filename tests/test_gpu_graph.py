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
    """transpose = 0 under capture: a warm-up call first sets up the stream's
    split-K workspace, then every replay must reproduce the eager bits."""
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
    """The split-K matrix-core path (M = 32 rows of x) under capture: a
    warm-up call sets up the stream's workspace; replays alternate with eager
    calls on the capture stream and on another stream, and every replay must
    reproduce the eager bits."""
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
