"""Split-K calls with a caller-owned workspace (qmv_with_workspace) against
qmv's stream-ordered one: the same kernels add the same fp32 partials in
slice order, so the outputs must be bit-identical, and both must meet the
oracle's tolerance.  One workspace serves any later call, of any shape,
that it is large enough for, and calls queued back to back on one stream
may share it."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import bf16_to_np_bits, check_t1, check_t2, to_dev_bf16, to_dev_u32

pytestmark = pytest.mark.gpu


def _case(dev, M, N, K, transpose, seed, g=64, bits=4):
    shape = (N, K) if transpose else (K, N)
    w_q, s, b = oracle.quantize_pack(synth.weight(shape, seed), g, bits)
    x = synth.activation_bf16((M, K), seed + 70)
    ref = oracle.qmv(x, w_q, s, b, g, bits) if transpose else oracle.qvm(x, w_q, s, b, N, g, bits)
    return dict(M=M, N=N, K=K, transpose=transpose, g=g, bits=bits, ref=ref,
                x=to_dev_bf16(x, dev), w=(to_dev_u32(w_q, dev), to_dev_bf16(s, dev), to_dev_bf16(b, dev)))


def _call(q, c, out_f32, workspace=None):
    import torch
    y = q.qmv(c["x"], *c["w"], transpose=c["transpose"], group_size=c["g"], bits=c["bits"],
              out_dtype=torch.float32 if out_f32 else None, workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy() if out_f32 else bf16_to_np_bits(y)


# (M, N, K, transpose): qvm with one and four vectors, a ragged column block
# (N not a multiple of 512) and many slices (large K); the split-K
# matrix-core path with one and two 64-row slabs (the second launch reuses
# the counters) and a ragged row block (N not a multiple of 64).  (4-bit with
# K = 2048 or 4096 and at most 16 rows runs in one pass with no workspace:
# test_one_pass_shapes_need_no_workspace.)
CASES = [
    (1, 4096, 4096, False), (4, 1024, 4096, False), (2, 4160, 2048, False),
    (1, 512, 16384, False),
    (8, 4096, 8192, True), (64, 1024, 2048, True), (100, 1000, 1024, True),
    (5, 2112, 1024, True),
]


@pytest.mark.parametrize("M,N,K,transpose", CASES)
@pytest.mark.parametrize("out_f32", (False, True))
def test_with_workspace_equals_qmv_and_oracle(dev, M, N, K, transpose, out_f32):
    import torch

    import bit_affine_quantized_amd as q
    c = _case(dev, M, N, K, transpose, seed=M + N + K)
    nb = q.qmv_workspace_bytes(M, N, K, 64, 4, transpose)
    assert nb > 0
    ws = torch.full((nb,), 0x7F, dtype=torch.uint8, device=dev)   # stale contents
    y2 = _call(q, c, out_f32)
    for rep in range(3):
        y1 = _call(q, c, out_f32, ws)
        np.testing.assert_array_equal(y1, y2, err_msg=f"call {rep}")
    (check_t2 if out_f32 else check_t1)(y1, c["ref"], f"M={M} N={N} K={K} transpose={transpose}")


def test_one_workspace_serves_calls_of_different_shapes(dev):
    """A workspace sized for the largest call, used by split-K calls of both
    kinds and several shapes in turn, then by the same calls again: every
    output equals qmv's."""
    import torch

    import bit_affine_quantized_amd as q
    shapes = [(64, 4096, 4096, True), (1, 4096, 4096, False), (8, 1000, 1024, True),
              (4, 4160, 2048, False)]
    cases = [_case(dev, *sh, seed=100 + i) for i, sh in enumerate(shapes)]
    nb = max(q.qmv_workspace_bytes(M, N, K, 64, 4, t) for (M, N, K, t) in shapes)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    want = [_call(q, c, False) for c in cases]
    for rnd in range(2):
        for i, c in enumerate(cases):
            np.testing.assert_array_equal(_call(q, c, False, ws), want[i], err_msg=f"round {rnd} case {i}")


def test_with_workspace_back_to_back_without_sync(dev):
    """Many calls queued on one stream with one workspace and no host
    synchronization between them: stream order keeps each call's partial
    sums from the next call's."""
    import torch

    import bit_affine_quantized_amd as q
    c = _case(dev, 24, 2048, 4096, True, seed=7)
    nb = q.qmv_workspace_bytes(24, 2048, 4096, 64, 4, True)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    want = _call(q, c, False)
    ys = [q.qmv(c["x"], *c["w"], group_size=64, bits=4, workspace=ws) for _ in range(20)]
    torch.cuda.synchronize()
    for i, y in enumerate(ys):
        np.testing.assert_array_equal(bf16_to_np_bits(y), want, err_msg=f"call {i}")


@pytest.mark.parametrize("M,N,K", [(5, 4096, 4096), (16, 1000, 2048)])
def test_one_pass_shapes_need_no_workspace(dev, M, N, K):
    """4-bit, K = 2048 or 4096, 5-16 rows of x: the one-pass matrix-core
    product splits K inside a workgroup only, so the workspace size is 0 and
    qmv_with_workspace runs without one, equal to qmv."""
    import torch

    import bit_affine_quantized_amd as q
    c = _case(dev, M, N, K, True, seed=M + K)
    assert q.qmv_workspace_bytes(M, N, K, 64, 4, True) == 0
    y1 = _call(q, c, True)
    y2 = _call(q, c, True, torch.empty(0, dtype=torch.uint8, device=dev))
    np.testing.assert_array_equal(y1.view(np.uint32), y2.view(np.uint32))
    check_t2(y1, c["ref"], "f32")
