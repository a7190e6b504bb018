"""qmv_noalloc (the entry point for callers that cannot allocate) against
qmv_with_workspace, through the C ABI: the same kernels, so the outputs must
be bit-identical.  Two calls in a row share the static scratch array, the
second with a smaller input; both split-K paths (transpose = 0 and the
matrix-core path for 5 or more rows of x) and a call that needs no
workspace."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests.parity import bf16_to_np_bits, check_t2, to_dev_bf16, to_dev_u32

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _case(dev, M, N, K, transpose, seed, g=64, bits=4):
    shape = (N, K) if transpose else (K, N)
    w_q, s, b = oracle.quantize_pack(synth.weight(shape, seed), g, bits)
    x = synth.activation_bf16((M, K), seed + 50)
    ref = oracle.qmv(x, w_q, s, b, g, bits) if transpose else oracle.qvm(x, w_q, s, b, N, g, bits)
    return dict(M=M, N=N, K=K, transpose=transpose, g=g, bits=bits, ref=ref,
                x=to_dev_bf16(x, dev), w=to_dev_u32(w_q, dev), s=to_dev_bf16(s, dev),
                b=to_dev_bf16(b, dev))


def _run(q, c, entry, out_f32, workspace=None):
    import torch
    y = torch.empty((c["M"], c["N"]), dtype=torch.float32 if out_f32 else torch.bfloat16,
                    device=c["x"].device)
    args = [_ptr(c["x"]), _ptr(c["w"]), _ptr(c["s"]), _ptr(c["b"]), _ptr(y), c["M"], c["N"],
            c["K"], c["g"], c["bits"], 1 if c["transpose"] else 0, 1 if out_f32 else 0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L = q.lib()
    if entry == "noalloc":
        rc = L.qmv_noalloc(*args, stream)
    else:
        rc = L.qmv_with_workspace(*args, _ptr(workspace), workspace.numel(), stream)
    assert rc == 0, L.qmv_last_error()
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("transpose", (True, False))
@pytest.mark.parametrize("out_f32", (False, True))
def test_noalloc_matches_with_workspace_two_calls(dev, transpose, out_f32):
    import torch

    import bit_affine_quantized_amd as q
    big = _case(dev, 64 if transpose else 4, 4096, 4096, transpose, 31)
    small = _case(dev, 8 if transpose else 2, 1024, 1024 if transpose else 2048, transpose, 32)
    assert q.qmv_workspace_bytes(big["M"], big["N"], big["K"], 64, 4, transpose) > \
        q.qmv_workspace_bytes(small["M"], small["N"], small["K"], 64, 4, transpose) > 0
    for c in (big, small):
        nb = q.qmv_workspace_bytes(c["M"], c["N"], c["K"], 64, 4, transpose)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        y_ws = _run(q, c, "with_workspace", out_f32, ws)
        y_na = _run(q, c, "noalloc", out_f32)
        if out_f32:
            np.testing.assert_array_equal(y_na.cpu().numpy(), y_ws.cpu().numpy())
            check_t2(y_na.cpu().numpy(), c["ref"], "noalloc")
        else:
            np.testing.assert_array_equal(bf16_to_np_bits(y_na), bf16_to_np_bits(y_ws))


def test_noalloc_without_split_k(dev):
    """One row of x with transpose = 1 needs no workspace: qmv_noalloc runs
    the matvec kernel and equals qmv_with_workspace with none."""
    import torch

    import bit_affine_quantized_amd as q
    c = _case(dev, 1, 2048, 4096, True, 33)
    assert q.qmv_workspace_bytes(1, 2048, 4096, 64, 4, True) == 0
    y_na = _run(q, c, "noalloc", True)
    L = q.lib()
    y = torch.empty((1, 2048), dtype=torch.float32, device=dev)
    rc = L.qmv_with_workspace(_ptr(c["x"]), _ptr(c["w"]), _ptr(c["s"]), _ptr(c["b"]), _ptr(y), 1, 2048,
                              4096, 64, 4, 1, 1, None, 0,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y_na.cpu().numpy(), y.cpu().numpy())
