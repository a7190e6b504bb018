"""The oracle (and on a GPU the device quantizer and matvec) against the
hand-derived fixtures in tests/golden/: values that follow from the pages'
quantizer and pack definitions by hand arithmetic, not from any code here."""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, vals = line.split(":", 1)
            out[key.strip()] = [int(v, 0) if not any(c in v for c in ".e") or v.startswith("0x")
                                else float(v) for v in vals.split()]
    return out


def lattice_weights(f):
    return (np.array(f["j"], np.float32) * np.float32(f["weight_scale"][0]))[None, :]


def test_lattice_group_quantize_and_pack():
    f = load("quantize_lattice_4bit_g32.txt")
    w = lattice_weights(f)
    codes, _, _, s16, b16 = oracle.quantize(w, f["group_size"][0], f["bits"][0])
    assert codes[0].tolist() == f["codes"]
    assert int(s16[0, 0]) == f["scale_bits"][0] and int(b16[0, 0]) == f["bias_bits"][0]
    w_q = oracle.pack(codes, f["bits"][0])
    assert [int(v) for v in w_q[0]] == f["words"]


def test_lattice_group_qmv():
    f = load("quantize_lattice_4bit_g32.txt")
    w_q, s16, b16 = oracle.quantize_pack(lattice_weights(f), f["group_size"][0], f["bits"][0])
    x = synth.f32_to_bf16_bits(np.array(f["x"], np.float32))[None, :]
    y = oracle.qmv(x, w_q, s16, b16, f["group_size"][0], f["bits"][0])
    assert float(y[0, 0]) == f["y"][0]
    assert int(synth.f32_to_bf16_bits(np.array([y[0, 0]], np.float32))[0]) == f["y_bits"][0]


def test_zero_group():
    f = load("quantize_zero_group.txt")
    w = np.zeros((1, f["group_size"][0]), np.float32)
    codes, _, _, s16, b16 = oracle.quantize(w, f["group_size"][0], f["bits"][0])
    assert codes[0].tolist() == f["codes"]
    assert int(s16[0, 0]) == f["scale_bits"][0] and int(b16[0, 0]) == f["bias_bits"][0]
    assert [int(v) for v in oracle.pack(codes, f["bits"][0])[0]] == f["words"]


def test_pack_3bit():
    f = load("pack_3bit_codes_0_to_7.txt")
    w_q = oracle.pack(np.array(f["codes"], np.uint8)[None, :], f["bits"][0])
    assert w_q.view(np.uint8).ravel().tolist() == f["bytes"]


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["quantize_lattice_4bit_g32.txt", "quantize_zero_group.txt"])
def test_device_quantizer_and_qmv(name):
    """qmv_pack and qmv on the GPU reproduce the hand-derived bits."""
    import torch

    import bit_affine_quantized_amd as q
    f = load(name)
    g, bits = f["group_size"][0], f["bits"][0]
    w = lattice_weights(f) if "j" in f else np.zeros((1, g), np.float32)
    w_q, s, b = q.qmv_pack(torch.from_numpy(w).cuda(), g, bits)
    assert [int(v) for v in w_q.cpu().numpy().view(np.uint32)[0]] == f["words"]
    assert int(s.cpu().view(torch.int16).numpy().view(np.uint16)[0, 0]) == f["scale_bits"][0]
    assert int(b.cpu().view(torch.int16).numpy().view(np.uint16)[0, 0]) == f["bias_bits"][0]
    if "x" in f:
        xb = synth.f32_to_bf16_bits(np.array(f["x"], np.float32))[None, :]
        x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        y = q.qmv(x, w_q, s, b, group_size=g, bits=bits)
        assert int(y.cpu().view(torch.int16).numpy().view(np.uint16)[0, 0]) == f["y_bits"][0]
