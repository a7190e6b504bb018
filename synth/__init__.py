"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the quantized product: it only draws
numbers.  Both the CPU oracle and the HIP library receive the same input bits
from here (weights as fp32, activations as bf16 bits), never each other's
results.

Recipe (LLM-shaped decode workloads; the pages measure no dataset):
  * weights   W ~ N(0, 0.02^2): numpy PCG64 ``standard_normal(float32) * 0.02``
  * activations x ~ N(0, 1) drawn in fp32, narrowed to bf16 (nearest-even)
  * MoE routing: per token, ``choice(E, top_k, replace=False)``; lhs = token id
Seeds: W/gate 0, up 1, down 2, x 100, x_resid 101, indices 200.
"""
from __future__ import annotations

import numpy as np

SEED_W = 0
SEED_UP = 1
SEED_DOWN = 2
SEED_X = 100
SEED_XRESID = 101
SEED_IDX = 200


def weight(shape, seed: int = SEED_W) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Nearest-even narrowing of finite fp32 values to bf16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = u.astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32)


def activation_bf16(shape, seed: int = SEED_X) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def moe_indices(tokens: int, top_k: int, experts: int, seed: int = SEED_IDX):
    """-> lhs [tokens, top_k] (token id), rhs [tokens, top_k] uint32."""
    rng = np.random.default_rng(seed)
    rhs = np.stack([rng.choice(experts, top_k, replace=False)
                    for _ in range(tokens)]).astype(np.uint32)
    lhs = np.repeat(np.arange(tokens, dtype=np.uint32)[:, None], top_k, 1)
    return lhs, rhs


# The workloads (shapes from the decode configurations this library targets).
TINY = dict(name="tiny_qmv_256x512_b4_g64", N=256, K=512, bits=4, group=64,
            M=1)
DECODE = dict(name="decode_qmv_4096x4096_b4_g64", N=4096, K=4096, bits=4,
              group=64, M=(1, 4))
HEADLINE = dict(name="qmv_14336x4096_b4_g64_m1", N=14336, K=4096, bits=4,
                group=64, M=1)
SWEEP = dict(name="sweep_qmv_14336x4096", N=14336, K=4096,
             bits=(2, 3, 5, 6, 8), group=(32, 64, 128), M=1)
FFN = dict(name="ffn_gateup_14336x4096_down_4096x14336_b8_g64", N=14336,
           K=4096, bits=8, group=64)
MOE = dict(name="moe_gather_64x2048x2048_b4_g64_t16_top8", E=64, N=2048,
           K=2048, bits=4, group=64, tokens=16, top_k=8)
