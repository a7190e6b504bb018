// Device quantizer/packer and the code-unpacking debug kernel.
#pragma once

#include <float.h>

#include "qmv_device.h"

namespace qmvk {

// One thread per group of g consecutive K-elements (mlx-cpu 0.30.1
// quantized.h, affine_quantize).  Every step is one IEEE fp32 operation:
// the library is built without FMA contraction and with correctly rounded
// division, and roundf rounds half away from zero, so the codes and the bf16
// scale/bias bits are fully determined by the input.
__global__ __launch_bounds__(256) void pack_kernel(const float *__restrict__ w, int64_t N, int64_t K,
                                                   int g, int bits, uint32_t *__restrict__ w_q,
                                                   uint16_t *__restrict__ scales,
                                                   uint16_t *__restrict__ biases) {
  const int64_t groups = K / g;
  const int64_t gi = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gi >= N * groups) return;
  const int64_t n = gi / groups;
  const int64_t j = gi - n * groups;
  const float *src = w + n * K + j * g;

  const float n_bins = static_cast<float>((1 << bits) - 1);
  const float eps = 1e-7f;
  float w_min = FLT_MAX;
  float w_max = 0.0f;
  for (int i = 0; i < g; ++i) {
    const float v = src[i];
    w_min = v < w_min ? v : w_min;
    w_max = v > w_max ? v : w_max;
  }
  float scale = (w_max - w_min) / n_bins;
  scale = scale < eps ? eps : scale;
  const bool side = fabsf(w_min) > fabsf(w_max);
  scale = side ? scale : -scale;
  const float edge = side ? w_min : w_max;
  const float q0 = roundf(edge / scale);
  float bias = 0.0f;
  if (q0 != 0.0f) {
    scale = edge / q0;
    bias = edge;
  }
  scales[gi] = f32_to_bf16(scale);
  biases[gi] = f32_to_bf16(bias);

  // The group's codes fill g*bits/32 whole words of the row's bit stream.
  uint32_t *dst = w_q + n * (K * bits / 32) + j * (static_cast<int64_t>(g) * bits / 32);
  uint64_t acc = 0;
  int nacc = 0;
  int wi = 0;
  for (int i = 0; i < g; ++i) {
    float r = roundf((src[i] - bias) / scale);
    r = r > n_bins ? n_bins : r;
    const uint32_t q = static_cast<uint32_t>(static_cast<int>(r));
    acc |= static_cast<uint64_t>(q) << nacc;
    nacc += bits;
    if (nacc >= 32) {
      dst[wi++] = static_cast<uint32_t>(acc);
      acc >>= 32;
      nacc -= 32;
    }
  }
}

// Debug export: unpack with the qmv kernels' own pair / fp32 code builders.
template <int BITS>
__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t *__restrict__ w_q, int64_t N,
                                                     int64_t K, uint8_t *__restrict__ codes) {
  const int64_t Kc = K >> 5;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= N * Kc) return;
  const int64_t n = t / Kc, c = t - n * Kc;
  uint32_t w[BITS];
  load_chunk<BITS>(w_q + n * Kc * BITS + c * BITS, w);
  uint8_t *out = codes + n * K + c * 32;
  if constexpr (BITS <= 6) {
    const PairConsts pk = pair_consts<BITS>();
    static_for<0, 16>([&](auto i) {
      constexpr int I = decltype(i)::value;
      uint32_t lo, hi;
      pair_codes<BITS>(make_pair<BITS, I>(w, pk), lo, hi);
      out[PairPlan<BITS>::lo(I)] = static_cast<uint8_t>(lo);
      out[PairPlan<BITS>::hi(I)] = static_cast<uint8_t>(hi);
    });
  } else {
    static_for<0, 32>([&](auto k) {
      constexpr int Kk = decltype(k)::value;
      out[Kk] = static_cast<uint8_t>(code_f32<BITS, Kk>(w));
    });
  }
}

}  // namespace qmvk
