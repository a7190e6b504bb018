// Device quantizer/packer and the code-unpacking debug kernel.
#pragma once

#include <float.h>

#include "qmv_device.h"

namespace qmvk {

// Quantize and pack (mlx-cpu 0.30.1 quantized.h, affine_quantize).
//
// A group of g consecutive values is spread over g/4 adjacent lanes, four
// values per lane, as the page's quantizer spreads a group over a SIMD
// group: one 16-byte load per lane, and since groups are consecutive in
// memory (row-major W, K a multiple of g) a wave's loads are one contiguous
// 1 KB run.  w_min and w_max are reduced across the group's lanes (min and
// max are exact, so the reduction order cannot change them; the sign of a
// zero minimum or maximum never reaches the scale, bias or codes), every
// lane then runs the page's scale and bias steps, and each lane quantizes
// its four values.  Every step is one IEEE fp32 operation: the library is
// built without FMA contraction and with correctly rounded division, and
// roundf rounds half away from zero, so codes and bf16 scale/bias bits are
// fully determined by the input.  A lane's four codes form one 4b-bit field
// at bit 4b*u of its group's bit stream; the fields are OR-ed into the
// workgroup's words in LDS (at most two words per lane; OR is order
// independent) and the words are then written out contiguously.
// (One thread per group, reading its group straight from memory: 1.74 ms for
// a 14336x4096 pack on MI355X; one thread per group staged through LDS:
// 126 us.)
constexpr int kPackThreads = 256;

template <int G>
struct PackShape {
  static constexpr int LPG = G / 4;                  // lanes per group
  static constexpr int GPB = kPackThreads / LPG;     // groups per workgroup
  static constexpr int MAX_WORDS = GPB * G * 8 / 32; // LDS words for 8-bit codes
};

template <int LPG>
__device__ __forceinline__ float group_reduce(float v, bool is_min) {
#pragma unroll
  for (int off = 1; off < LPG; off <<= 1) {
    const float o = __shfl_xor(v, off, 64);
    v = is_min ? (o < v ? o : v) : (o > v ? o : v);
  }
  return v;
}

template <int G>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const float *__restrict__ w, int64_t ngroups,
                                                            int bits, uint32_t *__restrict__ w_q,
                                                            uint16_t *__restrict__ scales,
                                                            uint16_t *__restrict__ biases) {
  using S = PackShape<G>;
  __shared__ uint32_t words[S::MAX_WORDS];
  const int wpg = G * bits / 32;                     // words per group
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * S::GPB;
  const int gl = threadIdx.x / S::LPG, u = threadIdx.x % S::LPG;
  const int64_t gi = g0 + gl;
  const bool live = gi < ngroups;

  for (int i = threadIdx.x; i < S::GPB * wpg; i += kPackThreads) words[i] = 0u;

  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
  if (live) v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(w + gi * G) + u);   // read once

  float w_min = FLT_MAX;
  float w_max = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w_min = v[e] < w_min ? v[e] : w_min;
    w_max = v[e] > w_max ? v[e] : w_max;
  }
  w_min = group_reduce<S::LPG>(w_min, true);
  w_max = group_reduce<S::LPG>(w_max, false);

  const float n_bins = static_cast<float>((1 << bits) - 1);
  const float eps = 1e-7f;
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
  if (live && u == 0) {
    scales[gi] = f32_to_bf16(scale);
    biases[gi] = f32_to_bf16(bias);
  }

  uint32_t field = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float r = roundf((v[e] - bias) / scale);
    r = r > n_bins ? n_bins : r;
    field |= static_cast<uint32_t>(static_cast<int>(r)) << (bits * e);
  }
  __syncthreads();   // words cleared
  if (live) {
    const int bit = 4 * bits * u;                    // the field's offset in the group's stream
    const int wj = gl * wpg + (bit >> 5), sh = bit & 31;
    atomicOr(&words[wj], field << sh);
    if (sh + 4 * bits > 32) atomicOr(&words[wj + 1], field >> (32 - sh));
  }
  __syncthreads();
  const int64_t nwords = min(static_cast<int64_t>(S::GPB), ngroups - g0) * wpg;
  uint32_t *dst = w_q + g0 * wpg;
  for (int i = threadIdx.x; i < nwords; i += kPackThreads) dst[i] = words[i];
}

// ----------------------------------------------------------------------------
// Dequantize (mlx-metal quantized.h, affine_dequantize): w_hat = s*q + z per
// group with the stored bf16 scale and bias.  s*q is exact in fp32 (8-bit by
// 8-bit significands).  The sum with z is split into its fp32 rounding and
// its exact error (Knuth's TwoSum; the library is built without contraction),
// so both outputs are the exact value rounded once: fp32 to nearest even, and
// bf16 to nearest even.
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint16_t bf16_of_sum(float hi, float lo) {
  const uint32_t u = __float_as_uint(hi);
  // hi is the exact sum rounded to fp32.  Only when hi sits exactly halfway
  // between two bf16 values can the exact sum round differently from hi, and
  // then the sign of the error decides (truncating the bits rounds the
  // magnitude down).
  if ((u & 0xFFFFu) == 0x8000u && lo != 0.0f) {
    const bool away = (lo > 0.0f) == (hi > 0.0f);
    return static_cast<uint16_t>((u >> 16) + (away ? 1u : 0u));
  }
  return f32_to_bf16(hi);
}

// Each thread writes U units of 16 output bytes (8 bf16 or 4 fp32 values),
// units t, t + T, t + 2T, ... for T threads in all, so that consecutive
// threads write consecutive bytes and every store instruction writes one
// contiguous run; all of a thread's loads are issued before its first
// store.  A unit's E codes are E*b consecutive bits of its chunk (at most
// 64, inside two consecutive words), read straight from memory: the 4 or 8
// units of a chunk share its words through the cache.  The output is
// written with non-temporal stores: it is never read back by this kernel,
// and streaming it past the cache measured 38.5 -> 35.5 us for 14336x4096
// 4-bit -> bf16 (with 2 units per thread; 1 unit 46 us, 4 units 36.3 us).
#ifndef QMV_DEQUANT_UNITS
#define QMV_DEQUANT_UNITS 2
#endif
constexpr int kDequantUnits = QMV_DEQUANT_UNITS;

template <int BITS, bool F32>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t *__restrict__ w_q,
                                                      const uint16_t *__restrict__ scales,
                                                      const uint16_t *__restrict__ biases,
                                                      int64_t N, int64_t K, int gshift,
                                                      void *__restrict__ out) {
  constexpr int E = F32 ? 4 : 8;                  // values per unit
  constexpr int U = kDequantUnits;
  const int64_t Kc = K >> 5;
  const int64_t units = N * (K / E);
  const int64_t T = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t lo[U], hi[U];
  uint16_t sb[U], bb[U];
  int sh[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    int64_t t = t0 + i * T;
    t = t < units ? t : units - 1;                // past the end: recomputes the last unit
    const int64_t chunk = t / (32 / E);           // flat chunk index n*Kc + c
    const int j = static_cast<int>(t - chunk * (32 / E)) * E;   // first code of the unit
    const int64_t n = chunk / Kc, c = chunk - n * Kc;
    const uint32_t *cw = w_q + chunk * BITS;
    const int bit0 = j * BITS, wi = bit0 >> 5;
    sh[i] = bit0 & 31;
    lo[i] = cw[wi];
    hi[i] = (sh[i] + E * BITS > 32) ? cw[wi + 1] : 0u;   // only when the codes straddle
    const int64_t gi = n * (Kc >> gshift) + (c >> gshift);
    sb[i] = scales[gi];
    bb[i] = biases[gi];
  }
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int64_t t = t0 + i * T;
    if (t >= units) break;
    const uint64_t v = ((static_cast<uint64_t>(hi[i]) << 32) | lo[i]) >> sh[i];
    const float sf = bf16_to_f32(sb[i]);
    const float zf = bf16_to_f32(bb[i]);
    float h[E], l[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t q = static_cast<uint32_t>(v >> (e * BITS)) & ((1u << BITS) - 1u);
      const float p = sf * static_cast<float>(q);   // exact
      const float sum = p + zf;
      const float b2 = sum - p;
      h[e] = sum;
      l[e] = (p - (sum - b2)) + (zf - b2);
    }
    if constexpr (F32) {
      typedef float f32x4v __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(f32x4v{h[0], h[1], h[2], h[3]}, reinterpret_cast<f32x4v *>(out) + t);
    } else {
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = static_cast<uint32_t>(bf16_of_sum(h[2 * k], l[2 * k])) |
               (static_cast<uint32_t>(bf16_of_sum(h[2 * k + 1], l[2 * k + 1])) << 16);
      typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(u32x4v{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4v *>(out) + t);
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
      pair_codes<BITS, I>(make_pair<BITS, I>(w, pk), lo, hi);
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
