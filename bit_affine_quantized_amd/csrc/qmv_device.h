// Device building blocks for the gfx950 quantized matvec kernels.
//
// The packed row layout is a little-endian bit stream: code k of a row sits
// at stream bits [b*k, b*k + b) (mlx-cpu 0.30.1 quantized.h, affine_quantize
// and affine_dequantize).  The kernels work on "chunks" of 32 consecutive
// codes of one row: a chunk is exactly `b` uint32 words, starts on a word
// boundary, and never crosses a group (group sizes are multiples of 32).
//
// Two inner products are used:
//
//  * bf16 pair path (b <= 6).  Each code q is written into the top b bits of
//    the 7-bit mantissa of a bf16 whose exponent is fixed at 2^7:
//        value = 128 + q * 2^P,   P = 7 - b   (exact, 128 + q*2^P <= 255)
//    Two such values share a dword and meet a dword of two x values that were
//    staged pre-multiplied by 2^-P, so one v_dot2c_f32_bf16 adds
//        (2^b + q_lo) * x_lo + (2^b + q_hi) * x_hi
//    into an fp32 accumulator.  Over a chunk that is D = sum(q*x) + 2^b*sum(x),
//    and the affine fold s*sum(q*x) + z*sum(x) (quantized.h, qdot) becomes
//        s*D + (z - 2^b*s) * sum(x).
//    The offset 2^b is at most ~2x the mean code, so the cancellation costs
//    about one bit of the fp32 accumulator.
//
//  * fp32 path (b = 8, and the fused silu tail whose input is not bf16): each
//    code is converted to fp32 (v_cvt_f32_ubyteN for bytes) and FMA'd with an
//    fp32 x; fold s*D + z*sum(x).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace qmvk {

// Build-time tuning knobs (defaults are the measured best on MI355X).
#ifndef QMV_WAVES_PER_BLOCK
#define QMV_WAVES_PER_BLOCK 4
#endif
#ifndef QMV_NT_LOADS
#define QMV_NT_LOADS 0
#endif

constexpr int kWave = 64;
constexpr int kWavesPerBlock = QMV_WAVES_PER_BLOCK;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr uint32_t kMagic2 = 0x43004300u;   // two bf16 values of 128.0

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Shift left for positive amounts, right for negative (compile-time amount).
template <int SH>
__device__ __forceinline__ uint32_t shl_signed(uint32_t v) {
  if constexpr (SH >= 0) return v << SH;
  else return v >> (-SH);
}

// Code k (0..31) of a chunk held in BITS words, right-aligned.
template <int BITS, int K>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[BITS]) {
  constexpr int bit = K * BITS;
  constexpr int wd = bit >> 5;
  constexpr int off = bit & 31;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  if constexpr (off + BITS <= 32) {
    return (w[wd] >> off) & mask;
  } else {
    return __builtin_amdgcn_alignbit(w[wd + 1], w[wd], off) & mask;
  }
}

// ----------------------------------------------------------------------------
// Pair plans: which two codes of a chunk share bf16 pair i (i = 0..15).  The
// x staging uses the same plan, so any pairing is valid; the plans below are
// chosen so that for b = 2 and 4 one shift and one and-or build each pair
// (the two codes sit exactly 16 bits apart in one word).
// ----------------------------------------------------------------------------
template <int BITS>
struct PairPlan {
  static constexpr int P = 7 - BITS;   // mantissa position of the code
  // code index of the low / high half of pair i
  static constexpr __host__ __device__ int lo(int i) {
    return BITS == 4 ? 8 * (i >> 2) + (i & 3)
         : BITS == 2 ? 16 * (i >> 3) + (i & 7)
         : i;
  }
  static constexpr __host__ __device__ int hi(int i) {
    return BITS == 4 ? lo(i) + 4 : BITS == 2 ? lo(i) + 8 : i + 16;
  }
};

template <int BITS, int I>
__device__ __forceinline__ uint32_t make_pair(const uint32_t (&w)[BITS]) {
  constexpr int P = PairPlan<BITS>::P;
  if constexpr (BITS == 4) {
    constexpr int d = I >> 2, j = I & 3;
    // code j at bit 4j -> bit 3; code j+4 at bit 4j+16 -> bit 19
    return (shl_signed<3 - 4 * j>(w[d]) & 0x00780078u) | kMagic2;
  } else if constexpr (BITS == 2) {
    constexpr int d = I >> 3, j = I & 7;
    // code j at bit 2j -> bit 5; code j+8 at bit 2j+16 -> bit 21
    return (shl_signed<5 - 2 * j>(w[d]) & 0x00600060u) | kMagic2;
  } else {
    constexpr int klo = PairPlan<BITS>::lo(I), khi = PairPlan<BITS>::hi(I);
    return (code_at<BITS, klo>(w) << P) | (code_at<BITS, khi>(w) << (16 + P)) | kMagic2;
  }
}

// Recover code index / value of both halves from a built pair (debug export).
template <int BITS>
__device__ __forceinline__ void pair_codes(uint32_t p, uint32_t &lo, uint32_t &hi) {
  constexpr int P = PairPlan<BITS>::P;
  lo = (p & 0x7Fu) >> P;
  hi = ((p >> 16) & 0x7Fu) >> P;
}

// Code k of a chunk as fp32 (fp32 path).  Bytes use v_cvt_f32_ubyteN.
template <int BITS, int K>
__device__ __forceinline__ float code_f32(const uint32_t (&w)[BITS]) {
  if constexpr (BITS == 8) {
    return static_cast<float>((w[K >> 2] >> (8 * (K & 3))) & 0xFFu);
  } else {
    return static_cast<float>(code_at<BITS, K>(w));
  }
}

// ----------------------------------------------------------------------------
// Chunk loads: BITS consecutive dwords at a dword-aligned address; the chunk
// offset c*BITS keeps 8-byte alignment for b = 2, 16 for b = 4 and 32 for 8.
// ----------------------------------------------------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Weight words are read exactly once per call: optionally mark them
// non-temporal so they do not displace x, scales and biases in the caches.
template <typename T>
__device__ __forceinline__ T stream_load(const T *p) {
#if QMV_NT_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

template <int BITS>
__device__ __forceinline__ void load_chunk(const uint32_t *__restrict__ p, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4) {
    const u32x4_t v = stream_load(reinterpret_cast<const u32x4_t *>(p));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 8) {
    const u32x4_t v0 = stream_load(reinterpret_cast<const u32x4_t *>(p));
    const u32x4_t v1 = stream_load(reinterpret_cast<const u32x4_t *>(p) + 1);
    w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
    w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
  } else if constexpr (BITS == 2) {
    const u32x2_t v = stream_load(reinterpret_cast<const u32x2_t *>(p));
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int d = 0; d < BITS; ++d) w[d] = stream_load(p + d);
  }
}

// ----------------------------------------------------------------------------
// Wave reduction of V values per lane (V a power of two, V <= 64).  A
// butterfly that halves the value count at each step: lanes in the upper
// half of each xor pair keep the upper half of the values.  Every value is
// summed over the same lane tree (pairs by lane bit 5, then 4, ...), so the
// result for a value does not depend on its index.  On return lane l holds
// the total of value index reduce_index<V>(l); all lanes of a group agree.
// ----------------------------------------------------------------------------
template <int V>
__device__ __forceinline__ float wave_reduce_many(float (&v)[V], int lane) {
  static_assert((V & (V - 1)) == 0 && V >= 1 && V <= 64, "V must be a power of two");
  constexpr int LOGV = (V >= 64) ? 6 : (V >= 32) ? 5 : (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : (V >= 2) ? 1 : 0;
  float cur[V];
#pragma unroll
  for (int i = 0; i < V; ++i) cur[i] = v[i];
  static_for<0, LOGV>([&](auto t) {
    constexpr int step = decltype(t)::value;
    constexpr int half = V >> (step + 1);
    constexpr int off = 32 >> step;
    const bool upper = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      float keep = upper ? cur[half + i] : cur[i];
      float send = upper ? cur[i] : cur[half + i];
      float recv = __shfl_xor(send, off, kWave);
      cur[i] = keep + recv;
    }
  });
  float r = cur[0];
#pragma unroll
  for (int off = 32 >> LOGV; off >= 1; off >>= 1) r += __shfl_xor(r, off, kWave);
  return r;
}

template <int V>
__device__ __forceinline__ int reduce_index(int lane) {
  int idx = 0;
  int h = V;
#pragma unroll
  for (int step = 0; (V >> step) > 1; ++step) {
    h >>= 1;
    if (lane & (32 >> step)) idx += h;
  }
  return idx;
}

template <int V>
__device__ __forceinline__ bool reduce_leader(int lane) {
  // the lowest lane of each group of lanes that share a value index
  constexpr int LOGV = (V >= 64) ? 6 : (V >= 32) ? 5 : (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : (V >= 2) ? 1 : 0;
  constexpr int low_mask = (1 << (6 - LOGV)) - 1;
  return (lane & low_mask) == 0;
}

constexpr int pow2_ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace qmvk
