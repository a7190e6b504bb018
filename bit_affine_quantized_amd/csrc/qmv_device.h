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
//        v = 128 + q * 2^P,   P = 7 - b   (exact: v <= 255)
//    Two such values share a dword and meet a dword holding the two matching
//    raw bf16 x values, so one v_dot2c_f32_bf16 adds v_lo*x_lo + v_hi*x_hi
//    into an fp32 accumulator.  Over a chunk that is
//        D = 128*sum(x) + 2^P * sum(q*x),
//    and the affine fold s*sum(q*x) + z*sum(x) (quantized.h, qdot) becomes
//        2^-P * s*D + (z - 2^b*s) * sum(x)        (2^b = 128 * 2^-P).
//    The offset 2^b is about twice the mean code, so the cancellation costs
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
#ifndef QMV_NT_LOADS
#define QMV_NT_LOADS 1
#endif

constexpr int kWave = 64;
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

// Pair building is (w >> sh) & mask | magic.  With both constants as 32-bit
// literals the compiler must split it into v_and_b32 + v_or_b32 (a VOP3
// encoding holds no literal on gfx9); with the mask in an SGPR and the magic
// in a VGPR it selects one v_and_or_b32.  These empty asm statements, run
// once per kernel, hide the values so they stay in registers.
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

struct PairConsts {
  uint32_t mask;    // SGPR
  uint32_t magic;   // VGPR
};

template <int BITS>
__device__ __forceinline__ PairConsts pair_consts() {
  // the code bits of both halves of a pair built by shift/window + and-or
  const uint32_t m = BITS == 4 ? 0x00780078u : BITS == 2 ? 0x00600060u
                   : BITS == 3 ? 0x00380070u : BITS == 5 ? 0x003E007Cu
                   : BITS == 6 ? 0x007E007Eu : 0u;
  return PairConsts{opaque_sgpr(m), opaque_vgpr(kMagic2)};
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
// x staging uses the same plan, so any pairing is valid.  The plans are
// chosen so that one shift (or one alignbit window) and one and-or build a
// pair:
//  * b = 2, 4: the two codes sit exactly 16 bits apart in one word.
//  * b = 3, 5: no two codes are 16 bits apart, but codes k and k + 5 (3-bit)
//    or k + 3 (5-bit) are 15 bits apart.  One 32-bit window of the stream
//    puts code k at mantissa bit P and its partner one bit lower in the high
//    half, at P - 1: that half holds 128 + q * 2^(P-1).  Its x is staged
//    doubled (exact in bf16), so the product is (256 + q * 2^P) * x: the same
//    q * 2^P * x as the low half, and 256 x in place of 128 x.  Each chunk
//    then carries two sums, X = sum x and X' = sum of the staged x values (x
//    of the low halves plus 2x of the doubled high halves), and the fold is
//        2^-P * s*D + z*X - 2^b * s*X'.
//    15 pairs are built this way; codes 30 and 31 form a plain pair (both
//    halves at P, x not doubled).
//  * b = 6: code k = 4m + r lies in byte group m (bytes 3m..3m+2) at bits
//    6r..6r+5 of the group, in one byte (r = 0, 3) or two (r = 1, 2).  A pair
//    joins the same r of two groups: one v_perm_b32 gathers the code's
//    byte(s) of each group into its half, one shift moves both codes to
//    mantissa bit 1 (P = 1), and one and-or finishes.  The group pairs of
//    each r are chosen so that the four bytes lie in at most two words.
// ----------------------------------------------------------------------------
struct SixBitPlan {
  // group pairs (m, m') of pair j of class r
  static constexpr int kGroups[4][4][2] = {{{0, 1}, {2, 3}, {4, 5}, {6, 7}},
                                           {{1, 0}, {5, 4}, {2, 3}, {6, 7}},
                                           {{2, 1}, {6, 5}, {0, 3}, {4, 7}},
                                           {{0, 1}, {2, 3}, {4, 5}, {6, 7}}};
  static constexpr int kByte0[4] = {0, 0, 1, 2};    // first byte of the code in its group
  static constexpr int kByte1[4] = {-1, 1, 2, -1};  // second byte, if any
  static constexpr int kShift[4] = {-1, 5, 3, 1};   // right shift to bit 1 (-1: left by 1)
  // chunk byte at position pos (0, 1: low half; 2, 3: high half) of pair i, or -1
  static constexpr int byte_of(int i, int pos) {
    const int r = i >> 2, j = i & 3;
    const int m = kGroups[r][j][pos >> 1];
    const int b = (pos & 1) ? kByte1[r] : kByte0[r];
    return b < 0 ? -1 : 3 * m + b;
  }
  static constexpr int word_a(int i) {   // lower source word
    int d = 1 << 20;
    for (int pos = 0; pos < 4; ++pos)
      if (byte_of(i, pos) >= 0 && (byte_of(i, pos) >> 2) < d) d = byte_of(i, pos) >> 2;
    return d;
  }
  static constexpr int word_b(int i) {   // upper source word
    int d = -1;
    for (int pos = 0; pos < 4; ++pos)
      if (byte_of(i, pos) >= 0 && (byte_of(i, pos) >> 2) > d) d = byte_of(i, pos) >> 2;
    return d;
  }
  // v_perm_b32 selector: 0-3 pick word_a's bytes, 4-7 word_b's, 0x0C a zero
  static constexpr uint32_t selector(int i) {
    uint32_t sel = 0;
    for (int pos = 0; pos < 4; ++pos) {
      const int b = byte_of(i, pos);
      const uint32_t v = b < 0 ? 0x0Cu : (b >> 2) == word_a(i) ? static_cast<uint32_t>(b & 3)
                                                                : 4u + static_cast<uint32_t>(b & 3);
      sel |= v << (8 * pos);
    }
    return sel;
  }
};

template <int BITS>
struct PairPlan {
  static constexpr int P = 7 - BITS;   // mantissa position of the (low) code
  static constexpr bool kWindow = BITS == 3 || BITS == 5;   // 15-bit-apart pairs
  static constexpr int kGap = BITS == 3 ? 5 : 3;             // partner distance (codes)
  static constexpr int kBlock = 2 * kGap;                   // codes per block of pairs
  // code index of the low / high half of pair i
  static constexpr __host__ __device__ int lo(int i) {
    return BITS == 4 ? 8 * (i >> 2) + (i & 3)
         : BITS == 2 ? 16 * (i >> 3) + (i & 7)
         : kWindow ? (i < 15 ? kBlock * (i / kGap) + i % kGap : 30)
         : BITS == 6 ? 4 * SixBitPlan::kGroups[i >> 2][i & 3][0] + (i >> 2)
         : i;
  }
  static constexpr __host__ __device__ int hi(int i) {
    return BITS == 4 ? lo(i) + 4 : BITS == 2 ? lo(i) + 8
         : kWindow ? (i < 15 ? lo(i) + kGap : 31)
         : BITS == 6 ? 4 * SixBitPlan::kGroups[i >> 2][i & 3][1] + (i >> 2)
         : i + 16;
  }
  // the high half of pair i holds its code at P - 1 and meets doubled x
  static constexpr __host__ __device__ bool doubled(int i) { return kWindow && i < 15; }
};

// whether a chunk's staging carries the second sum X' (see PairPlan)
template <int BITS>
constexpr bool two_sums() { return PairPlan<BITS>::kWindow; }

template <int BITS, int I>
__device__ __forceinline__ uint32_t make_pair(const uint32_t (&w)[BITS], PairConsts k) {
  constexpr int P = PairPlan<BITS>::P;
  if constexpr (BITS == 4) {
    constexpr int d = I >> 2, j = I & 3;
    // code j at bit 4j -> bit 3; code j+4 at bit 4j+16 -> bit 19
    return (shl_signed<3 - 4 * j>(w[d]) & k.mask) | k.magic;
  } else if constexpr (BITS == 2) {
    constexpr int d = I >> 3, j = I & 7;
    // code j at bit 2j -> bit 5; code j+8 at bit 2j+16 -> bit 21
    return (shl_signed<5 - 2 * j>(w[d]) & k.mask) | k.magic;
  } else if constexpr (BITS == 6) {
    constexpr uint32_t sel = SixBitPlan::selector(I);
    constexpr int sh = SixBitPlan::kShift[I >> 2];
    const uint32_t v = __builtin_amdgcn_perm(w[SixBitPlan::word_b(I)], w[SixBitPlan::word_a(I)], sel);
    return (shl_signed<-sh>(v) & k.mask) | k.magic;
  } else if constexpr (PairPlan<BITS>::doubled(I)) {
    // the 22-bit window whose bit P is code lo's first bit: code hi then
    // sits at bit 16 + P - 1
    constexpr int s = BITS * PairPlan<BITS>::lo(I) - P;   // stream bit at window bit 0
    uint32_t win;
    if constexpr (s < 0) {
      win = w[0] << (-s);
    } else {
      constexpr int j = s >> 5, o = s & 31;
      if constexpr (o + 22 <= 32) win = w[j] >> o;
      else win = __builtin_amdgcn_alignbit(w[j + 1], w[j], o);
    }
    return (win & k.mask) | k.magic;
  } else {
    constexpr int klo = PairPlan<BITS>::lo(I), khi = PairPlan<BITS>::hi(I);
    return (code_at<BITS, klo>(w) << P) | (code_at<BITS, khi>(w) << (16 + P)) | k.magic;
  }
}

// Recover the codes of both halves of built pair I (debug export).
template <int BITS, int I>
__device__ __forceinline__ void pair_codes(uint32_t p, uint32_t &lo, uint32_t &hi) {
  constexpr int P = PairPlan<BITS>::P;
  constexpr int PH = PairPlan<BITS>::doubled(I) ? P - 1 : P;
  lo = (p & 0x7Fu) >> P;
  hi = ((p >> 16) & 0x7Fu) >> PH;
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

// base + a 32-bit byte offset: lets the compiler use the global_load
// "saddr + 32-bit voffset" form when the base is wave-uniform.
template <typename T>
__device__ __forceinline__ const T *byte_offset(const T *base, uint32_t bytes) {
  return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + bytes);
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

// The same chunk through a buffer resource: `off` is the chunk's byte offset
// from the resource base, held in the VGPR operand.  The hardware range
// check covers that operand: a chunk at or past the resource's byte count
// reads as zeros.  Dword 3 of a raw gfx9 resource: 32-bit data format, no
// swizzle, no index stride.
constexpr int kBufferDword3 = 0x00020000;
constexpr int kBufferNt = QMV_NT_LOADS ? 2 : 0;   // cache policy of the weight words

template <int BITS>
__device__ __forceinline__ void buffer_load_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4 || BITS == 8) {
#pragma unroll
    for (int h = 0; h < BITS / 4; ++h) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * h, 0, kBufferNt);
      w[4 * h] = v.x; w[4 * h + 1] = v.y; w[4 * h + 2] = v.z; w[4 * h + 3] = v.w;
    }
  } else if constexpr (BITS == 2) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kBufferNt);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int d = 0; d < BITS; ++d) w[d] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * d, 0, kBufferNt);
  }
}

// ----------------------------------------------------------------------------
// Wave reduction of V values per lane (V a power of two, V <= 64).  A
// transposing butterfly over lane bits 5, 4, 3, ...: at each step the lanes
// whose bit is set keep the upper half of the values, the others the lower
// half, so the value count halves; the remaining lane bits are then summed
// out.  Bits 5 and 4 use the gfx950 v_permlane32_swap / v_permlane16_swap
// (which exchange whole half-waves / rows, so no select is needed), bits 3..0
// use DPP moves fused into the adds.  Every value is summed over the same
// lane tree, so its result does not depend on its index.  On return lane l
// holds the total of value reduce_index<V>(l); all lanes of a group agree.
// ----------------------------------------------------------------------------
__device__ __forceinline__ void swap32(float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRor8 = 0x128;     // row_ror:8 == xor 8 within a 16-lane row

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
#pragma unroll
    for (int i = 0; i < half; ++i) {
      float a = cur[i], b = cur[half + i];
      if constexpr (off == 32) {
        swap32(a, b);
        cur[i] = a + b;
      } else if constexpr (off == 16) {
        swap16(a, b);
        cur[i] = a + b;
      } else {
        const bool upper = (lane & off) != 0;
        const float keep = upper ? b : a;
        const float send = upper ? a : b;
        float recv;
        if constexpr (off == 8) recv = dpp<kDppRor8>(send);
        else recv = __shfl_xor(send, off, kWave);
        cur[i] = keep + recv;
      }
    }
  });
  float r = cur[0];
  static_for<LOGV, 6>([&](auto t) {
    constexpr int off = 32 >> decltype(t)::value;
    if constexpr (off == 32) {
      float a = r, b = r;
      swap32(a, b);
      r = a + b;
    } else if constexpr (off == 16) {
      float a = r, b = r;
      swap16(a, b);
      r = a + b;
    } else if constexpr (off == 8) {
      r += dpp<kDppRor8>(r);
    } else if constexpr (off == 4) {
      r += dpp<kDppHalfMirror>(r);   // all 8 lanes of the group share the value
    } else if constexpr (off == 2) {
      r += dpp<kDppXor2>(r);
    } else {
      r += dpp<kDppXor1>(r);
    }
  });
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

// Workgroup b of a launch runs on XCD (b mod 8): the dispatcher deals
// workgroups to the eight XCDs in turn.  xcd_block maps the dispatch index
// to a logical block index such that XCD x owns one contiguous run of
// logical blocks (the x-th eighth, the first nb mod 8 XCDs one block more).
// Kernels that give consecutive logical blocks consecutive rows then have
// each XCD stream its own contiguous part of the weight, scales and output;
// on MI355X this measured 4-5% faster for the one-vector matvec than the
// dispatch order (whose neighbouring blocks sit on different XCDs).
__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t nb) {
  const int64_t x = b & 7, k = b >> 3;
  const int64_t q = nb >> 3, r = nb & 7;
  return x * q + (x < r ? x : r) + k;
}

constexpr int pow2_ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace qmvk
