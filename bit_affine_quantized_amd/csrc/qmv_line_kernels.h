// One-vector quantized matvec with a straight-line body (gfx950).
//
// Same work split and arithmetic as qmv_kernel (qmv_kernels.h) for one x
// vector: a workgroup of WPB waves owns RPW * WPB consecutive rows, lane l of
// a wave takes chunks l, l + 64, ... of each of its rows, and x is staged once
// per workgroup in LDS.  The difference is that the number of 64-lane chunk
// steps per row, CPL, is a compile-time constant, so the kernel has no loop
// and no data-dependent branch between its loads and their uses.  That lets
// the compiler count the memory counter exactly.  The loads are issued in the
// order
//     x staging item(s), scales and biases of every step, then the weight
//     chunks step by step (row by row within a step),
// and since loads retire in issue order, the product of (step t, row r)
// waits only for the chunks issued before it: a wave starts on its first
// chunk as soon as that chunk lands instead of after its whole weight stream.
// (The loop kernel's waits are merged over loop paths and wait for the next
// step's loads as well.)  Row blocks follow the XCD order of xcd_block.
//
// Measured on MI355X for 14336x4096 4-bit g64 (graph replays over 16
// rotated input sets, medians of interleaved rounds on one box): loop kernel
// 7.94 us, straight line with XCD row order 7.62-7.80 us.
#pragma once

#include "qmv_kernels.h"

namespace qmvk {

// FULL: Kc == CPL * 64 (every lane has a chunk at every step).  Otherwise
// Kc > (CPL - 1) * 64 and lanes past Kc in the last step re-read the row's
// last chunk and contribute zero (scale and bias term forced to 0).
template <int BITS, int RPW, int WPB, int CPL, bool FULL>
__global__ __launch_bounds__(WPB * kWave) void qmv_line_kernel(QmvArgs a) {
  constexpr int NT = WPB * kWave;
  constexpr bool PAIR = BITS <= 6;
  constexpr int kStride = chunk_stride_for<BITS, PAIR, 1>();
  constexpr bool TWO = PAIR && two_sums<BITS>();   // X' follows X (PairPlan)
  constexpr int XI = (CPL * kWave + NT - 1) / NT;   // x staging items per thread
  // 8-bit codes, and 4-bit codes at one row per wave, stage x in 16-byte
  // pieces (a quarter chunk) taken by consecutive lanes, so each load
  // instruction reads 1 KB of x: a float, or a 4-bit pair's two values, lie
  // inside one piece.  (Against whole chunks per lane, MI355X, 3
  // alternations: 8-bit 14336x4096 g32/64/128 13.4/13.3/13.2 ->
  // 13.1/13.0/12.8 us, gate/up 24.5 -> 24.0, 4096x4096 4-bit 4.06 -> 3.98;
  // but 14336x4096 4-bit, two rows per wave, 7.57 -> 7.71.)
  constexpr bool PIECES = BITS == 8 || (BITS == 4 && RPW == 1);
  constexpr int XP = (4 * CPL * kWave + NT - 1) / NT;   // pieces per thread
  extern __shared__ __align__(16) unsigned char smem[];

  const int Kc = a.K >> 5;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t total = static_cast<int64_t>(a.nmat) * a.N;
  const int64_t row0 = (xcd_block(blockIdx.x, gridDim.x) * WPB + wid) * RPW;
  const int64_t wstride = static_cast<int64_t>(Kc) * BITS;
  const int64_t gstride = Kc >> a.gshift;

  uint32_t raw[PIECES ? 1 : XI][16];
  uint4 praw[PIECES ? XP : 1];
  if constexpr (PIECES) {
    // piece t + i NT is quarter (t & 3) of chunk (t + i NT) / 4; a wave
    // whose pieces all lie past Kc loads nothing, lanes past it re-read
    // chunk Kc - 1.  Issued before the row addresses are formed (measured
    // faster here for one and two rows per wave).
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      if ((wid * kWave + i * NT) / 4 < Kc) {                  // wave-uniform
        const int pc = static_cast<int>(threadIdx.x) + i * NT;
        const int c = min(pc >> 2, Kc - 1);
        praw[i] = *reinterpret_cast<const uint4 *>(byte_offset(a.x, static_cast<uint32_t>(c * 64 + (pc & 3) * 16)));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  } else if constexpr (RPW == 1) {
    // x first: one row per wave is used for small matrices, where issuing
    // x before the row addresses are formed measured faster
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      if (wid * kWave + i * NT < Kc) {                        // wave-uniform
        const int it = min(static_cast<int>(threadIdx.x) + i * NT, Kc - 1);
        load_x_chunk(byte_offset(a.x, static_cast<uint32_t>(it) * 64), raw[i]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  const uint32_t *wrow[RPW];
  const uint16_t *srow[RPW], *brow[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    int64_t gr = row0 + r;
    if (gr > total - 1) gr = total - 1;
    const bool second = gr >= a.N;
    const int64_t lr = second ? gr - a.N : gr;
    wrow[r] = (second ? a.mat1.w : a.mat0.w) + lr * wstride;
    srow[r] = (second ? a.mat1.s : a.mat0.s) + lr * gstride;
    brow[r] = (second ? a.mat1.b : a.mat0.b) + lr * gstride;
  }
  auto chunk_of = [&](int t) -> uint32_t {
    return static_cast<uint32_t>(FULL ? t * kWave + lane : min(t * kWave + lane, Kc - 1));
  };

  // ---- 1. raw x of this thread's staging item(s); a wave whose items all
  // lie past Kc loads nothing (its threads would only re-read chunk Kc - 1).
  // With one row per wave (small matrices) they were issued above, before
  // the row addresses are formed.
  if constexpr (RPW != 1 && !PIECES) {
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      if (wid * kWave + i * NT < Kc) {                        // wave-uniform
        const int it = min(static_cast<int>(threadIdx.x) + i * NT, Kc - 1);
        load_x_chunk(byte_offset(a.x, static_cast<uint32_t>(it) * 64), raw[i]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- 2. scales and biases of every step
  uint16_t sv[CPL][RPW], bv[CPL][RPW];
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const uint32_t gi = chunk_of(t) >> a.gshift;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      sv[t][r] = *byte_offset(srow[r], gi * 2);
      bv[t][r] = *byte_offset(brow[r], gi * 2);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. the weight chunks, in a fixed issue order (the waits follow it)
  uint32_t w[CPL][RPW][BITS];
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const uint32_t c = chunk_of(t);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      load_chunk<BITS>(byte_offset(wrow[r], c * (BITS * 4)), w[t][r]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- 4. x into LDS (waits for x only), one barrier
  if constexpr (PIECES) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      if ((wid * kWave + i * NT) / 4 < Kc) {                  // wave-uniform
        const int pc = static_cast<int>(threadIdx.x) + i * NT;
        const int c = min(pc >> 2, Kc - 1), q = pc & 3;
        const uint4 v = praw[i];
        // the chunk's sum: this piece's 8 values in order, then the four
        // pieces' partial sums across the chunk's adjacent lanes
        float sum;
        unsigned char *chunk = smem + c * kStride;
        if constexpr (PAIR) {
          sum = dot2_bf16(v.x, 0x3F803F80u, 0.0f);
          sum = dot2_bf16(v.y, 0x3F803F80u, sum);
          sum = dot2_bf16(v.z, 0x3F803F80u, sum);
          sum = dot2_bf16(v.w, 0x3F803F80u, sum);
          // pair j of the piece = (x[j], x[j + 4])
          *reinterpret_cast<uint4 *>(chunk + q * 16) = make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                                                                  __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                                                                  __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                                                                  __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
        } else {
          const uint32_t r[4] = {v.x, v.y, v.z, v.w};
          float f[8];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            f[k] = (k & 1) ? __uint_as_float(r[k >> 1] & 0xFFFF0000u) : __uint_as_float(r[k >> 1] << 16);
          sum = f[0];
#pragma unroll
          for (int k = 1; k < 8; ++k) sum += f[k];
          *reinterpret_cast<float4 *>(chunk + q * 32) = make_float4(f[0], f[1], f[2], f[3]);
          *reinterpret_cast<float4 *>(chunk + q * 32 + 16) = make_float4(f[4], f[5], f[6], f[7]);
        }
        sum += dpp<kDppXor1>(sum);
        sum += dpp<kDppXor2>(sum);
        if (q == 0) *reinterpret_cast<float *>(chunk + vec_bytes<PAIR>()) = sum;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int it = static_cast<int>(threadIdx.x) + i * NT;
      if (wid * kWave + i * NT < Kc && ((i + 1) * NT <= CPL * kWave || it < Kc)) {
        const int its = min(it, Kc - 1);
        if constexpr (PAIR) stage_pairs_raw<BITS, 1>(raw[i], smem, 0, its);
        else stage_f32_raw<1>(raw[i], smem, 0, its);
      }
    }
  }
  __syncthreads();

  // ---- 5. products, one step at a time
  const PairConsts pk = pair_consts<BITS>();
  float acc[RPW], accz[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = accz[r] = 0.0f;
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const bool live = FULL || (t + 1) * kWave <= Kc || t * kWave + lane < Kc;
    const unsigned char *chunk = smem + chunk_of(t) * kStride;
    const float xs = *reinterpret_cast<const float *>(chunk + vec_bytes<PAIR>());
    const float xs2 = TWO ? *reinterpret_cast<const float *>(chunk + vec_bytes<PAIR>() + 4) : 0.0f;
    if constexpr (PAIR) {
      uint32_t xp[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = *reinterpret_cast<const uint4 *>(chunk + q * 16);
        xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        float d = 0.0f;
        static_for<0, 16>([&](auto i) {
          constexpr int I = decltype(i)::value;
          d = dot2_bf16(make_pair<BITS, I>(w[t][r], pk), xp[I], d);
        });
        float s = bf16_to_f32(sv[t][r]);
        // coefficient of X: z - 2^b s, or z with the second sum X' (times -2^b s)
        float zc = TWO ? bf16_to_f32(bv[t][r]) : fmaf(-static_cast<float>(1 << BITS), s, bf16_to_f32(bv[t][r]));
        if (!live) s = zc = 0.0f;
        acc[r] = fmaf(s, d, acc[r]);
        accz[r] = fmaf(zc, xs, accz[r]);
        if constexpr (TWO) accz[r] = fmaf(-static_cast<float>(1 << BITS) * s, xs2, accz[r]);
      }
    } else {
      float xf[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = *reinterpret_cast<const float4 *>(chunk + q * 16);
        xf[4 * q] = v.x; xf[4 * q + 1] = v.y; xf[4 * q + 2] = v.z; xf[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        float d0 = 0.0f, d1 = 0.0f;
        static_for<0, 16>([&](auto h) {
          constexpr int k = 2 * decltype(h)::value;
          d0 = fmaf(code_f32<BITS, k>(w[t][r]), xf[k], d0);
          d1 = fmaf(code_f32<BITS, k + 1>(w[t][r]), xf[k + 1], d1);
        });
        float s = bf16_to_f32(sv[t][r]);
        float z = bf16_to_f32(bv[t][r]);
        if (!live) s = z = 0.0f;
        acc[r] = fmaf(s, d0 + d1, fmaf(z, xs, acc[r]));
      }
    }
  }

  // ---- 6. reduce across the wave and store (one bf16 rounding)
  constexpr int V = pow2_ceil(RPW);
  float vals[V];
#pragma unroll
  for (int i = 0; i < V; ++i) vals[i] = 0.0f;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    if constexpr (PAIR) vals[r] = fmaf(acc[r], 1.0f / static_cast<float>(1 << PairPlan<BITS>::P), accz[r]);
    else vals[r] = acc[r];
  }
  const float tot = wave_reduce_many<V>(vals, lane);
  if (reduce_leader<V>(lane)) {
    const int r = reduce_index<V>(lane);
    const int64_t gr = row0 + r;
    if (r < RPW && gr < total) {
      const bool second = gr >= a.N;
      const int64_t lr = second ? gr - a.N : gr;
      void *y = second ? a.mat1.y : a.mat0.y;
      if (a.out_f32) static_cast<float *>(y)[lr] = tot;
      else static_cast<uint16_t *>(y)[lr] = f32_to_bf16(tot);
    }
  }
}

}  // namespace qmvk
