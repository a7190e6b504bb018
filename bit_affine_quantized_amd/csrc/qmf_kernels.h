// qmf: 2 to 16 rows of x against one 4-bit weight on the matrix cores, with
// K split across the waves of one workgroup instead of across workgroups, so
// no partial sums leave the workgroup and no second kernel adds them.
//
// A workgroup owns 16 W rows (one MFMA column tile) and all of K; wave w of
// its 8 takes the K range of CW chunks starting at chunk w * CW.  The
// arithmetic is the matrix-core product of qmm_kernels.h: the magic-bf16
// code 128 + q * 2^P (P = 3) is an exact bf16 B operand, one
// v_mfma_f32_16x16x32_bf16 contracts one 32-code chunk for 16 W rows by 16 x
// rows, the chunks of a group chain in the accumulator and the group is
// folded once, 2^-P s D + (z - 16 s) X.  Here the x sums X come from a
// second MFMA against a B operand of ones, and lane group kb of both
// operands holds the pair order (8kb + e, 8kb + e + 4) of the chunk.
//
// Each wave issues all of its loads at once (straight-line code, exact
// memory-counter waits): its W in 16-byte pieces, consecutive lanes taking
// consecutive chunks of one row (every load instruction reads whole cache
// lines), the scales and biases of its groups, and for every chunk one
// 16-byte x piece per lane (lanes of x rows past M read zeros without a
// memory request; their results are never stored).  W then goes through the
// wave's own LDS region once to reach the MFMA's row-per-lane layout.  The 8
// waves' 16 x 16 results meet in LDS and are added in wave order.
#pragma once

#include "qmm_kernels.h"

namespace qmvk {

struct QmfArgs {
  const uint16_t *x;        // [M, K] bf16
  const uint32_t *w;        // [N, K/8] (4-bit codes)
  const uint16_t *s, *b;    // [N, K/g]
  void *y;                  // [M, N], row stride y_ld
  int64_t N;
  int64_t y_ld;
  int K;
  int M;                    // 1..16
  int out_f32;
};

constexpr int kQmfWaves = 8;
constexpr int kQmfThreads = kQmfWaves * kWave;

template <int CW>
constexpr int qmf_row_bytes() { return CW * 16 + 4; }   // padded: row-per-lane reads avoid bank conflicts
template <int CW>
constexpr int qmf_lds_bytes() {
  return kQmfWaves * 16 * qmf_row_bytes<CW>() > kQmfWaves * 16 * 16 * 4
             ? kQmfWaves * 16 * qmf_row_bytes<CW>() : kQmfWaves * 16 * 16 * 4;
}

// NG consecutive bf16 values (NG * 2 bytes, aligned to that size) as raw bits
template <int NG>
__device__ __forceinline__ void load_bf16s(const uint16_t *p, uint16_t (&out)[NG]) {
  static_assert(NG == 2 || NG == 4 || NG == 8 || NG == 16, "2-16 values");
  uint32_t w[NG / 2];
  if constexpr (NG == 2) {
    w[0] = *reinterpret_cast<const uint32_t *>(p);
  } else if constexpr (NG == 4) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int h = 0; h < NG / 8; ++h) {
      const uint4 v = reinterpret_cast<const uint4 *>(p)[h];
      w[4 * h] = v.x; w[4 * h + 1] = v.y; w[4 * h + 2] = v.z; w[4 * h + 3] = v.w;
    }
  }
#pragma unroll
  for (int i = 0; i < NG; ++i) out[i] = static_cast<uint16_t>(w[i >> 1] >> (16 * (i & 1)));
}

template <int CW, int CPG>
__global__ __launch_bounds__(kQmfThreads) void qmf_kernel(QmfArgs a) {
  static_assert(CW % 4 == 0 && CW % CPG == 0, "whole pieces and groups per wave");
  constexpr int NPL = CW / 4;              // W pieces per lane: 16 rows x CW chunks / 64 lanes
  constexpr int NG = CW / CPG;             // groups per wave
  constexpr int RB = qmf_row_bytes<CW>();
  constexpr int P = 3;
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int j = lane & 15, kb = lane >> 4;
  const int Kc = a.K >> 5;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int c0 = wid * CW;                            // the wave's first chunk
  const uint32_t rowb = static_cast<uint32_t>(Kc) * 16u;   // W bytes per row
  const uint32_t gpr = static_cast<uint32_t>(Kc / CPG);    // groups per row

  // ---- 1. W: piece p = i * 64 + lane is chunk p % CW of row p / CW
  uint32_t wp[NPL][4];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int p = i * kWave + lane;
    const int r = p / CW, cc = p % CW;
    const int64_t n = n0 + r < a.N ? n0 + r : a.N - 1;
    const uint4 v = *reinterpret_cast<const uint4 *>(
        byte_offset(a.w, static_cast<uint32_t>(n) * rowb + static_cast<uint32_t>(c0 + cc) * 16u));
    wp[i][0] = v.x; wp[i][1] = v.y; wp[i][2] = v.z; wp[i][3] = v.w;
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. scales and biases of W row j over the wave's NG groups
  uint16_t sv[NG], bv[NG];
  {
    const int64_t n = n0 + j < a.N ? n0 + j : a.N - 1;
    const uint32_t o = (static_cast<uint32_t>(n) * gpr + static_cast<uint32_t>(c0 / CPG)) * 2u;
    load_bf16s<NG>(byte_offset(a.s, o), sv);
    load_bf16s<NG>(byte_offset(a.b, o), bv);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. x: chunk cc's 8 values 8kb..8kb+7 of x row j, through a buffer
  // resource over the M rows: lanes of rows past M take an offset past its
  // end, so their loads return zeros and make no memory request (the A rows
  // they fill only meet outputs that are never stored), while every lane
  // still issues the same instructions
  uint4 xv[CW];
  {
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.x), 0, a.M * a.K * 2, kBufferDword3);
    const uint32_t xo = j < a.M ? static_cast<uint32_t>(j) * static_cast<uint32_t>(a.K) * 2u +
                                      static_cast<uint32_t>(c0) * 64u + static_cast<uint32_t>(kb) * 16u
                                : 0x80000000u;
#pragma unroll
    for (int cc = 0; cc < CW; ++cc) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + cc * 64u, 0, 0);
      xv[cc] = make_uint4(v.x, v.y, v.z, v.w);
    }
  }

  // ---- 4. W through the wave's LDS region: row r, chunk cc at r RB + 16 cc
  unsigned char *wl = smem + wid * (16 * RB);
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int p = i * kWave + lane;
    *reinterpret_cast<uint4 *>(wl + (p / CW) * RB + (p % CW) * 16) = make_uint4(wp[i][0], wp[i][1], wp[i][2], wp[i][3]);
  }

  // ---- 5. products: per chunk, D += A.B (codes) and DX += A.1 (x sums)
  const PairConsts pk = pair_consts<4>();
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc = zero, accz = zero, D = zero, DX = zero;
  const unsigned char *wrow = wl + j * RB + kb * 4;   // dword kb of row j's chunks
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int v = 0; v < CPG; ++v) {
      const int cc = g * CPG + v;
      const uint32_t wd = *reinterpret_cast<const uint32_t *>(wrow + cc * 16);
      uint32_t bq[4];
      qmm_b_pairs<4>(wd, wd, 0u, pk, bq);
      const bf16x8_t B = __builtin_bit_cast(bf16x8_t, make_uint4(bq[0], bq[1], bq[2], bq[3]));
      const uint4 xr = xv[cc];
      // pair e = (x[8kb + e], x[8kb + e + 4])
      const bf16x8_t A = __builtin_bit_cast(
          bf16x8_t, make_uint4(__builtin_amdgcn_perm(xr.z, xr.x, 0x05040100u), __builtin_amdgcn_perm(xr.z, xr.x, 0x07060302u),
                               __builtin_amdgcn_perm(xr.w, xr.y, 0x05040100u), __builtin_amdgcn_perm(xr.w, xr.y, 0x07060302u)));
      D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, v == 0 ? zero : D, 0, 0, 0);
      DX = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, ones, v == 0 ? zero : DX, 0, 0, 0);
    }
    // fold the group: lane (j, kb) holds x rows 4kb + e against W row j
    const float s = bf16_to_f32(sv[g]);
    const float zc = fmaf(-16.0f, s, bf16_to_f32(bv[g]));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = fmaf(s, D[e], acc[e]);
      accz[e] = fmaf(zc, DX[e], accz[e]);
    }
  }

  // ---- 6. the 8 waves' results, added in wave order
  __syncthreads();                                     // every wave is done with its W region
  float *red = reinterpret_cast<float *>(smem);        // [wave][x row][W row]
#pragma unroll
  for (int e = 0; e < 4; ++e)
    red[(wid * 16 + 4 * kb + e) * 16 + j] = fmaf(acc[e], 1.0f / static_cast<float>(1 << P), accz[e]);
  __syncthreads();
  if (threadIdx.x < 256) {
    const int m = threadIdx.x >> 4, jj = threadIdx.x & 15;
    float v = red[m * 16 + jj];
#pragma unroll
    for (int w = 1; w < kQmfWaves; ++w) v += red[(w * 16 + m) * 16 + jj];
    const int64_t n = n0 + jj;
    if (m < a.M && n < a.N) {
      const int64_t o = static_cast<int64_t>(m) * a.y_ld + n;
      if (a.out_f32) static_cast<float *>(a.y)[o] = v;
      else static_cast<uint16_t *>(a.y)[o] = f32_to_bf16(v);
    }
  }
}

}  // namespace qmvk
