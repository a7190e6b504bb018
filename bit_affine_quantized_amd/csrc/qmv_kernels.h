// Kernel bodies for the gfx950 quantized matvec family.
//
// Work decomposition (all kernels):
//   * a workgroup is 4 waves; each wave owns RPW consecutive output rows;
//   * the K axis of a row is cut into 32-code chunks (b dwords each); lane l
//     of a wave takes chunks l, l+64, l+128, ... so one wave-wide load of
//     chunk words is a contiguous 64*b*4-byte run of the row (coalesced);
//   * x is staged once per workgroup into LDS in the layout the inner
//     product wants (pre-scaled bf16 pairs or fp32) together with one fp32
//     sum(x) per chunk, and each lane reads its chunk's x once and reuses it
//     for all RPW rows and for every x vector;
//   * the first two chunk steps of W are loaded before x is staged, so the
//     weight stream is already in flight while the workgroup converts x;
//   * partial sums (RPW rows x MV vectors per lane) meet in one butterfly
//     wave reduction and the leaders write y.
#pragma once

#include "qmv_device.h"

namespace qmvk {

struct MatDesc {
  const uint32_t *w;
  const uint16_t *s;
  const uint16_t *b;
  void *y;
};

// Bytes of LDS that a staged x vector takes per 32-code chunk.
template <bool PAIR>
constexpr int stage_bytes_per_chunk() { return PAIR ? 64 + 4 : 128 + 4; }

// ----------------------------------------------------------------------------
// x staging.  Pair layout: quad q (pairs 4q..4q+3) of vector m, chunk c at
// uint4 index (m*4 + q)*Kc + c.  fp32 layout: quad q (codes 4q..4q+3) at
// float4 index (m*8 + q)*Kc + c.  Sums at float index m*Kc + c after the
// quads.  Consecutive lanes read consecutive 16-byte slots: no bank conflict.
// ----------------------------------------------------------------------------
// Raw x of one chunk: 32 bf16 = 16 words.
__device__ __forceinline__ void load_x_chunk(const uint16_t *__restrict__ xk, uint32_t (&raw)[16]) {
  const uint4 *src = reinterpret_cast<const uint4 *>(xk);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = src[q];
    raw[4 * q] = v.x; raw[4 * q + 1] = v.y; raw[4 * q + 2] = v.z; raw[4 * q + 3] = v.w;
  }
}

__device__ __forceinline__ float raw_x(const uint32_t (&raw)[16], int k) {
  const uint32_t wv = raw[k >> 1];
  return (k & 1) ? __uint_as_float(wv & 0xFFFF0000u) : __uint_as_float(wv << 16);
}

// Pair staging: pair i of a chunk holds x[lo(i)] in its low half and x[hi(i)]
// in its high half, both raw bf16 (one v_perm_b32 per pair).  The chunk sum
// is taken with dot2 against (1, 1): products by 1 are exact, so it is a
// plain fp32 sum of the 32 values in a fixed order.
template <int BITS>
__device__ __forceinline__ void stage_pairs_raw(const uint32_t (&raw)[16], unsigned char *lds,
                                                int Kc, int MVtot, int m, int c) {
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) sum = dot2_bf16(raw[k], 0x3F803F80u, sum);
  uint4 *dst = reinterpret_cast<uint4 *>(lds);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * q + e;
      const int klo = PairPlan<BITS>::lo(i), khi = PairPlan<BITS>::hi(i);
      // v_perm_b32(S0, S1, sel): selector bytes 0-3 pick S1's bytes, 4-7 S0's
      const uint32_t sel = ((khi & 1) ? 0x07060000u : 0x05040000u) | ((klo & 1) ? 0x0302u : 0x0100u);
      pr[e] = __builtin_amdgcn_perm(raw[khi >> 1], raw[klo >> 1], sel);
    }
    dst[(m * 4 + q) * Kc + c] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
  }
  float *sums = reinterpret_cast<float *>(lds + static_cast<size_t>(MVtot) * Kc * 64);
  sums[m * Kc + c] = sum;
}

template <int BITS>
__device__ __forceinline__ void stage_pairs_chunk(const uint16_t *__restrict__ xk,
                                                  unsigned char *lds, int Kc, int MVtot,
                                                  int m, int c) {
  uint32_t raw[16];
  load_x_chunk(xk, raw);
  stage_pairs_raw<BITS>(raw, lds, Kc, MVtot, m, c);
}

__device__ __forceinline__ void store_f32_chunk(const float (&v)[32], unsigned char *lds, int Kc,
                                                int MVtot, int m, int c) {
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) sum += v[k];
  float4 *dst = reinterpret_cast<float4 *>(lds);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    dst[(m * 8 + q) * Kc + c] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  float *sums = reinterpret_cast<float *>(lds + static_cast<size_t>(MVtot) * Kc * 128);
  sums[m * Kc + c] = sum;
}

__device__ __forceinline__ void stage_f32_raw(const uint32_t (&raw)[16], unsigned char *lds,
                                              int Kc, int MVtot, int m, int c) {
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) v[k] = raw_x(raw, k);
  store_f32_chunk(v, lds, Kc, MVtot, m, c);
}

__device__ __forceinline__ void stage_f32_chunk(const uint16_t *__restrict__ xk, unsigned char *lds,
                                                int Kc, int MVtot, int m, int c) {
  uint32_t raw[16];
  load_x_chunk(xk, raw);
  stage_f32_raw(raw, lds, Kc, MVtot, m, c);
}

// h = silu(gate) * up in fp32 (metrale QuantWeights::gemv_silu_gate_resid).
__device__ __forceinline__ void stage_silu_raw(const uint32_t (&graw)[16], const uint32_t (&uraw)[16],
                                               unsigned char *lds, int Kc, int c) {
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const float g = raw_x(graw, k);
    const float u = raw_x(uraw, k);
    v[k] = g / (1.0f + __expf(-g)) * u;
  }
  store_f32_chunk(v, lds, Kc, 1, 0, c);
}

// ----------------------------------------------------------------------------
// The streaming dot-product engine for one wave: RPW rows x MV x-vectors.
// ----------------------------------------------------------------------------
template <int BITS, int RPW>
struct ChunkStep {
  uint32_t w[RPW][BITS];
  uint16_t s[RPW];
  uint16_t b[RPW];
};

template <int BITS, int RPW, int MV, bool PAIR>
struct WaveEngine {
  const uint32_t *wrow[RPW];
  const uint16_t *srow[RPW];
  const uint16_t *brow[RPW];
  int Kc;
  int gshift;
  int lane;
  int nsteps;
  PairConsts pk;
  // pair path: acc = sum s*D (D carries the codes scaled by 2^P), accz =
  // sum (z - 2^b s)*sum(x); result = 2^-P acc + accz.  fp32 path: acc only.
  float acc[RPW][MV];
  float accz[RPW][MV];
  ChunkStep<BITS, RPW> A, B;

  __device__ __forceinline__ float result(int r, int m) const {
    if constexpr (PAIR) return fmaf(acc[r][m], 1.0f / static_cast<float>(1 << PairPlan<BITS>::P), accz[r][m]);
    else return acc[r][m];
  }

  __device__ __forceinline__ void init(int Kc_, int gshift_, int lane_) {
    Kc = Kc_;
    gshift = gshift_;
    lane = lane_;
    pk = pair_consts<BITS>();
    nsteps = (Kc + kWave - 1) / kWave;
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        acc[r][m] = 0.0f;
        accz[r][m] = 0.0f;
      }
  }

  // Loads are branch-free: lanes past the row's end re-read its last chunk
  // (compute() ignores them).  With no divergent branches around the loads
  // the compiler's memory-counter waits stay exact, so waiting for x (loaded
  // first) never waits for weight words that are still in flight.
  __device__ __forceinline__ void load(int step, ChunkStep<BITS, RPW> &st) const {
    // 32-bit offsets from wave-uniform row bases: one VGPR offset per load
    const uint32_t c = static_cast<uint32_t>(min(step * kWave + lane, Kc - 1));
    const uint32_t gi = c >> gshift;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      load_chunk<BITS>(byte_offset(wrow[r], c * (BITS * 4)), st.w[r]);
      st.s[r] = *byte_offset(srow[r], gi * 2);
      st.b[r] = *byte_offset(brow[r], gi * 2);
    }
  }

  __device__ __forceinline__ void compute(int step, const ChunkStep<BITS, RPW> &st,
                                          const unsigned char *lds, int MVtot, int nv) {
    const int c = step * kWave + lane;
    if (c >= Kc) return;
    if constexpr (PAIR && MV == 1) {
      // one x vector: keep its pairs in registers, build one row's pairs at a time
      const uint4 *xq = reinterpret_cast<const uint4 *>(lds);
      const float *sums = reinterpret_cast<const float *>(lds + static_cast<size_t>(MVtot) * Kc * 64);
      uint32_t xp[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 v = xq[q * Kc + c];
        xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
      }
      const float xs = sums[c];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float s = bf16_to_f32(st.s[r]);
        const float zc = fmaf(-static_cast<float>(1 << BITS), s, bf16_to_f32(st.b[r]));  // z - 2^b s
        float d = 0.0f;
        static_for<0, 16>([&](auto i) {
          constexpr int I = decltype(i)::value;
          d = dot2_bf16(make_pair<BITS, I>(st.w[r], pk), xp[I], d);
        });
        acc[r][0] = fmaf(s, d, acc[r][0]);
        accz[r][0] = fmaf(zc, xs, accz[r][0]);
      }
    } else if constexpr (PAIR) {
      // build every row's pairs once, then stream the x vectors past them
      const uint4 *xq = reinterpret_cast<const uint4 *>(lds);
      const float *sums = reinterpret_cast<const float *>(lds + static_cast<size_t>(MVtot) * Kc * 64);
      uint32_t pr[RPW][16];
      float sc[RPW], zc[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        sc[r] = bf16_to_f32(st.s[r]);
        zc[r] = fmaf(-static_cast<float>(1 << BITS), sc[r], bf16_to_f32(st.b[r]));  // z - 2^b s
        static_for<0, 16>([&](auto i) { pr[r][decltype(i)::value] = make_pair<BITS, decltype(i)::value>(st.w[r], pk); });
      }
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        if (m < nv) {
          uint32_t xp[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint4 v = xq[(m * 4 + q) * Kc + c];
            xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
          }
          const float xs = sums[m * Kc + c];
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            float d = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) d = dot2_bf16(pr[r][i], xp[i], d);
            acc[r][m] = fmaf(sc[r], d, acc[r][m]);
            accz[r][m] = fmaf(zc[r], xs, accz[r][m]);
          }
        }
      }
    } else {
      const float4 *xq = reinterpret_cast<const float4 *>(lds);
      const float *sums = reinterpret_cast<const float *>(lds + static_cast<size_t>(MVtot) * Kc * 128);
      if constexpr (MV == 1) {
        // one x vector: keep it in registers, convert one row's codes at a time
        float xf[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          float4 v = xq[q * Kc + c];
          xf[4 * q] = v.x; xf[4 * q + 1] = v.y; xf[4 * q + 2] = v.z; xf[4 * q + 3] = v.w;
        }
        const float xs = sums[c];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          float d0 = 0.0f, d1 = 0.0f;
          static_for<0, 16>([&](auto h) {
            constexpr int k = 2 * decltype(h)::value;
            d0 = fmaf(code_f32<BITS, k>(st.w[r]), xf[k], d0);
            d1 = fmaf(code_f32<BITS, k + 1>(st.w[r]), xf[k + 1], d1);
          });
          acc[r][0] = fmaf(bf16_to_f32(st.s[r]), d0 + d1, fmaf(bf16_to_f32(st.b[r]), xs, acc[r][0]));
        }
      } else {
        float qf[RPW][32];
#pragma unroll
        for (int r = 0; r < RPW; ++r)
          static_for<0, 32>([&](auto k) { qf[r][decltype(k)::value] = code_f32<BITS, decltype(k)::value>(st.w[r]); });
#pragma unroll
        for (int m = 0; m < MV; ++m) {
          if (m < nv) {
            float xf[32];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              float4 v = xq[(m * 8 + q) * Kc + c];
              xf[4 * q] = v.x; xf[4 * q + 1] = v.y; xf[4 * q + 2] = v.z; xf[4 * q + 3] = v.w;
            }
            const float xs = sums[m * Kc + c];
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
              float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
              for (int k = 0; k < 32; k += 2) {
                d0 = fmaf(qf[r][k], xf[k], d0);
                d1 = fmaf(qf[r][k + 1], xf[k + 1], d1);
              }
              acc[r][m] = fmaf(bf16_to_f32(st.s[r]), d0 + d1, fmaf(bf16_to_f32(st.b[r]), xs, acc[r][m]));
            }
          }
        }
      }
    }
  }

  // Issue the first two steps' loads (before x staging); with one step the
  // second load re-reads cached words and is never used.
  __device__ __forceinline__ void prefetch() {
    load(0, A);
    load(1, B);
  }

  __device__ __forceinline__ void run(const unsigned char *lds, int MVtot, int nv) {
    for (int step = 0; step < nsteps; step += 2) {
      compute(step, A, lds, MVtot, nv);
      if (step + 2 < nsteps) load(step + 2, A);
      if (step + 1 < nsteps) {
        compute(step + 1, B, lds, MVtot, nv);
        if (step + 3 < nsteps) load(step + 3, B);
      }
    }
  }
};

// ----------------------------------------------------------------------------
// qmv / gate_up / silu-tail kernel.  Rows of `nmat` matrices (same N, K, bits,
// group size) are concatenated; wave w of block b owns rows (4b + w)*RPW...
// ----------------------------------------------------------------------------
enum { XIN_PLAIN = 0, XIN_SILU = 1 };

struct QmvArgs {
  const uint16_t *x;      // [M, K] bf16 (plain) or gate [K] (silu)
  const uint16_t *up;     // silu: up [K]
  const uint16_t *xres;   // silu: residual [N] or null
  MatDesc mat0, mat1;
  int nmat;
  int64_t N;              // rows per matrix
  int K;
  int M;                  // x vectors in this launch (<= MV)
  int gshift;             // log2(group_size / 32)
  int out_f32;
  int64_t y_ld;           // stride between output vectors (elements)
};

template <int BITS, int RPW, int MV, int XIN>
__global__ __launch_bounds__(kBlock) void qmv_kernel(QmvArgs a) {
  constexpr bool PAIR = (BITS <= 6) && (XIN == XIN_PLAIN);
  extern __shared__ __align__(16) unsigned char smem[];
  const int Kc = a.K >> 5;
  const int lane = threadIdx.x & (kWave - 1);
  // wave index, made visibly wave-uniform so row pointers live in SGPRs
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t total = static_cast<int64_t>(a.nmat) * a.N;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wid) * RPW;
  const int64_t wstride = static_cast<int64_t>(Kc) * BITS;
  const int64_t gstride = Kc >> a.gshift;

  WaveEngine<BITS, RPW, MV, PAIR> eng;
  eng.init(Kc, a.gshift, lane);
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    int64_t gr = row0 + r;
    if (gr > total - 1) gr = total - 1;
    const bool second = gr >= a.N;
    const int64_t lr = second ? gr - a.N : gr;
    eng.wrow[r] = (second ? a.mat1.w : a.mat0.w) + lr * wstride;
    eng.srow[r] = (second ? a.mat1.s : a.mat0.s) + lr * gstride;
    eng.brow[r] = (second ? a.mat1.b : a.mat0.b) + lr * gstride;
  }

  // Stage x for the whole workgroup.  The first staging item's raw x is
  // loaded BEFORE the weight prefetch: memory counters retire in issue
  // order, so converting it then waits only for x, not for the weights.
  const int items = (XIN == XIN_SILU) ? Kc : a.M * Kc;
  uint32_t raw0[16], raw1[16];
  auto load_item = [&](int it) {
    const uint32_t off = static_cast<uint32_t>(it) * 64;   // bytes of m*K + c*32 == it*32
    load_x_chunk(byte_offset(a.x, off), raw0);
    if constexpr (XIN == XIN_SILU) load_x_chunk(byte_offset(a.up, off), raw1);
  };
  auto stage_item = [&](int it) {
    if constexpr (XIN == XIN_SILU) {
      stage_silu_raw(raw0, raw1, smem, Kc, it);
    } else {
      const int m = it / Kc, c = it - m * Kc;
      if constexpr (PAIR) stage_pairs_raw<BITS>(raw0, smem, Kc, MV, m, c);
      else stage_f32_raw(raw0, smem, Kc, MV, m, c);
    }
  };
  // First item: an unconditional (clamped) load issued before the weight
  // prefetch and pinned there, then staged by every thread (threads past the
  // end restage the last item: identical bytes to identical addresses).
  const int it0 = threadIdx.x;
  load_item(min(it0, items - 1));
  __builtin_amdgcn_sched_barrier(0);
  eng.prefetch();
  if (wid * kWave < items) stage_item(min(it0, items - 1));   // wave-uniform
  for (int it = it0 + kBlock; it < items; it += kBlock) {
    load_item(it);
    stage_item(it);
  }
  __syncthreads();

  eng.run(smem, (XIN == XIN_SILU) ? 1 : MV, a.M);

  constexpr int V = pow2_ceil(RPW * MV);
  float vals[V];
#pragma unroll
  for (int i = 0; i < V; ++i) vals[i] = 0.0f;
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MV; ++m) vals[r * MV + m] = eng.result(r, m);
  const float tot = wave_reduce_many<V>(vals, lane);
  if (reduce_leader<V>(lane)) {
    const int idx = reduce_index<V>(lane);
    const int r = idx / MV, m = idx % MV;
    const int64_t gr = row0 + r;
    if (idx < RPW * MV && m < a.M && gr < total) {
      const bool second = gr >= a.N;
      const int64_t lr = second ? gr - a.N : gr;
      void *y = second ? a.mat1.y : a.mat0.y;
      float out = tot;
      if constexpr (XIN == XIN_SILU) {
        if (a.xres) out += bf16_to_f32(a.xres[lr]);
      }
      const int64_t o = static_cast<int64_t>(m) * a.y_ld + lr;
      if (a.out_f32) static_cast<float *>(y)[o] = out;
      else static_cast<uint16_t *>(y)[o] = f32_to_bf16(out);
    }
  }
}

// ----------------------------------------------------------------------------
// Gather kernel (mlx.core.gather_qmm; quantized.h adjust_matrix_offsets):
// y[p] = x[lhs[p]] @ W[rhs[p]]^T.  Workgroup (e, tile) serves every pair p
// with rhs[p] == e: it reads tile rows of expert e's W ONCE for all of them
// (x vectors batched MV at a time).  The pairs of e are found in order of p,
// by a scan of rhs (any order) or by binary search when rhs is sorted, so
// both modes run the same arithmetic for every output.
// ----------------------------------------------------------------------------
struct GatherArgs {
  const uint16_t *x;        // [Bx, M, K]
  const uint32_t *w;        // [E, N, K*bits/32]
  const uint16_t *s, *b;    // [E, N, K/g]
  const uint32_t *lhs, *rhs;
  int64_t P;
  int64_t N;
  int K;
  int M;
  int gshift;
  int tiles;                // row tiles per expert
  int sorted;
  int out_f32;
  void *y;                  // [P, M, N]
};

constexpr int kGatherListMax = 1024;   // pairs of one expert handled per pass

template <int BITS, int RPW, int MV>
__global__ __launch_bounds__(kBlock) void gather_kernel(GatherArgs a) {
  constexpr bool PAIR = BITS <= 6;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int list[kGatherListMax];
  __shared__ int list_n;
  __shared__ int list_base;
  const int e = blockIdx.x / a.tiles;
  const int tile = blockIdx.x - e * a.tiles;
  const int lane = threadIdx.x & (kWave - 1);
  // wave index, made visibly wave-uniform so row pointers live in SGPRs
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Kc = a.K >> 5;
  const int64_t wstride = static_cast<int64_t>(Kc) * BITS;
  const int64_t gstride = Kc >> a.gshift;
  const int64_t row0 = (static_cast<int64_t>(tile) * kWavesPerBlock + wid) * RPW;

  // ---- the ordered list of pairs routed to expert e
  if (a.sorted) {
    if (threadIdx.x == 0) {
      int64_t lo = 0, hi = a.P;
      while (lo < hi) { int64_t mid = (lo + hi) >> 1; if (a.rhs[mid] < static_cast<uint32_t>(e)) lo = mid + 1; else hi = mid; }
      int64_t lo2 = lo, hi2 = a.P;
      while (lo2 < hi2) { int64_t mid = (lo2 + hi2) >> 1; if (a.rhs[mid] <= static_cast<uint32_t>(e)) lo2 = mid + 1; else hi2 = mid; }
      list_base = static_cast<int>(lo);
      list_n = static_cast<int>(lo2 - lo);
    }
    __syncthreads();
  } else {
    if (wid == 0) {
      int n = 0;
      for (int64_t p0 = 0; p0 < a.P; p0 += kWave) {
        const int64_t p = p0 + lane;
        const bool hit = p < a.P && a.rhs[p] == static_cast<uint32_t>(e);
        const unsigned long long mask = __ballot(hit);
        const int before = __popcll(mask & ((1ull << lane) - 1ull));
        if (hit && n + before < kGatherListMax) list[n + before] = static_cast<int>(p);
        n += __popcll(mask);
      }
      if (lane == 0) { list_n = n; list_base = -1; }
    }
    __syncthreads();
  }
  const int npairs = list_n;
  if (npairs == 0) return;   // uniform across the workgroup
  const int base = list_base;
  const int nvec_total = npairs * a.M;

  const uint32_t *we = a.w + static_cast<int64_t>(e) * a.N * wstride;
  const uint16_t *se = a.s + static_cast<int64_t>(e) * a.N * gstride;
  const uint16_t *be = a.b + static_cast<int64_t>(e) * a.N * gstride;

  for (int v0 = 0; v0 < nvec_total; v0 += MV) {
    const int nv = min(MV, nvec_total - v0);
    WaveEngine<BITS, RPW, MV, PAIR> eng;
    eng.init(Kc, a.gshift, lane);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      int64_t gr = row0 + r;
      if (gr > a.N - 1) gr = a.N - 1;
      eng.wrow[r] = we + gr * wstride;
      eng.srow[r] = se + gr * gstride;
      eng.brow[r] = be + gr * gstride;
    }
    eng.prefetch();
    for (int it = threadIdx.x; it < nv * Kc; it += kBlock) {
      const int mv = it / Kc, c = it - mv * Kc;
      const int vec = v0 + mv;
      const int pi = vec / a.M, m = vec - pi * a.M;
      const int p = base >= 0 ? base + pi : (pi < kGatherListMax ? list[pi] : 0);
      const uint16_t *xk = a.x + (static_cast<int64_t>(a.lhs[p]) * a.M + m) * a.K + static_cast<int64_t>(c) * 32;
      if constexpr (PAIR) stage_pairs_chunk<BITS>(xk, smem, Kc, MV, mv, c);
      else stage_f32_chunk(xk, smem, Kc, MV, mv, c);
    }
    __syncthreads();
    eng.run(smem, MV, nv);

    constexpr int V = pow2_ceil(RPW * MV);
    float vals[V];
#pragma unroll
    for (int i = 0; i < V; ++i) vals[i] = 0.0f;
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int m = 0; m < MV; ++m) vals[r * MV + m] = eng.result(r, m);
    const float tot = wave_reduce_many<V>(vals, lane);
    if (reduce_leader<V>(lane)) {
      const int idx = reduce_index<V>(lane);
      const int r = idx / MV, mv = idx % MV;
      const int64_t gr = row0 + r;
      if (idx < RPW * MV && mv < nv && gr < a.N) {
        const int vec = v0 + mv;
        const int pi = vec / a.M, m = vec - pi * a.M;
        const int p = base >= 0 ? base + pi : list[pi];
        const int64_t o = (static_cast<int64_t>(p) * a.M + m) * a.N + gr;
        if (a.out_f32) static_cast<float *>(a.y)[o] = tot;
        else static_cast<uint16_t *>(a.y)[o] = f32_to_bf16(tot);
      }
    }
    __syncthreads();   // LDS reuse by the next batch of vectors
  }
}

}  // namespace qmvk
