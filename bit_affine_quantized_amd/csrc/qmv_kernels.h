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

// Staged-x layout in LDS, chunk-major: chunk c of the staged vectors starts
// at c * chunk_stride<PAIR, MV, TWO>(); vector m's data sits at m * vec_bytes
// and the MV fp32 chunk sums X follow, in a 16-byte tail; with TWO (3- and
// 5-bit pairs, see PairPlan) the tail is 48 bytes and the MV second sums X'
// follow the first.  Every offset inside a chunk is a compile-time
// immediate, and the strides (an odd multiple of 16 bytes: 80/144/272 or
// 112/176/304 for bf16 pairs, 144/272/528 for fp32) put 16 consecutive lanes
// on 16 distinct 4-bank quads of LDS, so 128-bit reads do not conflict.
template <bool PAIR>
constexpr int vec_bytes() { return PAIR ? 64 : 128; }
template <bool PAIR, int MV, bool TWO = false>
constexpr int chunk_stride() {
  static_assert(MV >= 1 && MV <= 4, "at most 4 staged x vectors");
  return MV * vec_bytes<PAIR>() + (TWO ? 48 : 16);
}
// the staged layout of a kernel for BITS-bit codes
template <int BITS, bool PAIR, int MV>
constexpr int chunk_stride_for() { return chunk_stride<PAIR, MV, PAIR && two_sums<BITS>()>(); }
template <bool PAIR>
constexpr int stage_bytes_per_chunk() { return vec_bytes<PAIR>() + 16; }   // one vector (host sizing)

// ----------------------------------------------------------------------------
// x staging (layout above).
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
template <int BITS, int MV>
__device__ __forceinline__ void stage_pairs_raw(const uint32_t (&raw)[16], unsigned char *lds,
                                                int m, int c) {
  constexpr bool TWO = two_sums<BITS>();
  float sum = 0.0f, sum2 = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) sum = dot2_bf16(raw[k], 0x3F803F80u, sum);
  unsigned char *chunk = lds + c * chunk_stride<true, MV, TWO>();
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
      if (PairPlan<BITS>::doubled(i)) {
        // high half x -> 2x: an exact fp32 product whose low 16 bits stay 0
        const float h2 = 2.0f * __uint_as_float(pr[e] & 0xFFFF0000u);
        pr[e] = (pr[e] & 0xFFFFu) | __float_as_uint(h2);
      }
      if constexpr (TWO) sum2 = dot2_bf16(pr[e], 0x3F803F80u, sum2);
    }
    *reinterpret_cast<uint4 *>(chunk + m * 64 + q * 16) = make_uint4(pr[0], pr[1], pr[2], pr[3]);
  }
  reinterpret_cast<float *>(chunk + MV * 64)[m] = sum;
  if constexpr (TWO) reinterpret_cast<float *>(chunk + MV * 64)[MV + m] = sum2;
}

template <int BITS, int MV>
__device__ __forceinline__ void stage_pairs_chunk(const uint16_t *__restrict__ xk,
                                                  unsigned char *lds, int m, int c) {
  uint32_t raw[16];
  load_x_chunk(xk, raw);
  stage_pairs_raw<BITS, MV>(raw, lds, m, c);
}

template <int MV>
__device__ __forceinline__ void store_f32_chunk(const float (&v)[32], unsigned char *lds, int m, int c) {
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) sum += v[k];
  unsigned char *chunk = lds + c * chunk_stride<false, MV>();
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *reinterpret_cast<float4 *>(chunk + m * 128 + q * 16) =
        make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  reinterpret_cast<float *>(chunk + MV * 128)[m] = sum;
}

template <int MV>
__device__ __forceinline__ void stage_f32_raw(const uint32_t (&raw)[16], unsigned char *lds, int m, int c) {
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) v[k] = raw_x(raw, k);
  store_f32_chunk<MV>(v, lds, m, c);
}

template <int MV>
__device__ __forceinline__ void stage_f32_chunk(const uint16_t *__restrict__ xk, unsigned char *lds,
                                                int m, int c) {
  uint32_t raw[16];
  load_x_chunk(xk, raw);
  stage_f32_raw<MV>(raw, lds, m, c);
}

// h = silu(gate) * up in fp32 (metrale QuantWeights::gemv_silu_gate_resid).
// The quotient g / (1 + e^-g) is taken as g times the hardware reciprocal
// (v_rcp_f32, within 1 ulp) instead of an IEEE division: every workgroup
// recomputes h for the whole K, and the division's scale/refine/fixup
// sequence was most of that cost.  h then carries a few ulp of fp32 error,
// far inside the fp32 output tolerance.
__device__ __forceinline__ void stage_silu_raw(const uint32_t (&graw)[16], const uint32_t (&uraw)[16],
                                               unsigned char *lds, int c) {
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const float g = raw_x(graw, k);
    const float u = raw_x(uraw, k);
    v[k] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
  }
  store_f32_chunk<1>(v, lds, 0, c);
}

// ----------------------------------------------------------------------------
// The streaming dot-product engine for one wave: RPW rows x MV x-vectors.
// ----------------------------------------------------------------------------
// One chunk step of RPW rows: the chunk words and each row's scale and bias
// bf16 bits.  (Separate registers: packing the two into one register with
// d16/d16_hi loads chains the second load on the first and measured slower.)
template <int BITS, int RPW>
struct ChunkStep {
  uint32_t w[RPW][BITS];
  uint16_t s[RPW];
  uint16_t b[RPW];
  __device__ __forceinline__ float scale(int r) const { return bf16_to_f32(s[r]); }
  __device__ __forceinline__ float bias(int r) const { return bf16_to_f32(b[r]); }
};

// ----------------------------------------------------------------------------
// One 32-code chunk of RPW rows against MV staged x vectors; `chunk` is the
// staged chunk (layout above) and the caller has checked that it exists.
// ----------------------------------------------------------------------------
template <int BITS, int RPW, int MV, bool PAIR>
__device__ __forceinline__ void accumulate_chunk(const ChunkStep<BITS, RPW> &st, const unsigned char *chunk,
                                                 int nv, PairConsts pk,
                                                 float (&acc)[RPW][MV], float (&accz)[RPW][MV]) {
  const float *sums = reinterpret_cast<const float *>(chunk + MV * vec_bytes<PAIR>());
  constexpr bool TWO = PAIR && two_sums<BITS>();   // sums[MV + m] holds X' (PairPlan)
  if constexpr (PAIR && MV == 1) {
    // one x vector: keep its pairs in registers, build one row's pairs at a time
    uint32_t xp[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = *reinterpret_cast<const uint4 *>(chunk + q * 16);
      xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
    }
    const float xs = sums[0];
    const float xs2 = TWO ? sums[1] : 0.0f;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const float s = st.scale(r);
      // coefficient of X: z - 2^b s, or z with the second sum X' (times -2^b s)
      const float zc = TWO ? st.bias(r) : fmaf(-static_cast<float>(1 << BITS), s, st.bias(r));
      float d = 0.0f;
      static_for<0, 16>([&](auto i) {
        constexpr int I = decltype(i)::value;
        d = dot2_bf16(make_pair<BITS, I>(st.w[r], pk), xp[I], d);
      });
      acc[r][0] = fmaf(s, d, acc[r][0]);
      accz[r][0] = fmaf(zc, xs, accz[r][0]);
      if constexpr (TWO) accz[r][0] = fmaf(-static_cast<float>(1 << BITS) * s, xs2, accz[r][0]);
    }
  } else if constexpr (PAIR) {
    // build every row's pairs once, then stream the x vectors past them
    uint32_t pr[RPW][16];
    float sc[RPW], zc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      sc[r] = st.scale(r);
      // coefficient of X: z - 2^b s, or z with the second sum X' (times -2^b s)
      zc[r] = TWO ? st.bias(r) : fmaf(-static_cast<float>(1 << BITS), sc[r], st.bias(r));
      static_for<0, 16>([&](auto i) { pr[r][decltype(i)::value] = make_pair<BITS, decltype(i)::value>(st.w[r], pk); });
    }
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      if (m < nv) {
        uint32_t xp[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = *reinterpret_cast<const uint4 *>(chunk + m * 64 + q * 16);
          xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
        }
        const float xs = sums[m];
        const float xs2 = TWO ? sums[MV + m] : 0.0f;
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          float d = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) d = dot2_bf16(pr[r][i], xp[i], d);
          acc[r][m] = fmaf(sc[r], d, acc[r][m]);
          accz[r][m] = fmaf(zc[r], xs, accz[r][m]);
          if constexpr (TWO) accz[r][m] = fmaf(-static_cast<float>(1 << BITS) * sc[r], xs2, accz[r][m]);
        }
      }
      // keep one vector's x pairs live at a time (no hoisting of the next
      // vector's LDS reads above these products)
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    if constexpr (MV == 1) {
      // one x vector: keep it in registers, convert one row's codes at a time
      float xf[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = *reinterpret_cast<const float4 *>(chunk + q * 16);
        xf[4 * q] = v.x; xf[4 * q + 1] = v.y; xf[4 * q + 2] = v.z; xf[4 * q + 3] = v.w;
      }
      const float xs = sums[0];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        float d0 = 0.0f, d1 = 0.0f;
        static_for<0, 16>([&](auto h) {
          constexpr int k = 2 * decltype(h)::value;
          d0 = fmaf(code_f32<BITS, k>(st.w[r]), xf[k], d0);
          d1 = fmaf(code_f32<BITS, k + 1>(st.w[r]), xf[k + 1], d1);
        });
        acc[r][0] = fmaf(st.scale(r), d0 + d1, fmaf(st.bias(r), xs, acc[r][0]));
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
            const float4 v = *reinterpret_cast<const float4 *>(chunk + m * 128 + q * 16);
            xf[4 * q] = v.x; xf[4 * q + 1] = v.y; xf[4 * q + 2] = v.z; xf[4 * q + 3] = v.w;
          }
          const float xs = sums[m];
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
            for (int k = 0; k < 32; k += 2) {
              d0 = fmaf(qf[r][k], xf[k], d0);
              d1 = fmaf(qf[r][k + 1], xf[k + 1], d1);
            }
            acc[r][m] = fmaf(st.scale(r), d0 + d1, fmaf(st.bias(r), xs, acc[r][m]));
          }
        }
      }
    }
  }
}


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
                                          const unsigned char *lds, int nv) {
    const int c = step * kWave + lane;
    if (c >= Kc) return;
    accumulate_chunk<BITS, RPW, MV, PAIR>(st, lds + c * chunk_stride_for<BITS, PAIR, MV>(), nv, pk, acc, accz);
  }

  // Issue the first two steps' loads (before x staging); with one step the
  // second load re-reads cached words and is never used.
  __device__ __forceinline__ void prefetch() {
    load(0, A);
    load(1, B);
  }

  __device__ __forceinline__ void run(const unsigned char *lds, int nv) {
    for (int step = 0; step < nsteps; step += 2) {
      compute(step, A, lds, nv);
      if (step + 2 < nsteps) load(step + 2, A);
      if (step + 1 < nsteps) {
        compute(step + 1, B, lds, nv);
        if (step + 3 < nsteps) load(step + 3, B);
      }
    }
  }
};

// ----------------------------------------------------------------------------
// qmv / gate_up / silu-tail kernel.  Rows of `nmat` matrices (same N, K, bits,
// group size) are concatenated; wave w of block b owns rows (WPB b + w)*RPW...
// The whole grid is normally resident at once, so every wave's weight loads
// are issued at the start (a streaming grid that walks rows with a bounded
// number of loads in flight measured far slower on MI355X).
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

template <int BITS, int RPW, int MV, int XIN, int WPB>
__global__ __launch_bounds__(WPB * kWave) void qmv_kernel(QmvArgs a) {
  constexpr int kBlock = WPB * kWave;
  constexpr bool PAIR = (BITS <= 6) && (XIN == XIN_PLAIN);
  extern __shared__ __align__(16) unsigned char smem[];
  const int Kc = a.K >> 5;
  const int lane = threadIdx.x & (kWave - 1);
  // wave index, made visibly wave-uniform so row pointers live in SGPRs
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t total = static_cast<int64_t>(a.nmat) * a.N;
  const int64_t blk = xcd_block(blockIdx.x, gridDim.x);   // each XCD a contiguous run of rows
  const int64_t row0 = (blk * WPB + wid) * RPW;
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
      stage_silu_raw(raw0, raw1, smem, it);
    } else {
      // one-vector launches (MV == 1) skip the division: it costs ~30 VALU
      const int m = (MV == 1) ? 0 : it / Kc, c = it - m * Kc;
      if constexpr (PAIR) stage_pairs_raw<BITS, MV>(raw0, smem, m, c);
      else stage_f32_raw<MV>(raw0, smem, m, c);
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

  eng.run(smem, a.M);

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
// One chunk of one row against NV staged x vectors (bf16 pairs), taken a
// quad of pairs at a time: the quad's 4 pairs are built, then each vector's
// matching 16 bytes of x are read and folded into its own dot chain.  Only a
// quad's pairs and x are live at once (instead of all 16 pairs and a whole
// vector), and the NV chains interleave.
// ----------------------------------------------------------------------------
// Sum over aligned groups of SEG lanes (SEG = 8, 16, 32 or 64), by the same
// lane tree in every group; every lane of a group receives the total.
template <int SEG>
__device__ __forceinline__ float segment_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  if constexpr (SEG >= 16) v += dpp<kDppRor8>(v);
  if constexpr (SEG >= 32) {
    float a = v, b = v;
    swap16(a, b);
    v = a + b;
  }
  if constexpr (SEG >= 64) {
    float a = v, b = v;
    swap32(a, b);
    v = a + b;
  }
  return v;
}

template <int BITS, int MV, int NV>
__device__ __forceinline__ void gather_chunk_pairs(const uint32_t (&w)[BITS], uint16_t sb, uint16_t bb,
                                                   const unsigned char *chunk, PairConsts pk,
                                                   float (&acc)[1][MV], float (&accz)[1][MV]) {
  float d[NV];
  static_for<0, 4>([&](auto qq) {
    constexpr int q = decltype(qq)::value;
    uint32_t p[4];
    static_for<0, 4>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      p[j] = make_pair<BITS, 4 * q + j>(w, pk);
    });
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const uint4 xv = *reinterpret_cast<const uint4 *>(chunk + m * 64 + q * 16);
      float t = q == 0 ? 0.0f : d[m];
      t = dot2_bf16(p[0], xv.x, t);
      t = dot2_bf16(p[1], xv.y, t);
      t = dot2_bf16(p[2], xv.z, t);
      d[m] = dot2_bf16(p[3], xv.w, t);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the next quad's reads below this one
  });
  constexpr bool TWO = two_sums<BITS>();   // sums[MV + m] holds X' (PairPlan)
  const float *sums = reinterpret_cast<const float *>(chunk + MV * 64);
  const float s = bf16_to_f32(sb);
  // coefficient of X: z - 2^b s, or z with the second sum X' (times -2^b s)
  const float zc = TWO ? bf16_to_f32(bb) : fmaf(-static_cast<float>(1 << BITS), s, bf16_to_f32(bb));
#pragma unroll
  for (int m = 0; m < NV; ++m) {
    acc[0][m] = fmaf(s, d[m], acc[0][m]);
    accz[0][m] = fmaf(zc, sums[m], accz[0][m]);
    if constexpr (TWO) accz[0][m] = fmaf(-static_cast<float>(1 << BITS) * s, sums[MV + m], accz[0][m]);
  }
}

// ----------------------------------------------------------------------------
// Gather kernel (mlx.core.gather_qmm; quantized.h adjust_matrix_offsets):
// y[p] = x[lhs[p]] @ W[rhs[p]]^T.
//
// Workgroup (e, tile) owns `tile_rows` consecutive rows of expert e and
// serves every pair p with rhs[p] == e, so each row of an expert's weight is
// read once for all the tokens routed to it (up to MV x vectors at a time).
// The pairs of e are found by a block-wide ordered scan of rhs (ballot +
// per-wave counts): the list is in increasing p whatever the order of rhs,
// so sorted and unsorted indices run identical arithmetic for every output.
// Lists longer than kGatherListMax are processed in windows.
//
// Rows are cut into segments of SEG lanes (8 by default): a wave step covers
// 64 / SEG rows, and lane u of a row's segment takes chunks u, u + SEG, ...,
// u + SEG (CPL - 1) of the step's K range, so each of the CPL loads reads
// SEG x (chunk bytes) contiguous bytes of every row.  A row's partial sums
// meet in a DPP reduction inside its segment once per row group, not once
// per step: with few x vectors per expert the per-row reduction and
// bookkeeping of a one-row-per-wave layout cost as much as the dot products.
// Each wave streams its row groups (tile_rows / (waves x rows per step) of
// them, each K / (SEG x 32 CPL) steps long) through a DEPTH-deep load ring
// of branch-free buffer loads.
// ----------------------------------------------------------------------------
struct GatherArgs {
  const uint16_t *x;        // [Bx, M, K]
  const uint32_t *w;        // [E, N, K*bits/32]
  const uint16_t *s, *b;    // [E, N, K/g]
  const uint32_t *lhs, *rhs;
  int64_t P;
  int64_t N;
  int64_t Bx;
  int K;
  int M;
  int gshift;
  int tiles;                // row tiles per expert
  int tile_rows;            // rows per tile (a multiple of waves * 8)
  int res_offset;           // LDS bytes before the parked row sums
  int out_f32;
  void *y;                  // [P, M, N]
};

constexpr int kGatherListMax = 1024;   // pairs of one expert per window
#ifndef QMV_GATHER_SEG
#define QMV_GATHER_SEG 8
#endif
constexpr int kGatherSeg = QMV_GATHER_SEG;   // lanes per row (8, 16, 32 or 64)
constexpr int kGatherRows = kWave / kGatherSeg;   // rows per wave step

// The pairs routed to expert e, in increasing p whatever the order of rhs:
// a block-wide scan of rhs (per-wave ballots, counts meeting in LDS).  Fills
// list[i] = p and xrow[i] = lhs[p] for the pairs of ranks [win, win +
// kGatherListMax) and returns the number of pairs of e.  (An lhs index past
// Bx gives undefined results and is clamped, so x is never overread.)
// Every thread of the workgroup must call it; the result is uniform.
template <int GW>
__device__ __forceinline__ int route_pairs(const GatherArgs &a, int e, int win, int *list, int *xrow,
                                           int *wcnt) {
  constexpr int NT = GW * kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int seen = 0;
  for (int64_t p0 = 0; p0 < a.P; p0 += NT) {
    const int64_t p = p0 + threadIdx.x;
    const bool hit = p < a.P && a.rhs[p] == static_cast<uint32_t>(e);
    const unsigned long long mask = __ballot(hit);
    if (lane == 0) wcnt[wid] = __popcll(mask);
    __syncthreads();
    int before = seen + __popcll(mask & ((1ull << lane) - 1ull));
    int round = 0;
#pragma unroll
    for (int w = 0; w < GW; ++w) {
      const int cnt = wcnt[w];
      before += (w < wid) ? cnt : 0;
      round += cnt;
    }
    if (hit && before >= win && before < win + kGatherListMax) {
      list[before - win] = static_cast<int>(p);
      xrow[before - win] = static_cast<int>(min(static_cast<int64_t>(a.lhs[p]), a.Bx - 1));
    }
    seen += round;
    __syncthreads();
  }
  return seen;
}

template <int BITS, int MV, int GW, int DEPTH, int CPL>
__global__ __launch_bounds__(GW * kWave) void gather_kernel(GatherArgs a) {
  constexpr bool PAIR = BITS <= 6;
  constexpr int NT = GW * kWave;
  constexpr int SEG = kGatherSeg, R = kGatherRows, KS = SEG * CPL;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int list[kGatherListMax];    // pair index p, in increasing order
  __shared__ int xrow[kGatherListMax];    // its x batch row lhs[p]
  __shared__ int wcnt[GW];

  const int e = blockIdx.x / a.tiles;
  const int tile = blockIdx.x - e * a.tiles;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int u = lane & (SEG - 1), rl = lane / SEG;
  const int Kc = a.K >> 5;
  const int nks = (Kc + KS - 1) / KS;                        // steps per row group
  const int64_t wstride = static_cast<int64_t>(Kc) * BITS;   // words per row
  const int64_t gstride = Kc >> a.gshift;                    // groups per row
  const int64_t row_base = static_cast<int64_t>(tile) * a.tile_rows + wid * R;
  const int RG = a.tile_rows / (GW * R);
  const int T = RG * nks;
  const uint32_t *we = a.w + static_cast<int64_t>(e) * a.N * wstride;
  const uint16_t *se = a.s + static_cast<int64_t>(e) * a.N * gstride;
  const uint16_t *be = a.b + static_cast<int64_t>(e) * a.N * gstride;
  const PairConsts pk = pair_consts<BITS>();
  // Row sums are parked in LDS (RG * R * MV floats per wave) and written out
  // after the row loop: global stores inside it would share the memory
  // counter with the weight loads and force full waits on every step.
  float *res = reinterpret_cast<float *>(smem + a.res_offset) + wid * (RG * R * MV);

  // ---- the weight stream, through buffer resources that span this
  // expert's rows: a load past its last row returns zeros instead of
  // reading out of bounds, so the loads need no clamps or selects.  (Rows
  // past N, chunks past a row's end and steps past the wave's last are
  // loaded but never consumed.)  Every offset is in the VGPR operand, which
  // the range check covers; the host keeps one expert under 2 GiB.  Lane (rl, u) reads chunk u of row rl of the
  // step; the scalar step offsets advance by one K range per step and to
  // the next row group (GW*R rows on) on a wrap.
  const uint32_t cb = BITS * 4;                              // bytes per chunk
  const uint32_t wrow_b = static_cast<uint32_t>(wstride * 4), grow_b = static_cast<uint32_t>(gstride * 2);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(we), 0, static_cast<int>(a.N * wrow_b), kBufferDword3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(se), 0, static_cast<int>(a.N * grow_b), kBufferDword3);
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(be), 0, static_cast<int>(a.N * grow_b), kBufferDword3);
  const uint32_t lrow = static_cast<uint32_t>(row_base) + rl;
  const uint32_t wlane = lrow * wrow_b + u * cb;
  const uint32_t glane = lrow * grow_b + (static_cast<uint32_t>(u) >> a.gshift) * 2;
  const uint32_t w_wrap = GW * R * wrow_b - (nks - 1) * (KS * cb);
  const uint32_t g_wrap = GW * R * grow_b - (nks - 1) * ((KS >> a.gshift) * 2);
  uint32_t w_step = 0, g_step = 0;
  int l_t = 0, l_ks = 0;
  auto load_next = [&](ChunkStep<BITS, CPL> &st) {
    // Steps past the wave's last are pushed out of range (2 GiB on; every
    // lane offset is below that), so they cost no memory traffic.
    const bool live = l_t < T;
    const uint32_t ws = live ? w_step : 0x80000000u, gs = live ? g_step : 0x80000000u;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      buffer_load_chunk<BITS>(wrs, wlane + (ws + i * SEG * cb), st.w[i]);
      const uint32_t go = glane + (gs + ((i * SEG) >> a.gshift) * 2);
      st.s[i] = __builtin_amdgcn_raw_buffer_load_b16(srs, go, 0, 0);
      st.b[i] = __builtin_amdgcn_raw_buffer_load_b16(brs, go, 0, 0);
    }
    // advance by selects (increments in branches end up in scratch)
    const bool wrap = l_ks + 1 == nks;
    l_t += 1;
    l_ks = wrap ? 0 : l_ks + 1;
    w_step += wrap ? w_wrap : KS * cb;
    g_step += wrap ? g_wrap : (KS >> a.gshift) * 2;
  };
  auto restart = [&] {
    // the cursors restart from an opaque zero: otherwise the first steps'
    // offsets are hoisted out of the slab loop into VGPRs
    int zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
    l_t = zero;
    l_ks = zero;
    w_step = static_cast<uint32_t>(zero);
    g_step = static_cast<uint32_t>(zero);
  };
  ChunkStep<BITS, CPL> ring[DEPTH];
  // Every slab's ring prologue is issued after routing, so an expert that no
  // pair uses loads nothing.  (Issuing the first prologue before the scan,
  // to overlap their latencies, measured no faster on MI355X at 64 experts
  // of 2048x2048 4-bit, top-8 of 16 tokens: 39.5 against 39.7 us; and its
  // loads for the ~12% of experts left unrouted raised HBM traffic from
  // 1.018x to 1.039x of the algorithmic bytes.)
  bool primed = false;

  for (int win = 0;; win += kGatherListMax) {
    // ---- ordered list of the pairs routed to e, ranks [win, win + max)
    const int seen = route_pairs<GW>(a, e, win, list, xrow, wcnt);
    const int npairs = min(seen - win, kGatherListMax);
    if (npairs <= 0) return;                           // uniform
    const int nvec = npairs * a.M;

    for (int v0 = 0; v0 < nvec; v0 += MV) {
      const int nv = min(MV, nvec - v0);
      if (!primed) {
        restart();
        static_for<0, DEPTH>([&](auto d) { load_next(ring[decltype(d)::value]); });
      }
      primed = false;

      // ---- stage this slab's x vectors (issued after the weights: by the
      // time x arrives the weight prologue has landed too)
      const int items = nv * Kc;
      for (int it = threadIdx.x; it < items; it += NT) {
        const int mv = it / Kc, c = it - mv * Kc;
        const int vec = v0 + mv;
        const int pi = vec / a.M, m = vec - pi * a.M;
        const uint16_t *xk = a.x + (static_cast<int64_t>(xrow[pi]) * a.M + m) * a.K + static_cast<int64_t>(c) * 32;
        if constexpr (PAIR) stage_pairs_chunk<BITS, MV>(xk, smem, mv, c);
        else stage_f32_chunk<MV>(xk, smem, mv, c);
      }
      __syncthreads();

      // The slab's vector count is a compile-time constant below: the
      // products of absent vectors vanish instead of being branched over.
      auto slab = [&](auto nvc) {
        constexpr int NV = decltype(nvc)::value;
        float acc[1][MV], accz[1][MV];
#pragma unroll
        for (int m = 0; m < MV; ++m) acc[0][m] = accz[0][m] = 0.0f;

        int c_rg = 0, c_ks = 0;
        constexpr int kStride = chunk_stride_for<BITS, PAIR, MV>();
        const unsigned char *xlane = smem + u * kStride;    // this lane's first staged chunk
        auto consume = [&](const ChunkStep<BITS, CPL> &st) {
          const int left = Kc - c_ks * KS;                 // chunks of this K range that exist
          const unsigned char *xc = xlane + c_ks * (KS * kStride);
#pragma unroll
          for (int i = 0; i < CPL; ++i) {
            if (u + i * SEG < left) {
              if constexpr (PAIR) {
                gather_chunk_pairs<BITS, MV, NV>(st.w[i], st.s[i], st.b[i], xc + i * (SEG * kStride), pk, acc, accz);
              } else {
                ChunkStep<BITS, 1> one;
#pragma unroll
                for (int d = 0; d < BITS; ++d) one.w[0][d] = st.w[i][d];
                one.s[0] = st.s[i];
                one.b[0] = st.b[i];
                accumulate_chunk<BITS, 1, MV, PAIR>(one, xc + i * (SEG * kStride), NV, pk, acc, accz);
              }
            }
          }
          const bool last = c_ks == nks - 1;
          if (last) {                                      // row group complete
#pragma unroll
            for (int m = 0; m < NV; ++m) {
              float v = PAIR ? fmaf(acc[0][m], 1.0f / static_cast<float>(1 << PairPlan<BITS>::P), accz[0][m])
                             : acc[0][m];
              acc[0][m] = accz[0][m] = 0.0f;
              // segment sum, the same lane tree for every row and vector
              v = segment_sum<SEG>(v);
              if (u == 0) res[(c_rg * R + rl) * MV + m] = v;
            }
          }
          c_rg += last ? 1 : 0;
          c_ks = last ? 0 : c_ks + 1;
        };
        for (int t = 0; t < T; t += DEPTH) {
          static_for<0, DEPTH>([&](auto d) {
            constexpr int dd = decltype(d)::value;
            if (t + dd < T) consume(ring[dd]);
            load_next(ring[dd]);
          });
        }

        // ---- write out this wave's rows (its own LDS writes, in order)
        for (int i = lane; i < RG * R * MV; i += kWave) {
          const int g = i / (R * MV), idx = i - g * (R * MV);
          const int r = idx / MV, mv = idx - r * MV;
          const int64_t row = row_base + static_cast<int64_t>(g) * (GW * R) + r;
          if (mv < NV && row < a.N) {
            const int vec = v0 + mv;
            const int pi = vec / a.M, m = vec - pi * a.M;
            const int64_t o = (static_cast<int64_t>(list[pi]) * a.M + m) * a.N + row;
            if (a.out_f32) static_cast<float *>(a.y)[o] = res[i];
            else static_cast<uint16_t *>(a.y)[o] = f32_to_bf16(res[i]);
          }
        }
      };
      if constexpr (MV >= 4) { if (nv == 4) slab(std::integral_constant<int, 4>{}); }
      if constexpr (MV >= 3) { if (nv == 3) slab(std::integral_constant<int, 3>{}); }
      if constexpr (MV >= 2) { if (nv == 2) slab(std::integral_constant<int, 2>{}); }
      if (nv == 1) slab(std::integral_constant<int, 1>{});
      __syncthreads();   // LDS and list reuse by the next slab / window
    }
    if (seen <= win + kGatherListMax) return;
  }
}

}  // namespace qmvk
