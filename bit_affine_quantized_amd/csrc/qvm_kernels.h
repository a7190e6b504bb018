// qvm: the transpose = 0 product y[m, n] = sum_k x[m, k] * w_hat[k, n], with W
// packed along N: w_q [K, N*b/32], scales and biases [K, N/g] (mlx-metal
// quantized.h, qvm_impl and the split-K qvm kernel).
//
// Decomposition.  The contraction runs over the rows of W, so each row's
// codes feed 32 different outputs per chunk and no dot-product pairing
// applies: a lane owns one 32-column chunk and keeps 32 fp32 sums per x
// vector, each sum_k (x_k s_k) q_kn, plus one sum_k x_k z_k for the chunk's
// group (the affine fold with the roles of the axes swapped).
//
// A wave is C = 16 chunk lanes by 4 row streams; a workgroup (8 waves, 32
// streams) owns a block of 16 chunks (512 columns) over one K-slice.  Each
// stream loads its next R rows' chunks at once (all in flight), then
// accumulates them.  A wave first sums its 4 streams across lanes (a
// transposing butterfly: each lane ends with 8 of its chunk's 32 columns),
// then the 8 waves' sums meet in LDS in a fixed order.  With one slice the
// workgroup writes y; otherwise it writes its partial block to the workspace
// and a second kernel adds the S partials in slice order, so the result does
// not depend on scheduling.  (A last-workgroup-finishes
// handshake inside one kernel needs device-scope fences, which on a chip
// with one L2 per XCD write back and invalidate L2 in every workgroup; the
// kernel boundary pays that once.)
#pragma once

#include "qmv_device.h"

namespace qmvk {

struct QvmArgs {
  const uint16_t *x;        // [M, K] bf16 (this launch's vectors)
  const uint32_t *w;        // [K, N*bits/32]
  const uint16_t *s, *b;    // [K, N/g]
  float *part;              // [S, MV, N] partial sums (S > 1)
  void *y;                  // [M, N] (row stride y_ld)
  int64_t N;
  int64_t y_ld;
  int K;
  int M;                    // vectors in this launch (<= MV)
  int gshift;               // log2(group_size / 32)
  int S;                    // K-slices
  int ks;                   // rows per slice (a multiple of R * 32)
  int out_f32;
};

constexpr int kQvmC = 16;                    // chunk lanes per wave row
constexpr int kQvmWaves = 8;
constexpr int kQvmStreams = kQvmWaves * (kWave / kQvmC);   // 32
constexpr int kQvmCols = kQvmC * 32;         // 512 columns per block

constexpr int kQvmRow = kQvmCols + kQvmCols / 8;   // 576 floats: 36 per chunk

// Sum 32 values per lane over the 4 row streams of a wave (lane bits 5 and
// 4), halving the values at each step: lane l returns the totals of values
// 8*(l/16) .. 8*(l/16)+7 of its chunk lane l%16.
__device__ __forceinline__ void qvm_stream_sum(const float (&v)[32], float (&out)[8]) {
  float h[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = v[i], y = v[16 + i];
    swap32(x, y);                 // lanes < 32 keep values 0..15, the others 16..31
    h[i] = x + y;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float x = h[i], y = h[8 + i];
    swap16(x, y);                 // even rows keep the lower 8, odd rows the upper 8
    out[i] = x + y;
  }
}

template <int BITS, int MV, int R>
__global__ __launch_bounds__(kQvmWaves * kWave) void qvm_kernel(QvmArgs a) {
  constexpr int NT = kQvmWaves * kWave;
  // x slice (fp32) then the per-wave sums
  extern __shared__ __align__(16) unsigned char smem[];
  float *xs = reinterpret_cast<float *>(smem);                       // [MV][ks]
  float *red = xs + MV * a.ks;                                       // [8 waves][MV][576]

  const int64_t Nc = a.N >> 5;
  const int64_t CB = (Nc + kQvmC - 1) / kQvmC;
  // the column blocks of one K-slice share each row's scale and bias cache
  // lines: consecutive logical blocks (one slice's blocks) go to one XCD
  // (4096x4096 4-bit on MI355X, against the dispatch order: HBM traffic
  // 18.1 -> 10.7 MB, 8.70 -> 8.04 us at M = 1, 12.40 -> 11.41 us at M = 4)
  const int64_t blk = xcd_block(blockIdx.x, gridDim.x);
  const int64_t cb = blk % CB;
  const int sl = static_cast<int>(blk / CB);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ci = lane % kQvmC;
  const int stream = wid * (kWave / kQvmC) + lane / kQvmC;
  const int64_t chunk_raw = cb * kQvmC + ci;
  const int64_t chunk = chunk_raw < Nc ? chunk_raw : Nc - 1;   // tail lanes: clamped, discarded
  const int64_t wstride = Nc * BITS;                           // words per row
  const int64_t gstride = Nc >> a.gshift;                      // groups per row
  const int64_t gi = chunk >> a.gshift;
  const int k0 = sl * a.ks;
  const int k1 = min(a.K, k0 + a.ks);

  // ---- rows k0 + stream + 32 j in blocks of R rows per stream, all of a
  // block's loads in flight.  The first block's loads go out before x is
  // staged: they do not depend on it.
  uint32_t w[R][BITS];
  uint16_t sv[R], zv[R];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int k = kb + stream + r * kQvmStreams;
      k = k < a.K - 1 ? k : a.K - 1;             // past K: x reads 0 there
      load_chunk<BITS>(a.w + static_cast<int64_t>(k) * wstride + chunk * BITS, w[r]);
      sv[r] = a.s[static_cast<int64_t>(k) * gstride + gi];
      zv[r] = a.b[static_cast<int64_t>(k) * gstride + gi];
    }
  };
  load_block(k0);

  // ---- stage this slice's x as fp32 (rows past K read as 0)
  for (int i = threadIdx.x; i < MV * a.ks; i += NT) {
    const int m = i / a.ks, r = i - m * a.ks;
    const int k = k0 + r;
    xs[i] = (m < a.M && k < a.K) ? bf16_to_f32(a.x[static_cast<int64_t>(m) * a.K + k]) : 0.0f;
  }
  __syncthreads();

  float acc[MV][32], accz[MV];
#pragma unroll
  for (int m = 0; m < MV; ++m) {
    accz[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[m][i] = 0.0f;
  }

  for (int kb = k0; kb < k1; kb += R * kQvmStreams) {
    if (kb != k0) load_block(kb);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int kr = kb - k0 + stream + r * kQvmStreams;    // < ks
      const float sf = bf16_to_f32(sv[r]);
      const float zf = bf16_to_f32(zv[r]);
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        const float xv = xs[m * a.ks + kr];
        const float xsv = xv * sf;
        accz[m] = fmaf(xv, zf, accz[m]);
        static_for<0, 32>([&](auto i) {
          constexpr int I = decltype(i)::value;
          acc[m][I] = fmaf(xsv, code_f32<BITS, I>(w[r]), acc[m][I]);
        });
      }
    }
  }

  // ---- sum the wave's 4 streams across lanes, then the 8 waves in LDS in
  // wave order (rows of 512 columns padded by 4 floats per 32, so a lane's
  // 32-byte run starts on its own bank octet)
#pragma unroll
  for (int m = 0; m < MV; ++m) {
    float v[32], part[8];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = acc[m][i] + accz[m];
    qvm_stream_sum(v, part);
    float *dst = red + (wid * MV + m) * kQvmRow + ci * 36 + 8 * (lane / kQvmC);
    reinterpret_cast<float4 *>(dst)[0] = make_float4(part[0], part[1], part[2], part[3]);
    reinterpret_cast<float4 *>(dst)[1] = make_float4(part[4], part[5], part[6], part[7]);
  }
  __syncthreads();
  const int64_t col0 = cb * kQvmCols;
  auto store_y = [&](int m, int64_t n, float v) {
    const int64_t o = static_cast<int64_t>(m) * a.y_ld + n;
    if (a.out_f32) static_cast<float *>(a.y)[o] = v;
    else static_cast<uint16_t *>(a.y)[o] = f32_to_bf16(v);
  };
  for (int i = threadIdx.x; i < MV * kQvmCols; i += NT) {
    const int m = i / kQvmCols, c = i - m * kQvmCols;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kQvmWaves; ++w) v += red[(w * MV + m) * kQvmRow + (c >> 5) * 36 + (c & 31)];
    const int64_t n = col0 + c;
    if (a.S == 1) {
      if (m < a.M && n < a.N) store_y(m, n, v);
    } else if (n < a.N) {
      a.part[(static_cast<int64_t>(sl) * MV + m) * a.N + n] = v;
    }
  }
}

// y[m, n] = sum over slices t = 0..S-1, in order, of part[t, m, n].  Each
// batch of B slices is loaded at once (indices past S re-read slice S - 1,
// unused): the host picks the smallest B that covers S, so no batch issues
// loads it does not need (8 slices with B = 32 cost 24 wasted load
// instructions per output: 4096x4096 M = 64 on the matrix cores 17.97 ->
// 16.46 us with B = 8).
template <int B>
__global__ __launch_bounds__(256) void qvm_reduce_kernel(const float *__restrict__ part, int S,
                                                         int MVs, int M, int64_t N, int64_t y_ld,
                                                         int out_f32, void *__restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(M) * N) return;
  const int m = static_cast<int>(i / N);
  const int64_t n = i - static_cast<int64_t>(m) * N;
  const float *pp = part + static_cast<int64_t>(m) * N + n;
  const int64_t pstride = static_cast<int64_t>(MVs) * N;
  float v = 0.0f;
  for (int t0 = 0; t0 < S; t0 += B) {
    float p[B];
#pragma unroll
    for (int j = 0; j < B; ++j) p[j] = pp[static_cast<int64_t>(min(t0 + j, S - 1)) * pstride];
#pragma unroll
    for (int j = 0; j < B; ++j) v += (t0 + j < S) ? p[j] : 0.0f;
  }
  const int64_t o = static_cast<int64_t>(m) * y_ld + n;
  if (out_f32) static_cast<float *>(y)[o] = v;
  else static_cast<uint16_t *>(y)[o] = f32_to_bf16(v);
}

}  // namespace qmvk
