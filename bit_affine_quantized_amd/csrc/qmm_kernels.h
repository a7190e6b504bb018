// qmm: the transposed quantized product for several x rows at once (prefill
// and batched decode; mlx-metal quantized.h qmm_t), y[m, n] =
// sum_k x[m, k] * w_hat[n, k], on the matrix cores.
//
// The magic-bf16 codes of the matvec path carry over exactly: a b-bit code q
// placed in the top of a bf16 mantissa with exponent 2^7 is the bf16 value
// 128 + q * 2^P (P = 7 - b), so one v_mfma_f32_16x16x32_bf16 on a 32-code
// chunk gives D = 128 * X + 2^P * sum q x for 16 W rows by 16 x rows, X being
// the chunk's sum of x.  Chaining the chunks of a group and folding once per
// group, y = 2^-P s D + (z - 2^b s) X, with exact operands: products of bf16
// values are exact and the accumulation is fp32.  8-bit codes do not fit the
// 7-bit mantissa and are split into nibbles, q = lo + 16 hi, with one MFMA
// each: y = (s / 8)(D_lo + 16 D_hi) + (z - 272 s) X.
//
// The contraction order inside one MFMA is free, so the 32 k of a chunk are
// taken in the pairing order (8i + j, 8i + j + 4) for every bit width: lane
// group i (= lane / 16) of the B operand holds codes 8i..8i+7, read from a
// byte-aligned window of the chunk, and x is staged once per workgroup in the
// same order.  With 2-, 4- or 8-bit codes and groups of several chunks, the
// plain product instead gives each lane group one contiguous window per
// group (an MFMA's 32 codes may come from any chunks of one group).
//
// A workgroup (kQmmWaves waves) covers 16 W rows per wave by up to 64 x rows
// (BM m-tiles) over a slice of K; x is staged in LDS 8 chunks at a time.  A
// slice's fp32 result goes to y directly, or, with several slices, to the
// workspace, whose slices are then added in order by a second kernel.
#pragma once

#include "qmv_device.h"

namespace qmvk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct QmmArgs {
  const uint16_t *x;        // [M, K] bf16 (this launch's rows)
  const uint32_t *w;        // [N, K*bits/32]
  const uint16_t *s, *b;    // [N, K/g]
  float *part;              // [S, 16*BM, N] (S > 1)
  void *y;                  // [M, N] (row stride y_ld)
  int64_t N;
  int64_t y_ld;
  int K;
  int M;                    // x rows in this launch (<= 16*BM)
  int gshift;               // log2(group_size / 32)
  int S;                    // K-slices
  int cps;                  // chunks per slice (a multiple of kQmmKB)
  int out_f32;
};

#ifndef QMV_QMM_WAVES
#define QMV_QMM_WAVES 4
#endif
#ifndef QMV_QMM_KB
#define QMV_QMM_KB 8
#endif
constexpr int kQmmKB = QMV_QMM_KB; // chunks per staged K-block (a multiple of 4)
constexpr int kQmmRow = 80;        // bytes per staged (x row, chunk): 64 B of pairs + pad
constexpr int kQmmWaves = QMV_QMM_WAVES;         // waves per workgroup, 16 W rows each
constexpr int kQmmThreads = kQmmWaves * kWave;
constexpr int kQmmRowsPerWG = 16 * kQmmWaves;    // W rows per workgroup

template <int BM>
constexpr int qmm_lds_bytes() {
  return kQmmKB * 16 * BM * kQmmRow + kQmmKB * 16 * BM * 4;   // pairs + (at most per-chunk) sums
}

// Magic-bf16 B operand (4 dwords = 8 bf16) from the lane's window: pair j
// holds codes j (low half) and j + 4 (high half).
template <int BITS>
__device__ __forceinline__ void qmm_b_pairs(uint32_t w0, uint32_t w1, uint32_t shift,
                                            const PairConsts &pk, uint32_t (&p)[4]) {
  if constexpr (BITS == 4) {
    // codes j, j+4 are nibbles j, j+4 of one word: the matvec's 4-bit plan
    const uint32_t w[4] = {w0, w0, w0, w0};
    static_for<0, 4>([&](auto jj) {
      constexpr int J = decltype(jj)::value;
      p[J] = make_pair<4, J>(w, pk);
    });
  } else if constexpr (BITS == 2) {
    // 8 codes = 16 bits; spread codes 4..7 to the high half, then the
    // matvec's 2-bit plan (pair j = codes at bits 2j and 2j + 16)
    const uint32_t v = (w0 >> shift) & 0xFFFFu;
    const uint32_t t = (v & 0xFFu) | ((v & 0xFF00u) << 8);
    const uint32_t w[2] = {t, t};
    static_for<0, 4>([&](auto jj) {
      constexpr int J = decltype(jj)::value;
      p[J] = make_pair<2, J>(w, pk);
    });
  } else {
    constexpr int P = 7 - BITS;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    const uint64_t v = ((static_cast<uint64_t>(w1) << 32) | w0) >> shift;
    static_for<0, 4>([&](auto jj) {
      constexpr int J = decltype(jj)::value;
      const uint32_t lo = static_cast<uint32_t>(v >> (BITS * J)) & mask;
      const uint32_t hi = static_cast<uint32_t>(v >> (BITS * (J + 4))) & mask;
      p[J] = (lo << P) | (hi << (16 + P)) | pk.magic;
    });
  }
}

// 8-bit codes: nibble operands.  Pair j takes bytes j (of w0) and j (of w1),
// i.e. codes j and j + 4; `lo` holds their low nibbles, `hi` their high ones.
__device__ __forceinline__ void qmm_b_nibbles(uint32_t w0, uint32_t w1, const PairConsts &pk,
                                              uint32_t (&lo)[4], uint32_t (&hi)[4]) {
  static_for<0, 4>([&](auto jj) {
    constexpr int J = decltype(jj)::value;
    // bytes: out0 = w0.byte J, out2 = w1.byte J, out1 = out3 = 0
    constexpr uint32_t sel = (0x0Cu << 24) | ((4u + J) << 16) | (0x0Cu << 8) | J;
    const uint32_t t = __builtin_amdgcn_perm(w1, w0, sel);
    lo[J] = ((t << 3) & pk.mask) | pk.magic;
    hi[J] = ((t >> 1) & pk.mask) | pk.magic;
  });
}

// One workgroup's contribution over chunks [c0, c1) of W rows nb*64 .. +64
// (wave wid: 16 of them) and the 16*BM staged x rows: acc and accz per
// m-tile, lane layout of the MFMA result (rows 4*(lane/16) + e, column
// lane % 16).  `xoff(r, c)` is the byte offset from `x` of chunk c of staged
// row r (r < 16*BM, callers clamp it to a valid row).  Every thread of the
// workgroup must call this (it holds workgroup barriers).
template <int BITS, int BM, int CPG, int GW, bool SPANS, typename XOff>
__device__ __forceinline__ void qmm_accumulate(const uint32_t *__restrict__ w, const uint16_t *__restrict__ sp,
                                               const uint16_t *__restrict__ bp_, const uint16_t *__restrict__ x,
                                               uint32_t nrow, int Kc, int c0, int c1, XOff &&xoff,
                                               unsigned char *smem, f32x4_t (&acc)[BM], f32x4_t (&accz)[BM]) {
  constexpr int MR = 16 * BM;
  constexpr bool NIB = BITS == 8;
  constexpr float kZc = NIB ? 272.0f : static_cast<float>(1 << BITS);   // z - kZc * s
  constexpr int GPB = kQmmKB / CPG;               // groups per K-block
  unsigned char *xp = smem;                                       // [KB][MR][80]
  float *xsum = reinterpret_cast<float *>(smem + kQmmKB * MR * kQmmRow);   // [GPB][MR] group sums
  const int lane = threadIdx.x & (kWave - 1);
  const int j = lane & 15, kb = lane >> 4;
  const uint32_t gpr = static_cast<uint32_t>(Kc / CPG);           // groups per row
  // 32-bit byte offsets from the arrays' scalar bases (the host keeps every
  // array under 4 GiB for this path).  The lane's window of 8 codes
  // (8kb..8kb+7) starts at byte b*kb of a chunk (8-bit codes: at word 2kb);
  // a second word is read only when the codes cross a word boundary
  // (otherwise the first word is read again: never past the chunk), and
  // w_shift aligns the window to bit 0.
  const uint32_t wlane = nrow * static_cast<uint32_t>(Kc * BITS * 4) +
                         (NIB ? static_cast<uint32_t>(kb) * 8u : static_cast<uint32_t>(BITS * kb) & ~3u);
  const uint32_t w_second = NIB ? 4u : ((((BITS * kb) & 3) + BITS > 4) ? 4u : 0u);
  const uint32_t w_shift = NIB ? 0u : static_cast<uint32_t>((BITS * kb) & 3) * 8u;
  const PairConsts pk = pair_consts<NIB ? 4 : (BITS <= 6 ? BITS : 4)>();
  // Spans: with 2-, 4- or 8-bit codes and groups of two or more chunks, the
  // codes of one MFMA may come from any chunks of the group, so lane group
  // kb takes a contiguous window of SPAN * 8 codes (SPAN * b bytes at
  // SPAN * b * kb) from each span of SPAN = CPG chunks, and MFMA v of the
  // span contracts codes 8v..8v+7 of every window.  One load per span
  // instead of one per chunk: fewer cache-line requests per byte of W
  // (4096x4096 4-bit g64: M = 16 12.2 -> 10.3 us, M = 64 19.5 -> 18.5 us;
  // gathered, 64 experts of 2048x2048, top-8: 8 vectors per expert 85.1 ->
  // 64.8 us, 64 per expert 175.9 -> 152.7 us).
  constexpr int SPAN = (SPANS && (BITS == 2 || BITS == 4 || BITS == 8) && CPG >= 2) ? CPG : 1;
  constexpr int kWinDw = SPAN > 1 ? SPAN * BITS / 4 : 1;   // dwords per lane window
  const uint32_t wspan = nrow * static_cast<uint32_t>(Kc * BITS * 4) + static_cast<uint32_t>(SPAN * BITS * kb);

  f32x4_t D[BM], Dh[BM];
#pragma unroll
  for (int t = 0; t < BM; ++t) {
    acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    accz[t] = acc[t];
    D[t] = acc[t];
    Dh[t] = acc[t];
  }

  constexpr int kThreads = GW * kWave;
  for (int cb = c0; cb < c1; cb += kQmmKB) {
    // ---- this block's x chunks (rows [0, MR) x chunks [cb, cb + KB)) are
    // loaded first, then the weight windows, scales and biases: the memory
    // counter retires loads in order, so converting x waits for x alone and
    // the weights' latency overlaps the conversion.  Chunks past the range
    // restage a valid chunk (their products are never used).
    //
    // Each 64-byte chunk of a row is loaded by four adjacent lanes, 16 bytes
    // (one lane group's 8 codes) each, so that one load instruction covers
    // whole cache lines: piece p = (group, row, chunk, quarter), quarter
    // fastest.  The CPG chunks of a row's group then sit in adjacent quads,
    // and the group's x sum is formed across those lanes, once.  (Whole
    // chunks per lane read 32 bytes of a line per request: 193 -> 175 us on
    // the 512-token top-8 gather over 64 experts.)
    constexpr int kPieces = MR * kQmmKB * 4;
    static_assert(kPieces % kThreads == 0, "x pieces must divide evenly");
    constexpr int kPer = kPieces / kThreads;
    uint4 raw[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int pc = static_cast<int>(threadIdx.x) + i * kThreads;
      const int qq = pc & 3, it = pc >> 2;
      const int ch = it % CPG, rest = it / CPG;
      const int r = rest % MR, gg = rest / MR;
      raw[i] = *reinterpret_cast<const uint4 *>(
          byte_offset(x, xoff(r, min(cb + gg * CPG + ch, c1 - 1)) + static_cast<uint32_t>(qq * 16)));
    }
    // Plain loads, not non-temporal ones: a lane's window is a few bytes of
    // a row, and the block's chunks read the rest of the same cache lines,
    // which non-temporal loads would not keep (measured 13% slower at
    // 4096x4096, M = 16).
    uint32_t wa[kQmmKB], wb[kQmmKB];
    uint32_t win[kQmmKB / SPAN][kWinDw];
    if constexpr (SPAN > 1) {
#pragma unroll
      for (int sp = 0; sp < kQmmKB / SPAN; ++sp) {
        const uint32_t c = static_cast<uint32_t>(min(cb + sp * SPAN, c1 - SPAN));   // spans are whole
        const uint32_t *src = byte_offset(w, wspan + c * (BITS * 4));
        if constexpr (kWinDw == 1) {
          win[sp][0] = *src;
        } else if constexpr (kWinDw == 2) {
          const uint2 v = *reinterpret_cast<const uint2 *>(src);
          win[sp][0] = v.x; win[sp][1] = v.y;
        } else {
#pragma unroll
          for (int h = 0; h < kWinDw / 4; ++h) {
            const uint4 v = reinterpret_cast<const uint4 *>(src)[h];
            win[sp][4 * h] = v.x; win[sp][4 * h + 1] = v.y; win[sp][4 * h + 2] = v.z; win[sp][4 * h + 3] = v.w;
          }
        }
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < kQmmKB; ++cc) {
        const uint32_t c = static_cast<uint32_t>(min(cb + cc, c1 - 1));
        const uint32_t off = wlane + c * (BITS * 4);
        wa[cc] = *byte_offset(w, off);
        wb[cc] = *byte_offset(w, off + w_second);
      }
    }
    // Scales and biases: lane group kb loads those of the block's groups kb
    // and kb + 4 for its row, packed (scale low, bias high); the fold takes
    // group gg's from lane j + 16 (gg % 4).  One load instruction then
    // serves four groups of the 16 rows instead of one: each of these 2-byte
    // loads costs a cache-line request per row, and the requests, not the
    // bytes, set the pace (4096x4096, M = 16: 14.6 -> 12.1 us; the 512-token
    // top-8 gather over 64 experts: 254 -> 193 us).
    constexpr int kSzLoads = (GPB + 3) / 4;
    uint32_t sz[kSzLoads];
#pragma unroll
    for (int q = 0; q < kSzLoads; ++q) {
      const int gg = min(kb + 4 * q, GPB - 1);
      const uint32_t gi = static_cast<uint32_t>(min(cb + gg * CPG, c1 - 1)) / CPG;
      const uint32_t o = (nrow * gpr + gi) * 2u;
      sz[q] = static_cast<uint32_t>(*byte_offset(sp, o)) | (static_cast<uint32_t>(*byte_offset(bp_, o)) << 16);
    }
    __syncthreads();                              // the previous block's LDS reads are done
    // ---- convert to pair order into LDS.  Rows of one chunk are 80 bytes
    // apart, so a chunk's 16-byte stores do not collide on banks.
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int pc = static_cast<int>(threadIdx.x) + i * kThreads;
      const int qq = pc & 3, it = pc >> 2;
      const int ch = it % CPG, rest = it / CPG;
      const int r = rest % MR, gg = rest / MR;
      const uint4 v = raw[i];
      float sum = dot2_bf16(v.x, 0x3F803F80u, 0.0f);
      sum = dot2_bf16(v.y, 0x3F803F80u, sum);
      sum = dot2_bf16(v.z, 0x3F803F80u, sum);
      sum = dot2_bf16(v.w, 0x3F803F80u, sum);
      // the group's sum: the quad's quarters, then the quads of the group's
      // chunks (adjacent lanes)
      sum += dpp<kDppXor1>(sum);
      sum += dpp<kDppXor2>(sum);
      if constexpr (CPG >= 2) sum += dpp<kDppHalfMirror>(sum);
      if constexpr (CPG >= 4) sum += dpp<kDppRor8>(sum);
      // piece m of its span goes to the span's chunk m % SPAN, lane group
      // m / SPAN (with SPAN = 1: chunk ch, lane group qq)
      const int m = 4 * (ch % SPAN) + qq;
      const int vch = ch - ch % SPAN + m % SPAN;
      unsigned char *dst = xp + ((gg * CPG + vch) * MR + r) * kQmmRow + (m / SPAN) * 16;
      // pair e = (x[e], x[e + 4]) of the piece's 8 values
      *reinterpret_cast<uint4 *>(dst) = make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                                                   __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                                                   __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                                                   __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
      if (ch == 0 && qq == 0) xsum[gg * MR + r] = sum;
    }
    __syncthreads();

    static_for<0, kQmmKB>([&](auto ccv) {
      constexpr int cc = decltype(ccv)::value;
      constexpr bool first = cc % CPG == 0, last = cc % CPG == CPG - 1;
      if (cb + cc < c1) {                         // uniform; groups are whole
        uint32_t bq[4], bh[4];
        if constexpr (SPAN > 1) {
          constexpr int spi = cc / SPAN, v = cc % SPAN;
          if constexpr (BITS == 4) qmm_b_pairs<4>(win[spi][v], win[spi][v], 0u, pk, bq);
          else if constexpr (BITS == 8) qmm_b_nibbles(win[spi][2 * v], win[spi][2 * v + 1], pk, bq, bh);
          else qmm_b_pairs<2>(win[spi][v / 2], 0u, 16u * (v & 1), pk, bq);
        } else if constexpr (NIB) {
          qmm_b_nibbles(wa[cc], wb[cc], pk, bq, bh);
        } else {
          qmm_b_pairs<BITS>(wa[cc], wb[cc], w_shift, pk, bq);
        }
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, make_uint4(bq[0], bq[1], bq[2], bq[3]));
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < BM; ++t) {
          const uint4 av = *reinterpret_cast<const uint4 *>(xp + (cc * MR + t * 16 + j) * kQmmRow + kb * 16);
          const bf16x8_t A = __builtin_bit_cast(bf16x8_t, av);
          D[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, first ? zero : D[t], 0, 0, 0);
          if constexpr (NIB) {
            const bf16x8_t Bh = __builtin_bit_cast(bf16x8_t, make_uint4(bh[0], bh[1], bh[2], bh[3]));
            Dh[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bh, first ? zero : Dh[t], 0, 0, 0);
          }
        }
        if constexpr (last) {                     // fold the group
          constexpr int gg = cc / CPG;
          const uint32_t szv = static_cast<uint32_t>(
              __builtin_amdgcn_ds_bpermute((j + 16 * (gg % 4)) * 4, static_cast<int>(sz[gg / 4])));
          const float s = __builtin_bit_cast(float, szv << 16);
          const float zc = fmaf(-kZc, s, __builtin_bit_cast(float, szv & 0xFFFF0000u));
#pragma unroll
          for (int t = 0; t < BM; ++t) {
            const float4 xg = *reinterpret_cast<const float4 *>(xsum + (cc / CPG) * MR + t * 16 + 4 * kb);
            const float xgv[4] = {xg.x, xg.y, xg.z, xg.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float d = NIB ? fmaf(16.0f, Dh[t][e], D[t][e]) : D[t][e];
              acc[t][e] = fmaf(s, d, acc[t][e]);
              accz[t][e] = fmaf(zc, xgv[e], accz[t][e]);
            }
          }
        }
      }
    });
  }
}

template <int BITS, int BM, int CPG>
__global__ __launch_bounds__(kQmmThreads) void qmm_kernel(QmmArgs a) {
  constexpr int MR = 16 * BM;                     // x rows per launch
  constexpr int P = BITS == 8 ? 3 : 7 - BITS;
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int j = lane & 15, kb = lane >> 4;
  const int64_t NB = (a.N + kQmmRowsPerWG - 1) / kQmmRowsPerWG;
  // dispatch order: with NB a multiple of 8 the K-slices of one row block
  // run on one XCD and share its scale and bias cache lines (giving one
  // slice's row blocks to one XCD instead, so that they share x, measured
  // worse on MI355X: 4096x4096 4-bit M = 8, 9.05 -> 9.44 us and 13.3 -> 20.2
  // MB of HBM traffic)
  const int64_t nb = blockIdx.x % NB;
  const int sl = static_cast<int>(blockIdx.x / NB);
  const int64_t n = nb * kQmmRowsPerWG + wid * 16 + j;
  const uint32_t nrow = static_cast<uint32_t>(n < a.N ? n : a.N - 1);   // rows past N: not stored
  const int Kc = a.K >> 5;
  const int c0 = sl * a.cps;
  const int c1 = min(Kc, c0 + a.cps);
  // rows past M restage row M - 1: their outputs are never stored
  auto xoff = [&](int r, int c) { return static_cast<uint32_t>(min(r, a.M - 1) * a.K + c * 32) * 2u; };
  f32x4_t acc[BM], accz[BM];
  qmm_accumulate<BITS, BM, CPG, kQmmWaves, true>(a.w, a.s, a.b, a.x, nrow, Kc, c0, c1, xoff, smem, acc, accz);

  // ---- lane holds rows 4*kb + e of each m-tile, column n
  constexpr float kInvP = 1.0f / static_cast<float>(1 << P);
#pragma unroll
  for (int t = 0; t < BM; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = t * 16 + 4 * kb + e;
      const float v = fmaf(acc[t][e], kInvP, accz[t][e]);
      if (n < a.N) {
        if (a.S == 1) {
          if (m < a.M) {
            const int64_t o = static_cast<int64_t>(m) * a.y_ld + n;
            if (a.out_f32) static_cast<float *>(a.y)[o] = v;
            else static_cast<uint16_t *>(a.y)[o] = f32_to_bf16(v);
          }
        } else {
          a.part[(static_cast<int64_t>(sl) * MR + m) * a.N + n] = v;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Gathered matrix-core product (gather_qmv with many tokens per expert):
// workgroup (e, nb) routes the pairs of expert e with the same ordered
// ballot scan as the matvec gather, then takes their x vectors 64 at a time
// through qmm_accumulate against W rows nb*64 .. +64 of expert e and
// scatters the results to y[p].  Lists longer than 1024 pairs are served in
// windows.
// ----------------------------------------------------------------------------
struct GatherQmmArgs {
  const uint16_t *x;        // [Bx, M, K]
  const uint32_t *w;        // [E, N, K*bits/32]
  const uint16_t *s, *b;    // [E, N, K/g]
  const uint32_t *lhs, *rhs;
  int64_t P;
  int64_t N;
  int64_t Bx;
  int K;
  int M;
  int out_f32;
  int slabs;                // workgroups per (expert, row block): slab s takes
                            // x vectors [64 s, 64 s + 64), [64 (s + slabs), ...), ...
  void *y;                  // [P, M, N]
};

constexpr int kGqmmListMax = 1024;
// Waves per gathered workgroup (16 W rows each): twice the plain product's,
// so each staged block of routed x serves 128 W rows (512 tokens x top-8
// over 64 experts of 2048x2048 on MI355X: 311 -> 280 us; the plain product
// measured 4-7% slower with 8).
#ifndef QMV_GQMM_WAVES
#define QMV_GQMM_WAVES 8
#endif
constexpr int kGqmmWaves = QMV_GQMM_WAVES;
constexpr int kGqmmThreads = kGqmmWaves * kWave;
constexpr int kGqmmRowsPerWG = 16 * kGqmmWaves;

template <int BITS, int CPG, int BM>
// At least 4 waves per SIMD (at most 128 VGPRs): with 64-vector slabs the
// kernel otherwise takes 129 and only one 8-wave workgroup fits per CU.
// 8-bit codes (two MFMAs per chunk) would spill under that cap and keep the
// compiler's choice.
__global__ __launch_bounds__(kGqmmThreads) __attribute__((amdgpu_waves_per_eu(BITS == 8 ? 1 : 4)))
void gather_qmm_kernel(GatherQmmArgs a) {
  constexpr int MR = 16 * BM;                     // x vectors per slab
  constexpr int P = BITS == 8 ? 3 : 7 - BITS;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int list[kGqmmListMax];
  __shared__ int xrow[kGqmmListMax];
  __shared__ uint32_t rowoff[MR];                  // x byte offset of each staged row
  __shared__ int wcnt[kGqmmWaves];

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int kb = lane >> 4;
  const int64_t NB = (a.N + kGqmmRowsPerWG - 1) / kGqmmRowsPerWG;
  // slab index outermost: every expert's first slab is dispatched first
  const int64_t per_slab = gridDim.x / a.slabs;
  const int sidx = static_cast<int>(blockIdx.x / per_slab);
  const int64_t rest = blockIdx.x - sidx * per_slab;
  const int e = static_cast<int>(rest / NB);
  const int64_t nb = rest % NB;
  const int64_t n = nb * kGqmmRowsPerWG + wid * 16 + (lane & 15);
  const uint32_t nrow = static_cast<uint32_t>(n < a.N ? n : a.N - 1);
  const int Kc = a.K >> 5;
  const int64_t wrows = static_cast<int64_t>(e) * a.N;
  const uint32_t *we = a.w + wrows * (static_cast<int64_t>(Kc) * BITS);
  const uint16_t *se = a.s + wrows * (Kc / CPG);
  const uint16_t *be = a.b + wrows * (Kc / CPG);

  for (int win = 0;; win += kGqmmListMax) {
    // ---- ordered list of the pairs routed to e, ranks [win, win + max).
    // Each thread takes a contiguous run of kRun pairs (its loads issued
    // together), counts its hits, and a block-wide exclusive scan of the
    // counts gives its first rank: ranks follow p whatever the order of rhs.
    constexpr int kRun = 16;
    int seen = 0;
    for (int64_t base = 0; base < a.P; base += static_cast<int64_t>(kGqmmThreads) * kRun) {
      const int64_t p0 = base + static_cast<int64_t>(threadIdx.x) * kRun;
      uint32_t hits = 0;
#pragma unroll
      for (int r = 0; r < kRun; ++r) {
        const int64_t p = p0 + r;
        if (p < a.P && a.rhs[p] == static_cast<uint32_t>(e)) hits |= 1u << r;
      }
      const int cnt = __popc(hits);
      // inclusive scan over the wave, then over the waves
      int incl = cnt;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += v;
      }
      if (lane == kWave - 1) wcnt[wid] = incl;
      __syncthreads();
      int before = seen + incl - cnt;
      int round = 0;
#pragma unroll
      for (int w = 0; w < kGqmmWaves; ++w) {
        const int c = wcnt[w];
        before += (w < wid) ? c : 0;
        round += c;
      }
      while (hits) {
        const int r = __ffs(hits) - 1;
        hits &= hits - 1u;
        if (before >= win && before < win + kGqmmListMax) {
          const int64_t p = p0 + r;
          list[before - win] = static_cast<int>(p);
          xrow[before - win] = static_cast<int>(min(static_cast<int64_t>(a.lhs[p]), a.Bx - 1));
        }
        ++before;
      }
      seen += round;
      __syncthreads();
    }
    const int npairs = min(seen - win, kGqmmListMax);
    if (npairs <= 0) return;                       // uniform
    const int nvec = npairs * a.M;

    for (int v0 = sidx * MR; v0 < nvec; v0 += MR * a.slabs) {
      const int nv = min(MR, nvec - v0);
      if (threadIdx.x < MR) {
        const int vec = v0 + min(static_cast<int>(threadIdx.x), nv - 1);   // past nv: restage the last
        const int pi = vec / a.M, m = vec - pi * a.M;
        rowoff[threadIdx.x] = static_cast<uint32_t>((xrow[pi] * a.M + m) * a.K) * 2u;
      }
      __syncthreads();
      auto xoff = [&](int r, int c) { return rowoff[r] + static_cast<uint32_t>(c) * 64u; };
      f32x4_t acc[BM], accz[BM];
      qmm_accumulate<BITS, BM, CPG, kGqmmWaves, true>(we, se, be, a.x, nrow, Kc, 0, Kc, xoff, smem, acc, accz);

      constexpr float kInvP = 1.0f / static_cast<float>(1 << P);
#pragma unroll
      for (int t = 0; t < BM; ++t) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = t * 16 + 4 * kb + q;
          if (r < nv && n < a.N) {
            const int vec = v0 + r;
            const int pi = vec / a.M, m = vec - pi * a.M;
            const float v = fmaf(acc[t][q], kInvP, accz[t][q]);
            const int64_t o = (static_cast<int64_t>(list[pi]) * a.M + m) * a.N + n;
            if (a.out_f32) static_cast<float *>(a.y)[o] = v;
            else static_cast<uint16_t *>(a.y)[o] = f32_to_bf16(v);
          }
        }
      }
      __syncthreads();                             // rowoff / LDS reuse by the next slab
    }
    if (seen <= win + kGqmmListMax) return;
  }
}

}  // namespace qmvk
