// Measurement references for bench.py (libqmv_bench.so; not part of the
// matvec library and never called by it).
//
// qmv_bench_read streams `bytes` bytes of device memory once: each wave
// reads one contiguous 4 KB block, four 16-byte non-temporal loads per lane
// all in flight together, and folds them with XOR.  This was the fastest
// one-launch streaming read found on MI355X for 33 MB (against grid-
// interleaved blocks, grid-stride persistent loops, 1-16 loads per lane and
// 256-1024 threads per workgroup).  With store_every > 0 the kernel also
// writes one 16-bit value per `store_every` bytes read, as a matvec writes
// one bf16 per row: the time of a read of the weight stream that also
// produces the output.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kLoads = 4;          // 16-byte loads per lane
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4_t *__restrict__ p, uint32_t n16,
                                                      uint16_t *out, uint32_t store_every16,
                                                      uint32_t n_out) {
  const uint32_t wave = (blockIdx.x * kThreads + threadIdx.x) / 64;
  const uint32_t lane = threadIdx.x & 63;
  u32x4_t v[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const uint32_t idx = min(wave * (kLoads * 64) + i * 64 + lane, n16 - 1);
    v[i] = __builtin_nontemporal_load(p + idx);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (store_every16 == 0) {
    // never true for real data patterns; keeps the loads live without a store
    if (acc == 0x9E3779B9u && out) out[0] = static_cast<uint16_t>(acc);
    return;
  }
  // one output per store_every16 16-byte units: lane 0 of each 64-lane group
  // of the wave's 256 units writes the outputs that fall in its block
  const uint32_t first = wave * (kLoads * 64);
  for (uint32_t o = (first + store_every16 - 1) / store_every16;
       o * store_every16 < first + kLoads * 64 && o < n_out; ++o) {
    if (lane == 0) out[o] = static_cast<uint16_t>(acc);
  }
}

// The read above split the way a matvec must read it: the weight words as
// one stream and the scales and biases as two more arrays, each wave taking
// `rows_per_wave` whole rows of all three (four 16-byte loads per lane of
// weight words, one 4-byte load per lane of each of the other two), then one
// 16-bit store per row.
__global__ __launch_bounds__(kThreads) void read3_kernel(const u32x4_t *__restrict__ w,
                                                       const uint32_t *__restrict__ s,
                                                       const uint32_t *__restrict__ b, uint32_t n16,
                                                       uint32_t nsb4, uint32_t sb4_per_wave,
                                                       uint32_t rows_per_wave, uint16_t *out,
                                                       uint32_t n_out) {
  const uint32_t wave = (blockIdx.x * kThreads + threadIdx.x) / 64;
  const uint32_t lane = threadIdx.x & 63;
  u32x4_t v[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const uint32_t idx = min(wave * (kLoads * 64) + i * 64 + lane, n16 - 1);
    v[i] = __builtin_nontemporal_load(w + idx);
  }
  const uint32_t j = min(wave * sb4_per_wave + min(lane, sb4_per_wave - 1), nsb4 - 1);
  uint32_t acc = s[j] ^ b[j];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  // every lane's loads must stay live (a store of acc by the row lanes only
  // would let the compiler issue the loads for those lanes alone), so acc
  // goes through a never-true test; the row lanes then write y
  if (acc == 0x9E3779B9u) out[0] = static_cast<uint16_t>(lane);
  if (lane < rows_per_wave) {
    const uint32_t o = wave * rows_per_wave + lane;
    if (o < n_out) out[o] = static_cast<uint16_t>(o);
  }
}

}  // namespace

extern "C" {

// Returns 0, or -1 for bad arguments, -3 if the launch failed.
int qmv_bench_read(const void *buf, uint64_t bytes, void *out, uint64_t store_every, void *stream) {
  if (!buf || bytes < 16 || bytes / 16 > 0xFFFFFFFFull) return -1;
  if (store_every && (!out || store_every % 16 != 0)) return -1;
  const uint32_t n16 = static_cast<uint32_t>(bytes / 16);
  const uint32_t per_block = kLoads * kThreads;
  const uint32_t blocks = (n16 + per_block - 1) / per_block;
  const uint32_t every16 = static_cast<uint32_t>(store_every / 16);
  const uint32_t n_out = every16 ? (n16 + every16 - 1) / every16 : 0;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t *>(buf), n16, static_cast<uint16_t *>(out), every16, n_out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Streams w_bytes of weight words and sb_bytes of each of two more arrays
// (scales, biases) as `rows` rows, writing one 16-bit value per row.  Each
// wave takes 4 KB of weight words, so a row must be at most 4 KB with 4 KB a
// multiple of it; a row's share of the other arrays must be a multiple of 4
// bytes, at most 256 bytes per wave.  Returns 0, -1 for bad arguments, -3 if
// the launch failed.
int qmv_bench_read3(const void *w, uint64_t w_bytes, const void *s, const void *b, uint64_t sb_bytes,
                    uint64_t rows, void *out, void *stream) {
  if (!w || !s || !b || !out || rows == 0 || w_bytes % rows || sb_bytes % rows) return -1;
  const uint64_t row_w = w_bytes / rows, row_sb = sb_bytes / rows;
  const uint64_t wave_w = static_cast<uint64_t>(kLoads) * 64 * 16;
  if (row_w == 0 || row_w > wave_w || wave_w % row_w || row_sb % 4) return -1;
  const uint64_t rows_per_wave = wave_w / row_w;
  const uint64_t sb4_per_wave = rows_per_wave * row_sb / 4;
  if (sb4_per_wave == 0 || sb4_per_wave > 64 || rows_per_wave > 64 || w_bytes / 16 > 0xFFFFFFFFull) return -1;
  const uint32_t n16 = static_cast<uint32_t>(w_bytes / 16);
  const uint64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
  const uint32_t blocks = static_cast<uint32_t>((waves + kThreads / 64 - 1) / (kThreads / 64));
  hipLaunchKernelGGL(read3_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t *>(w), static_cast<const uint32_t *>(s),
                     static_cast<const uint32_t *>(b), n16, static_cast<uint32_t>(sb_bytes / 4),
                     static_cast<uint32_t>(sb4_per_wave), static_cast<uint32_t>(rows_per_wave),
                     static_cast<uint16_t *>(out), static_cast<uint32_t>(rows));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
