// C ABI of libqmv.so (declared in include/qmv.h): host-side validation,
// kernel selection and launch.  Validation happens before any HIP call, so
// every argument error is reported without touching a device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "qmv.h"
#include "pack_kernels.h"
#include "qmv_kernels.h"
#include "qmv_line_kernels.h"
#include "qvm_kernels.h"
#include "qmm_kernels.h"
#include "qmf_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return QMV_OK;
}

int check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QMV_EHIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int64_t kMaxLds = 160 * 1024;   // gfx950 LDS per workgroup

bool bits_ok(int bits) {
  return bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 6 || bits == 8;
}
bool group_ok(int g) { return g == 32 || g == 64 || g == 128; }
int gshift_of(int g) { return g == 32 ? 0 : g == 64 ? 1 : 2; }

// Shape rules shared by every product (mlx/ops.cpp, extract_quantized_matmul_dims:
// w is uint32 with K*bits/32 words per row and K/group_size scales per row).
// `packed` is the axis the codes and groups run along (K for the usual
// x @ W^T; N for transpose = 0), `other` the remaining axis of W.
int check_shape(const char *fn, int64_t other, const char *other_name, int64_t packed,
                const char *packed_name, int group_size, int bits) {
  if (!bits_ok(bits)) return fail(QMV_EINVAL, "%s: bits=%d not in {2,3,4,5,6,8}", fn, bits);
  if (!group_ok(group_size))
    return fail(QMV_EINVAL, "%s: group_size=%d not in {32,64,128}", fn, group_size);
  if (other <= 0 || packed <= 0)
    return fail(QMV_EINVAL, "%s: %s=%lld and %s=%lld must be positive", fn, other_name,
                (long long)other, packed_name, (long long)packed);
  if (packed % group_size != 0)
    return fail(QMV_EINVAL, "%s: %s=%lld is not a multiple of group_size=%d", fn, packed_name,
                (long long)packed, group_size);
  if (packed > (int64_t(1) << 30) || other > (int64_t(1) << 40))
    return fail(QMV_EINVAL, "%s: %s=%lld or %s=%lld too large", fn, packed_name, (long long)packed,
                other_name, (long long)other);
  return QMV_OK;
}

int check_common(const char *fn, int64_t N, int64_t K, int group_size, int bits) {
  return check_shape(fn, N, "N", K, "K", group_size, bits);
}

// The kernels read x (and gate/up) and packed rows with 16-byte vector loads.
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_aligned(const char *fn, const void *p, const char *name) {
  if (!aligned16(p)) return fail(QMV_EINVAL, "%s: %s must be 16-byte aligned", fn, name);
  return QMV_OK;
}

template <typename Kern>
void allow_lds(Kern kern, int64_t bytes) {
  if (bytes > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

// ------------------------------------------------------------------ qmv family
#ifndef QMV_RPW
#define QMV_RPW 2
#endif
constexpr int kRpw = QMV_RPW;

#ifndef QMV_FORCE_WPB
#define QMV_FORCE_WPB 0   // 4 or 8 forces the waves per workgroup; 0 chooses by LDS
#endif

#ifndef QMV_SMALL_ROWS
// At most this many rows: one row per wave in 8-wave workgroups, so that a
// small matrix still fills the wave slots (4096x4096 4-bit on MI355X, one
// vector: 4.46 -> 4.20 us; at 14336 rows two rows per wave stay faster).
#define QMV_SMALL_ROWS 4096
#endif

template <int BITS, int MV, int XIN, int WPB, int RPW = kRpw>
int launch_qmv_wpb(const qmvk::QmvArgs &a, int64_t lds, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(a.nmat) * a.N;
  const int64_t rows_per_block = WPB * RPW;
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7FFFFFFF) return fail(QMV_EUNSUPPORTED, "qmv: too many rows");
  auto kern = qmvk::qmv_kernel<BITS, RPW, MV, XIN, WPB>;
  allow_lds(kern, lds);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(WPB * qmvk::kWave),
                     static_cast<size_t>(lds), st, a);
  return check_launch("qmv");
}

// Every workgroup stages the whole of x in LDS, so with a large K (or several
// vectors) few workgroups fit on a CU.  8-wave workgroups then keep more of
// the CU's wave slots filled and give more threads to the staging (measured
// on MI355X: 4096x14336 silu tail 17.2 -> 15.0 us, 4 vectors at 4096x4096
// 6.6 -> 6.0 us; 16-wave workgroups were slower everywhere).
int qmv_waves_per_block(int64_t lds) {
  if (QMV_FORCE_WPB) return QMV_FORCE_WPB;
  const int64_t per_cu = lds > 0 ? kMaxLds / lds : 32;
  return per_cu * 4 >= 32 ? 4 : 8;
}

// One x vector and at most two 64-lane chunk steps per row (K <= 4096): the
// straight-line kernel (qmv_line_kernels.h), same shapes as the loop kernel.
template <int BITS, int RPW, int WPB, int CPL>
int launch_line_t(const qmvk::QmvArgs &a, int64_t lds, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(a.nmat) * a.N;
  const int64_t blocks = (rows + WPB * RPW - 1) / (WPB * RPW);
  if (blocks > 0x7FFFFFFF) return fail(QMV_EUNSUPPORTED, "qmv: too many rows");
  const bool full = (a.K / 32) == CPL * qmvk::kWave;
  auto kern = full ? qmvk::qmv_line_kernel<BITS, RPW, WPB, CPL, true>
                   : qmvk::qmv_line_kernel<BITS, RPW, WPB, CPL, false>;
  allow_lds(kern, lds);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(WPB * qmvk::kWave),
                     static_cast<size_t>(lds), st, a);
  return check_launch("qmv");
}

template <int BITS, int RPW, int WPB>
int launch_line_cpl(const qmvk::QmvArgs &a, int64_t lds, hipStream_t st) {
  if (a.K / 32 <= qmvk::kWave) return launch_line_t<BITS, RPW, WPB, 1>(a, lds, st);
  return launch_line_t<BITS, RPW, WPB, 2>(a, lds, st);
}

template <int BITS, int MV, int XIN>
int launch_qmv_t(const qmvk::QmvArgs &a, hipStream_t st) {
  constexpr bool PAIR = (BITS <= 6) && (XIN == qmvk::XIN_PLAIN);
  const int64_t Kc = a.K / 32;
  const int64_t lds = Kc * qmvk::chunk_stride_for<BITS, PAIR, (XIN == qmvk::XIN_SILU ? 1 : MV)>();
  if constexpr (XIN == qmvk::XIN_PLAIN && MV == 1) {
    if (Kc <= 2 * qmvk::kWave && !QMV_FORCE_WPB) {
      if (static_cast<int64_t>(a.nmat) * a.N <= QMV_SMALL_ROWS) return launch_line_cpl<BITS, 1, 8>(a, lds, st);
      return launch_line_cpl<BITS, kRpw, 4>(a, lds, st);
    }
  }
  if constexpr (XIN == qmvk::XIN_PLAIN) {
    // one row per wave; 4-vector slabs in 16-wave workgroups (one per CU at
    // 4096 rows: 4096x4096 4-bit, 4 rows of x, on MI355X 5.70-5.75 ->
    // 5.59-5.61 us against 8 waves, 7.3-7.5 with 4)
    if (static_cast<int64_t>(a.nmat) * a.N <= QMV_SMALL_ROWS && !QMV_FORCE_WPB)
      return launch_qmv_wpb<BITS, MV, XIN, (MV == 4 ? 16 : 8), 1>(a, lds, st);
  }
  if (qmv_waves_per_block(lds) == 4) return launch_qmv_wpb<BITS, MV, XIN, 4>(a, lds, st);
  return launch_qmv_wpb<BITS, MV, XIN, 8>(a, lds, st);
}

template <int MV, int XIN>
int launch_qmv_bits(int bits, const qmvk::QmvArgs &a, hipStream_t st) {
  switch (bits) {
    case 2: return launch_qmv_t<2, MV, XIN>(a, st);
    case 3: return launch_qmv_t<3, MV, XIN>(a, st);
    case 4: return launch_qmv_t<4, MV, XIN>(a, st);
    case 5: return launch_qmv_t<5, MV, XIN>(a, st);
    case 6: return launch_qmv_t<6, MV, XIN>(a, st);
    case 8: return launch_qmv_t<8, MV, XIN>(a, st);
  }
  return fail(QMV_EINVAL, "bits=%d", bits);
}

int64_t qmv_lds_bytes(int bits, int mv, int64_t K) {
  const bool pair = bits <= 6;
  const bool two = bits == 3 || bits == 5;   // second chunk sum (PairPlan)
  return (K / 32) * (mv * (pair ? 64 : 128) + (two ? 48 : 16));
}

// ------------------------------------------------------------------ gather
#ifndef QMV_GATHER_WAVES
#define QMV_GATHER_WAVES 4
#endif
#ifndef QMV_GATHER_DEPTH
#define QMV_GATHER_DEPTH 2
#endif
#ifndef QMV_GATHER_CPL
#define QMV_GATHER_CPL 1          // chunks per lane per step (at most 2 for 5- to 8-bit codes)
#endif
#ifndef QMV_GATHER_TILES
#define QMV_GATHER_TILES 2048     // target workgroups over the whole expert stack
#endif
template <int BITS>
constexpr int gather_cpl() { return BITS <= 4 ? QMV_GATHER_CPL : (QMV_GATHER_CPL < 2 ? QMV_GATHER_CPL : 2); }
constexpr int64_t kGatherTiles = QMV_GATHER_TILES;
constexpr int kGatherWaves = QMV_GATHER_WAVES;
constexpr int kGatherDepth = QMV_GATHER_DEPTH;   // steps in flight per wave
// x vectors per pass over an expert's rows (fp32 staging is twice as wide)
#ifndef QMV_GATHER_MV
#define QMV_GATHER_MV 4           // x vectors per pass (fp32 staging: at most 2)
#endif
template <int BITS>
constexpr int gather_mv() { return BITS <= 6 ? QMV_GATHER_MV : (QMV_GATHER_MV < 2 ? QMV_GATHER_MV : 2); }
// static LDS of the gather kernel: pair list, x rows, per-wave counts
constexpr int64_t kGatherStaticLds = 2 * 4 * qmvk::kGatherListMax + 4 * kGatherWaves;

template <int BITS>
int launch_gather_t(const qmvk::GatherArgs &a0, int64_t E, hipStream_t st) {
  constexpr int kGatherMv = gather_mv<BITS>();
  qmvk::GatherArgs a = a0;
  const int64_t Kc = a.K / 32;
  const int64_t lds_x = Kc * qmvk::chunk_stride_for<BITS, (BITS <= 6), kGatherMv>();
  // Tiles of `tile_rows` rows: many small workgroups (~8 per CU over the
  // expert stack), so that most of the weight stream is in flight at once,
  // yet enough rows per tile that routing and x staging are paid once per
  // many rows; the parked row sums (tile_rows * MV floats) must fit in LDS
  // beside x and the pair list.  (64x2048x2048 4-bit, 128 pairs on MI355X:
  // 2048 tiles measured 7-10% ahead of 1024 or 4096.)
  const int64_t unit = kGatherWaves * qmvk::kGatherRows;
  int64_t tile_rows = (a.N * E + kGatherTiles - 1) / kGatherTiles;
  tile_rows = ((tile_rows + unit - 1) / unit) * unit;
  const int64_t n_round = ((a.N + unit - 1) / unit) * unit;
  if (tile_rows > n_round) tile_rows = n_round;
  if (tile_rows > 4096) tile_rows = 4096;
  if (tile_rows < unit) tile_rows = unit;
  const int64_t lds_budget = kMaxLds - kGatherStaticLds;
  while (tile_rows > unit && lds_x + tile_rows * kGatherMv * 4 > lds_budget)
    tile_rows = ((tile_rows / 2 + unit - 1) / unit) * unit;
  const int64_t lds = lds_x + tile_rows * kGatherMv * 4;
  if (lds > lds_budget) return fail(QMV_EUNSUPPORTED, "gather_qmv: K=%lld too large", (long long)a.K);
  const int64_t tiles = (a.N + tile_rows - 1) / tile_rows;
  if (E * tiles > 0x7FFFFFFF) return fail(QMV_EUNSUPPORTED, "gather_qmv: grid too large");
  a.tiles = static_cast<int>(tiles);
  a.tile_rows = static_cast<int>(tile_rows);
  a.res_offset = static_cast<int>(lds_x);
  auto kern = qmvk::gather_kernel<BITS, kGatherMv, kGatherWaves, kGatherDepth, gather_cpl<BITS>()>;
  allow_lds(kern, lds);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(E * tiles)), dim3(kGatherWaves * qmvk::kWave),
                     static_cast<size_t>(lds), st, a);
  return check_launch("gather_qmv");
}

#ifndef QMV_GATHER_QMM_MIN
// mean x vectors per expert from which gather_qmv uses the matrix cores (64
// experts of 2048x2048 4-bit, top-8, on MI355X, matvec vs matrix cores: 4
// per expert 64.1 vs 65.7 us, 5 per expert 75.5 vs 65.3, 6 per expert 86.0
// vs 65.8, 8 per expert 103 vs 64.8)
#define QMV_GATHER_QMM_MIN 5
#endif

// A path threshold, overridable by a positive integer in the environment
// variable `name` (read once per process).  The overrides exist to time both
// paths on one shape; the built-in values are the measured crossovers.
static int threshold_from_env(const char *name, int builtin) {
  const char *v = std::getenv(name);
  if (!v || !*v) return builtin;
  char *end = nullptr;
  const long n = std::strtol(v, &end, 10);
  return (end && *end == '\0' && n > 0 && n < (1L << 30)) ? static_cast<int>(n) : builtin;
}

static int gather_qmm_min() {
  static const int v = threshold_from_env("QMV_GATHER_QMM_MIN", QMV_GATHER_QMM_MIN);
  return v;
}

template <int BITS, int CPG, int BM>
int launch_gather_qmm_t(const qmvk::GatherQmmArgs &a0, int64_t E, hipStream_t st) {
  qmvk::GatherQmmArgs a = a0;
  constexpr int MR = 16 * BM;
  const int64_t NB = (a.N + qmvk::kGqmmRowsPerWG - 1) / qmvk::kGqmmRowsPerWG;
  // Slabs of MR x vectors run in parallel workgroups: an expert routed more
  // than MR vectors would otherwise take its slabs one after another and set
  // the kernel's critical path.  1.5x the mean slab count per expert covers
  // the usual spread; an expert with more slabs loops over them.  (512 tokens
  // x top-8 over 64 experts on MI355X, ~64 vectors per expert.)
  const int64_t mean_vec = (a.P * a.M + E - 1) / E;
  int64_t slabs = (3 * mean_vec + 2 * MR - 1) / (2 * MR);
  if (slabs < 1) slabs = 1;
  if (slabs > 8) slabs = 8;
  if (slabs * E * NB > 0x7FFFFFFF) return fail(QMV_EUNSUPPORTED, "gather_qmv: grid too large");
  a.slabs = static_cast<int>(slabs);
  constexpr int lds = qmvk::qmm_lds_bytes<BM>();
  auto kern = qmvk::gather_qmm_kernel<BITS, CPG, BM>;
  allow_lds(kern, lds);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(slabs * E * NB)), dim3(qmvk::kGqmmThreads), lds,
                     st, a);
  return check_launch("gather_qmv (matrix cores)");
}

// Slab height (m-tiles of 16 x vectors): the smallest whose one slab covers
// 1.5x the mean vectors per expert.  Taller slabs stage and multiply
// padding; shorter ones make most experts read their weights twice.
// (64 experts of 2048x2048 4-bit, top-8, on MI355X, slabs of 16 / 32 / 64:
// 8 per expert 85.8 / 99.5 / 106.7 us, 12 per expert 120 / 99.8 / 106.5,
// 16 per expert 145 / 100.9 / 107.)
#ifndef QMV_GQMM_BM
#define QMV_GQMM_BM 0             // 0: chosen per call; 1, 2 or 4: fixed
#endif
template <int BITS, int CPG>
int launch_gather_qmm_c(const qmvk::GatherQmmArgs &a, int64_t E, hipStream_t st) {
  const int64_t mean_vec = (a.P * a.M + E - 1) / E;
  const int bm = QMV_GQMM_BM ? QMV_GQMM_BM : (3 * mean_vec <= 2 * 16 ? 1 : 3 * mean_vec <= 2 * 32 ? 2 : 4);
  switch (bm) {
    case 1: return launch_gather_qmm_t<BITS, CPG, 1>(a, E, st);
    case 2: return launch_gather_qmm_t<BITS, CPG, 2>(a, E, st);
    default: return launch_gather_qmm_t<BITS, CPG, 4>(a, E, st);
  }
}

template <int BITS>
int launch_gather_qmm_g(int gshift, const qmvk::GatherQmmArgs &a, int64_t E, hipStream_t st) {
  switch (gshift) {
    case 0: return launch_gather_qmm_c<BITS, 1>(a, E, st);
    case 1: return launch_gather_qmm_c<BITS, 2>(a, E, st);
    default: return launch_gather_qmm_c<BITS, 4>(a, E, st);
  }
}

template <int BITS>
int launch_unpack_t(const uint32_t *w_q, int64_t N, int64_t K, uint8_t *codes, hipStream_t st) {
  const int64_t items = N * (K / 32);
  const int64_t blocks = (items + 255) / 256;
  if (blocks > 0x7FFFFFFF) return fail(QMV_EUNSUPPORTED, "qmv_unpack_codes: too large");
  hipLaunchKernelGGL(qmvk::unpack_kernel<BITS>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     st, w_q, N, K, codes);
  return check_launch("qmv_unpack_codes");
}

// ------------------------------------------------------------------ QMV_DEBUG
// With QMV_DEBUG set in the environment (non-empty, not "0"; read on every
// call), gather_qmv checks its index preconditions on the device first and
// waits for the answer.
bool debug_enabled() {
  const char *v = std::getenv("QMV_DEBUG");
  return v && *v && !(v[0] == '0' && v[1] == '\0');
}

__global__ __launch_bounds__(256) void check_indices_kernel(const uint32_t *__restrict__ lhs,
                                                            const uint32_t *__restrict__ rhs, int64_t P,
                                                            int64_t Bx, int64_t E, uint32_t *bad) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p < P && (static_cast<int64_t>(lhs[p]) >= Bx || static_cast<int64_t>(rhs[p]) >= E)) *bad = 1u;
}

__global__ void clear_flag_kernel(uint32_t *flag) { *flag = 0u; }

// QMV_OK if every lhs[p] < Bx and rhs[p] < E, QMV_EINVAL if not.  Skipped
// (QMV_OK) while the stream is being captured: the check must wait for the
// device, which a capture cannot.
int check_gather_indices(const uint32_t *lhs, const uint32_t *rhs, int64_t P, int64_t Bx, int64_t E,
                         hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return fail(QMV_EHIP, "gather_qmv: QMV_DEBUG: hipStreamIsCapturing failed");
  }
  if (cs != hipStreamCaptureStatusNone) return QMV_OK;
  uint32_t *flag = nullptr;
  if (hipMallocAsync(reinterpret_cast<void **>(&flag), sizeof(uint32_t), st) != hipSuccess) {
    (void)hipGetLastError();
    return fail(QMV_EHIP, "gather_qmv: QMV_DEBUG: allocating the check flag failed");
  }
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, st, flag);
  const int64_t blocks = (P + 255) / 256;
  hipLaunchKernelGGL(check_indices_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, lhs, rhs,
                     P, Bx, E, flag);
  uint32_t bad = 0;
  const bool ok = hipMemcpyAsync(&bad, flag, sizeof(bad), hipMemcpyDeviceToHost, st) == hipSuccess &&
                  hipFreeAsync(flag, st) == hipSuccess && hipStreamSynchronize(st) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    return fail(QMV_EHIP, "gather_qmv: QMV_DEBUG: the index check failed to run");
  }
  if (bad) return fail(QMV_EINVAL, "gather_qmv: QMV_DEBUG: an index is out of range (need lhs < Bx = %lld "
                       "and rhs < E = %lld for all %lld pairs)", (long long)Bx, (long long)E, (long long)P);
  return QMV_OK;
}

// ------------------------------------------------------------------ workspace
// The split-K paths (transpose = 0, and 5 or more rows of x on the matrix
// cores) write the S slices' fp32 partial sums to a workspace that a second
// kernel adds in slice order.  The workspace always belongs to one call:
// qmv_with_workspace takes it as an argument and qmv takes a stream-ordered
// allocation that it frees on the same stream.  In sizing mode nothing is launched and the
// largest size any launch of the call needs is recorded.
struct Ws {
  void *ptr = nullptr;
  size_t bytes = 0;
  bool sizing = false;
  size_t need = 0;
};

int take_workspace(Ws &ws, size_t bytes, float **out) {
  if (ws.sizing) {
    if (bytes > ws.need) ws.need = bytes;
    return QMV_OK;
  }
  if (ws.ptr == nullptr || ws.bytes < bytes)
    return fail(QMV_EINVAL, "qmv: this call needs a %zu-byte workspace, %zu given (qmv_workspace_bytes "
                "reports the size)", bytes, ws.ptr ? ws.bytes : static_cast<size_t>(0));
  *out = static_cast<float *>(ws.ptr);
  return QMV_OK;
}

// ------------------------------------------------------------------ qvm
// y = the S slices of `part` added in slice order (one thread per output),
// with the load batch sized to S.
void launch_slice_reduce(const float *part, int S, int MVs, int M, int64_t N, int64_t y_ld, int out_f32,
                         void *y, hipStream_t st) {
  const int64_t outs = static_cast<int64_t>(M) * N;
  const dim3 grid(static_cast<unsigned>((outs + 255) / 256)), block(256);
  if (S <= 8) hipLaunchKernelGGL(qmvk::qvm_reduce_kernel<8>, grid, block, 0, st, part, S, MVs, M, N, y_ld, out_f32, y);
  else if (S <= 16) hipLaunchKernelGGL(qmvk::qvm_reduce_kernel<16>, grid, block, 0, st, part, S, MVs, M, N, y_ld, out_f32, y);
  else if (S <= 32) hipLaunchKernelGGL(qmvk::qvm_reduce_kernel<32>, grid, block, 0, st, part, S, MVs, M, N, y_ld, out_f32, y);
  else hipLaunchKernelGGL(qmvk::qvm_reduce_kernel<64>, grid, block, 0, st, part, S, MVs, M, N, y_ld, out_f32, y);
}

#ifndef QMV_QVM_ROWS
#define QMV_QVM_ROWS 4            // rows in flight per stream
#endif
#ifndef QMV_QVM_WGS
#define QMV_QVM_WGS 1024          // split-K target: workgroups per launch
#endif
constexpr int kQvmRows = QMV_QVM_ROWS;

template <int BITS, int MV>
int launch_qvm_t(const qmvk::QvmArgs &a0, Ws &ws, hipStream_t st) {
  qmvk::QvmArgs a = a0;
  const int64_t Nc = a.N / 32;
  const int64_t CB = (Nc + qmvk::kQvmC - 1) / qmvk::kQvmC;
  const int64_t unit = static_cast<int64_t>(kQvmRows) * qmvk::kQvmStreams;
  // ~QMV_QVM_WGS workgroups, at most 64 slices, whole blocks of rows per
  // slice (4096x4096 4-bit on MI355X: 4 rows per stream measured 12-15%
  // ahead of 1 or 2, and 2048 workgroups no better than 1024)
  int64_t s_target = QMV_QVM_WGS / CB;
  if (s_target < 1) s_target = 1;
  if (s_target > 64) s_target = 64;
  int64_t ks = (a.K + s_target - 1) / s_target;
  ks = ((ks + unit - 1) / unit) * unit;
  if (ks > 1024) ks = 1024;             // the staged x slice stays small beside the sums
  const int64_t S = (a.K + ks - 1) / ks;
  if (CB * S > 0x7FFFFFFF) return fail(QMV_EUNSUPPORTED, "qmv: transpose=0 grid too large");
  const int64_t lds = 4 * (MV * ks + static_cast<int64_t>(qmvk::kQvmWaves) * MV * qmvk::kQvmRow);
  if (lds > kMaxLds) return fail(QMV_EUNSUPPORTED, "qmv: transpose=0 with K=%d too large", a.K);
  a.S = static_cast<int>(S);
  a.ks = static_cast<int>(ks);
  if (S > 1) {
    if (int rc = take_workspace(ws, static_cast<size_t>(S) * MV * a.N * 4, &a.part)) return rc;
  }
  if (ws.sizing) return QMV_OK;
  auto kern = qmvk::qvm_kernel<BITS, MV, kQvmRows>;
  allow_lds(kern, lds);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(CB * S)), dim3(qmvk::kQvmWaves * qmvk::kWave),
                     static_cast<size_t>(lds), st, a);
  if (int rc = check_launch("qmv (transpose=0)")) return rc;
  if (S > 1) {
    launch_slice_reduce(a.part, a.S, MV, a.M, a.N, a.y_ld, a.out_f32, a.y, st);
    return check_launch("qmv (transpose=0) reduce");
  }
  return QMV_OK;
}

template <int MV>
int launch_qvm_bits(int bits, const qmvk::QvmArgs &a, Ws &ws, hipStream_t st) {
  switch (bits) {
    case 2: return launch_qvm_t<2, MV>(a, ws, st);
    case 3: return launch_qvm_t<3, MV>(a, ws, st);
    case 4: return launch_qvm_t<4, MV>(a, ws, st);
    case 5: return launch_qvm_t<5, MV>(a, ws, st);
    case 6: return launch_qvm_t<6, MV>(a, ws, st);
    case 8: return launch_qvm_t<8, MV>(a, ws, st);
  }
  return fail(QMV_EINVAL, "bits=%d", bits);
}

// y = x @ W_hat with W packed [K, N] along N: slabs of up to 4 vectors.
int run_qvm(const uint16_t *x, const uint32_t *w_q, const uint16_t *scales, const uint16_t *biases,
            void *y, int64_t M, int64_t N, int64_t K, int group_size, int bits, int out_f32,
            Ws &ws, hipStream_t st) {
  for (int64_t m0 = 0; m0 < M; m0 += 4) {
    qmvk::QvmArgs a{};
    const int64_t nv = M - m0 < 4 ? M - m0 : 4;
    a.x = x + m0 * K;
    a.w = w_q;
    a.s = scales;
    a.b = biases;
    a.y = out_f32 ? static_cast<void *>(static_cast<float *>(y) + m0 * N)
                  : static_cast<void *>(static_cast<uint16_t *>(y) + m0 * N);
    a.N = N;
    a.y_ld = N;
    a.K = static_cast<int>(K);
    a.M = static_cast<int>(nv);
    a.gshift = gshift_of(group_size);
    a.out_f32 = out_f32;
    const int rc = nv == 1 ? launch_qvm_bits<1>(bits, a, ws, st)
                 : nv == 2 ? launch_qvm_bits<2>(bits, a, ws, st)
                           : launch_qvm_bits<4>(bits, a, ws, st);
    if (rc) return rc;
  }
  return ok();
}

// ------------------------------------------------------------------ qmm
#ifndef QMV_QMM_MIN_M
// x rows from which transpose=1 uses the matrix cores: anything past one
// 4-row slab (4096x4096 4-bit on MI355X, slabs vs matrix cores: M = 5
// 9.75 vs 9.69 us, M = 6 10.2 vs 9.7, M = 8 11.2 vs 9.75, M = 11 16.2 vs
// 9.9; 14336x4096 at M = 8: 25.1 vs 19.3)
#define QMV_QMM_MIN_M 5
#endif

static int qmm_min_m() {
  static const int v = threshold_from_env("QMV_QMM_MIN_M", QMV_QMM_MIN_M);
  return v;
}
#ifndef QMV_QMM_WGS
#define QMV_QMM_WGS 512           // split-K target: workgroups per launch
#endif

template <int BITS, int BM, int CPG>
int launch_qmm_t(const qmvk::QmmArgs &a0, Ws &ws, hipStream_t st) {
  qmvk::QmmArgs a = a0;
  constexpr int MR = 16 * BM;
  const int64_t Kc = a.K / 32;
  const int64_t NB = (a.N + qmvk::kQmmRowsPerWG - 1) / qmvk::kQmmRowsPerWG;
  const int64_t blocks = (Kc + qmvk::kQmmKB - 1) / qmvk::kQmmKB;
  int64_t S = (QMV_QMM_WGS + NB - 1) / NB;
  if (S > blocks) S = blocks;
  if (S < 1) S = 1;
  const int64_t cps = ((blocks + S - 1) / S) * qmvk::kQmmKB;   // chunks per slice
  S = (Kc + cps - 1) / cps;
  if (NB * S > 0x7FFFFFFF) return fail(QMV_EUNSUPPORTED, "qmv: grid too large");
  a.S = static_cast<int>(S);
  a.cps = static_cast<int>(cps);
  if (S > 1) {
    if (int rc = take_workspace(ws, static_cast<size_t>(S) * MR * a.N * 4, &a.part)) return rc;
  }
  if (ws.sizing) return QMV_OK;
  constexpr int lds = qmvk::qmm_lds_bytes<BM>();
  auto kern = qmvk::qmm_kernel<BITS, BM, CPG>;
  allow_lds(kern, lds);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(NB * S)), dim3(qmvk::kQmmThreads), lds, st, a);
  if (int rc = check_launch("qmv (matrix cores)")) return rc;
  if (S > 1) {
    launch_slice_reduce(a.part, a.S, MR, a.M, a.N, a.y_ld, a.out_f32, a.y, st);
    return check_launch("qmv (matrix cores) reduce");
  }
  return QMV_OK;
}

template <int BITS, int CPG>
int launch_qmm_bm(int bm, const qmvk::QmmArgs &a, Ws &ws, hipStream_t st) {
  switch (bm) {
    case 1: return launch_qmm_t<BITS, 1, CPG>(a, ws, st);
    case 2: return launch_qmm_t<BITS, 2, CPG>(a, ws, st);
    case 3: return launch_qmm_t<BITS, 3, CPG>(a, ws, st);
    default: return launch_qmm_t<BITS, 4, CPG>(a, ws, st);
  }
}

template <int BITS>
int launch_qmm_g(int bm, const qmvk::QmmArgs &a, Ws &ws, hipStream_t st) {
  switch (a.gshift) {
    case 0: return launch_qmm_bm<BITS, 1>(bm, a, ws, st);
    case 1: return launch_qmm_bm<BITS, 2>(bm, a, ws, st);
    default: return launch_qmm_bm<BITS, 4>(bm, a, ws, st);
  }
}

// y = x @ W_hat^T for many rows of x: slabs of up to 64 rows on the matrix cores.
int run_qmm(const uint16_t *x, const uint32_t *w_q, const uint16_t *scales, const uint16_t *biases,
            void *y, int64_t M, int64_t N, int64_t K, int group_size, int bits, int out_f32,
            Ws &ws, hipStream_t st) {
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int64_t rows = M - m0 < 64 ? M - m0 : 64;
    qmvk::QmmArgs a{};
    a.x = x + m0 * K;
    a.w = w_q;
    a.s = scales;
    a.b = biases;
    a.y = out_f32 ? static_cast<void *>(static_cast<float *>(y) + m0 * N)
                  : static_cast<void *>(static_cast<uint16_t *>(y) + m0 * N);
    a.N = N;
    a.y_ld = N;
    a.K = static_cast<int>(K);
    a.M = static_cast<int>(rows);
    a.gshift = gshift_of(group_size);
    a.out_f32 = out_f32;
    const int bm = static_cast<int>((rows + 15) / 16);
    int rc;
    switch (bits) {
      case 2: rc = launch_qmm_g<2>(bm, a, ws, st); break;
      case 3: rc = launch_qmm_g<3>(bm, a, ws, st); break;
      case 4: rc = launch_qmm_g<4>(bm, a, ws, st); break;
      case 5: rc = launch_qmm_g<5>(bm, a, ws, st); break;
      case 6: rc = launch_qmm_g<6>(bm, a, ws, st); break;
      default: rc = launch_qmm_g<8>(bm, a, ws, st); break;
    }
    if (rc) return rc;
  }
  return ok();
}

// ------------------------------------------------------------------ qmf
// From QMV_QMM_MIN_M up to 16 rows of x against a 4-bit weight with K = 2048
// or 4096: one pass on the matrix cores, K split across the waves of a
// workgroup (qmf_kernels.h), no partial sums and no second kernel.
// 4096x4096 g64 on MI355X against the split-K product: M = 5 9.07 -> 6.33
// us, M = 8 9.11 -> 6.92, M = 16 9.30 -> 8.10 (and at M = 4, 6.36 against
// 5.87 on the one-slab matvec, which keeps M <= 4).  QMV_QMF=0 in the
// environment turns it off (read once per process).
static int qmf_enabled() {
  static const int v = [] {
    const char *e = std::getenv("QMV_QMF");
    return (e && e[0] == '0' && e[1] == '\0') ? 0 : 1;
  }();
  return v;
}

static bool qmf_fits(int64_t M, int64_t N, int64_t K, int bits) {
  return bits == 4 && M >= 2 && M <= 16 && (K == 2048 || K == 4096) &&
         N * K / 2 < (int64_t(1) << 32) && M * K * 2 < (int64_t(1) << 32);
}

template <int CW, int CPG>
int launch_qmf_t(const qmvk::QmfArgs &a, hipStream_t st) {
  const int64_t blocks = (a.N + 15) / 16;
  if (blocks > 0x7FFFFFFF) return fail(QMV_EUNSUPPORTED, "qmv: too many rows");
  constexpr int lds = qmvk::qmf_lds_bytes<CW>();
  auto kern = qmvk::qmf_kernel<CW, CPG>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(qmvk::kQmfThreads), lds, st, a);
  return check_launch("qmv (matrix cores, one pass)");
}

template <int CW>
int launch_qmf_g(int gshift, const qmvk::QmfArgs &a, hipStream_t st) {
  switch (gshift) {
    case 0: return launch_qmf_t<CW, 1>(a, st);
    case 1: return launch_qmf_t<CW, 2>(a, st);
    default: return launch_qmf_t<CW, 4>(a, st);
  }
}

int run_qmf(const uint16_t *x, const uint32_t *w_q, const uint16_t *scales, const uint16_t *biases, void *y,
            int64_t M, int64_t N, int64_t K, int group_size, int out_f32, hipStream_t st) {
  qmvk::QmfArgs a{};
  a.x = x;
  a.w = w_q;
  a.s = scales;
  a.b = biases;
  a.y = y;
  a.N = N;
  a.y_ld = N;
  a.K = static_cast<int>(K);
  a.M = static_cast<int>(M);
  a.out_f32 = out_f32;
  const int gshift = gshift_of(group_size);
  return K == 2048 ? launch_qmf_g<8>(gshift, a, st) : launch_qmf_g<16>(gshift, a, st);
}

template <int BITS>
int launch_dequant_t(const uint32_t *w_q, const uint16_t *scales, const uint16_t *biases,
                     int64_t N, int64_t K, int gshift, int out_f32, void *out, hipStream_t st) {
  const int64_t items = N * (K / (out_f32 ? 4 : 8));   // units of 16 output bytes
  const int64_t threads = (items + qmvk::kDequantUnits - 1) / qmvk::kDequantUnits;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return fail(QMV_EUNSUPPORTED, "qmv_dequantize: too large");
  auto kern = out_f32 ? qmvk::dequant_kernel<BITS, true> : qmvk::dequant_kernel<BITS, false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, w_q, scales, biases,
                     N, K, gshift, out);
  return check_launch("qmv_dequantize");
}

}  // namespace

extern "C" {

const char *qmv_last_error(void) { return g_last_error.c_str(); }

int qmv_pack(const float *w, int64_t N, int64_t K, int group_size, int bits, uint32_t *w_q,
             uint16_t *scales, uint16_t *biases, void *stream) {
  if (int rc = check_common("qmv_pack", N, K, group_size, bits)) return rc;
  if (!w || !w_q || !scales || !biases) return fail(QMV_EINVAL, "qmv_pack: null pointer argument");
  if (int rc = check_aligned("qmv_pack", w, "w")) return rc;
  const int64_t groups = N * (K / group_size);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 block(qmvk::kPackThreads);
  auto grid = [&](int g) {
    const int64_t gpb = qmvk::kPackThreads / (g / 4);
    return (groups + gpb - 1) / gpb;
  };
  if (grid(group_size) > 0x7FFFFFFF) return fail(QMV_EUNSUPPORTED, "qmv_pack: too large");
  const dim3 blocks(static_cast<unsigned>(grid(group_size)));
  switch (group_size) {
    case 32:
      hipLaunchKernelGGL(qmvk::pack_kernel<32>, blocks, block, 0, st, w, groups, bits, w_q, scales, biases);
      break;
    case 64:
      hipLaunchKernelGGL(qmvk::pack_kernel<64>, blocks, block, 0, st, w, groups, bits, w_q, scales, biases);
      break;
    default:
      hipLaunchKernelGGL(qmvk::pack_kernel<128>, blocks, block, 0, st, w, groups, bits, w_q, scales, biases);
      break;
  }
  return check_launch("qmv_pack");
}

int qmv_unpack_codes(const uint32_t *w_q, int64_t N, int64_t K, int bits, uint8_t *codes,
                     void *stream) {
  if (!bits_ok(bits)) return fail(QMV_EINVAL, "qmv_unpack_codes: bits=%d not in {2,3,4,5,6,8}", bits);
  if (N <= 0 || K <= 0 || K % 32 != 0)
    return fail(QMV_EINVAL, "qmv_unpack_codes: need N > 0 and K a positive multiple of 32");
  if (!w_q || !codes) return fail(QMV_EINVAL, "qmv_unpack_codes: null pointer argument");
  if (int rc = check_aligned("qmv_unpack_codes", w_q, "w_q")) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (bits) {
    case 2: return launch_unpack_t<2>(w_q, N, K, codes, st);
    case 3: return launch_unpack_t<3>(w_q, N, K, codes, st);
    case 4: return launch_unpack_t<4>(w_q, N, K, codes, st);
    case 5: return launch_unpack_t<5>(w_q, N, K, codes, st);
    case 6: return launch_unpack_t<6>(w_q, N, K, codes, st);
    default: return launch_unpack_t<8>(w_q, N, K, codes, st);
  }
}

int qmv_dequantize(const uint32_t *w_q, const uint16_t *scales, const uint16_t *biases, void *out,
                   int64_t N, int64_t K, int group_size, int bits, int out_dtype, void *stream) {
  if (int rc = check_common("qmv_dequantize", N, K, group_size, bits)) return rc;
  if (!w_q || !scales || !biases || !out) return fail(QMV_EINVAL, "qmv_dequantize: null pointer argument");
  if (out_dtype != QMV_OUT_BF16 && out_dtype != QMV_OUT_F32)
    return fail(QMV_EINVAL, "qmv_dequantize: out_dtype=%d unknown", out_dtype);
  if (int rc = check_aligned("qmv_dequantize", w_q, "w_q")) return rc;
  if (int rc = check_aligned("qmv_dequantize", out, "out")) return rc;
  const int gs = gshift_of(group_size);
  const int f32 = out_dtype == QMV_OUT_F32;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (bits) {
    case 2: return launch_dequant_t<2>(w_q, scales, biases, N, K, gs, f32, out, st);
    case 3: return launch_dequant_t<3>(w_q, scales, biases, N, K, gs, f32, out, st);
    case 4: return launch_dequant_t<4>(w_q, scales, biases, N, K, gs, f32, out, st);
    case 5: return launch_dequant_t<5>(w_q, scales, biases, N, K, gs, f32, out, st);
    case 6: return launch_dequant_t<6>(w_q, scales, biases, N, K, gs, f32, out, st);
    default: return launch_dequant_t<8>(w_q, scales, biases, N, K, gs, f32, out, st);
  }
}

}  // extern "C"

namespace {

// qmv with its workspace supplied (or, in sizing mode, only measured).  In
// sizing mode no pointer is dereferenced or checked and nothing is launched.
int qmv_impl(const uint16_t *x, const uint32_t *w_q, const uint16_t *scales, const uint16_t *biases,
             void *y, int64_t M, int64_t N, int64_t K, int group_size, int bits, int transpose,
             int out_dtype, Ws &ws, hipStream_t st) {
  const bool ptrs = !ws.sizing;
  if (transpose != 0 && transpose != 1)
    return fail(QMV_EINVAL, "qmv: transpose=%d must be 0 or 1", transpose);
  // the packed (group) axis is K for transpose = 1 and N for transpose = 0
  if (int rc = transpose ? check_common("qmv", N, K, group_size, bits)
                         : check_shape("qmv (transpose=0)", K, "K", N, "N", group_size, bits)) return rc;
  if (M <= 0) return fail(QMV_EINVAL, "qmv: M=%lld must be positive", (long long)M);
  if (ptrs && (!x || !w_q || !scales || !biases || !y)) return fail(QMV_EINVAL, "qmv: null pointer argument");
  if (out_dtype != QMV_OUT_BF16 && out_dtype != QMV_OUT_F32)
    return fail(QMV_EINVAL, "qmv: out_dtype=%d unknown", out_dtype);
  if (transpose == 0) {
    if (ptrs) {
      if (int rc = check_aligned("qmv", w_q, "w_q")) return rc;
    }
    if (K > (int64_t(1) << 30) || M > (int64_t(1) << 30))
      return fail(QMV_EUNSUPPORTED, "qmv: transpose=0 with K or M too large");
    if (int rc = run_qvm(x, w_q, scales, biases, y, M, N, K, group_size, bits, out_dtype == QMV_OUT_F32, ws, st))
      return rc;
    return ok();
  }
  if (ptrs) {
    if (int rc = check_aligned("qmv", x, "x")) return rc;
    if (int rc = check_aligned("qmv", w_q, "w_q")) return rc;
  }
  if (M >= qmm_min_m() && qmf_fits(M, N, K, bits) && qmf_enabled()) {
    if (ws.sizing) return ok();   // no workspace
    if (int rc = run_qmf(x, w_q, scales, biases, y, M, N, K, group_size, out_dtype == QMV_OUT_F32, st)) return rc;
    return ok();
  }
  if (M >= qmm_min_m() && N * K * bits / 8 < (int64_t(1) << 32) &&
      N * (K / group_size) * 2 < (int64_t(1) << 32) && 64 * K * 2 < (int64_t(1) << 32)) {
    // (the matrix-core kernel addresses W, scales and biases and a 64-row
    // slab of x with 32-bit byte offsets)
    if (M > (int64_t(1) << 30)) return fail(QMV_EUNSUPPORTED, "qmv: M=%lld too large", (long long)M);
    if (int rc = run_qmm(x, w_q, scales, biases, y, M, N, K, group_size, bits, out_dtype == QMV_OUT_F32, ws, st))
      return rc;
    return ok();
  }
  const int mv_max = qmv_lds_bytes(bits, 4, K) <= kMaxLds ? 4
                   : qmv_lds_bytes(bits, 2, K) <= kMaxLds ? 2
                   : qmv_lds_bytes(bits, 1, K) <= kMaxLds ? 1 : 0;
  if (mv_max == 0)
    return fail(QMV_EUNSUPPORTED, "qmv: K=%lld too large for one workgroup's staged x", (long long)K);
  if (ws.sizing) return ok();   // the matvec slabs need no workspace
  const size_t esz = out_dtype == QMV_OUT_F32 ? 4 : 2;
  for (int64_t m0 = 0; m0 < M; m0 += mv_max) {
    const int mv = static_cast<int>(M - m0 < mv_max ? M - m0 : mv_max);
    qmvk::QmvArgs a{};
    a.x = x + m0 * K;
    a.mat0 = {w_q, scales, biases, static_cast<char *>(y) + m0 * N * esz};
    a.mat1 = a.mat0;
    a.nmat = 1;
    a.N = N;
    a.K = static_cast<int>(K);
    a.M = mv;
    a.gshift = gshift_of(group_size);
    a.out_f32 = out_dtype == QMV_OUT_F32;
    a.y_ld = N;
    int rc;
    if (mv == 1) rc = launch_qmv_bits<1, qmvk::XIN_PLAIN>(bits, a, st);
    else if (mv == 2) rc = launch_qmv_bits<2, qmvk::XIN_PLAIN>(bits, a, st);
    else rc = launch_qmv_bits<4, qmvk::XIN_PLAIN>(bits, a, st);
    if (rc) return rc;
  }
  return ok();
}

// ------------------------------------------------------------------ no-alloc scratch
// qmv_noalloc's workspace: a static device array, one copy per GPU, held from
// the module's load until the process ends.  In host code `scratch` only
// names the symbol; its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device (with that device current) on
// the entry point's first call there, and only that address is used.
constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

int scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QMV_EHIP, "qmv_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(QMV_EUNSUPPORTED, "qmv_noalloc: device %d out of range", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr)
    return fail(QMV_EHIP, "qmv_noalloc: hipGetSymbolAddress of the scratch array failed on device %d: %s",
                dev, hipGetErrorString(g_scratch_err[dev]));
  *out = g_scratch_ptr[dev];
  return QMV_OK;
}

}  // namespace

extern "C" {

int qmv_workspace_bytes(int64_t M, int64_t N, int64_t K, int group_size, int bits, int transpose,
                        size_t *bytes) {
  if (!bytes) return fail(QMV_EINVAL, "qmv_workspace_bytes: null bytes pointer");
  Ws ws;
  ws.sizing = true;
  if (int rc = qmv_impl(nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K, group_size, bits, transpose,
                        QMV_OUT_BF16, ws, nullptr))
    return rc;
  *bytes = ws.need;
  return ok();
}

int qmv_with_workspace(const uint16_t *x, const uint32_t *w_q, const uint16_t *scales,
                       const uint16_t *biases, void *y, int64_t M, int64_t N, int64_t K, int group_size,
                       int bits, int transpose, int out_dtype, void *workspace, size_t workspace_bytes,
                       void *stream) {
  if (workspace && !aligned16(workspace))
    return fail(QMV_EINVAL, "qmv_with_workspace: workspace must be 16-byte aligned");
  Ws ws;
  ws.ptr = workspace;
  ws.bytes = workspace ? workspace_bytes : 0;
  return qmv_impl(x, w_q, scales, biases, y, M, N, K, group_size, bits, transpose, out_dtype, ws,
                  static_cast<hipStream_t>(stream));
}

int qmv_noalloc(const uint16_t *x, const uint32_t *w_q, const uint16_t *scales, const uint16_t *biases,
                void *y, int64_t M, int64_t N, int64_t K, int group_size, int bits, int transpose,
                int out_dtype, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws sizing;
  sizing.sizing = true;
  if (int rc = qmv_impl(x, w_q, scales, biases, y, M, N, K, group_size, bits, transpose, out_dtype, sizing, st))
    return rc;
  if (sizing.need > kScratchBytes)
    return fail(QMV_EINVAL, "qmv_noalloc: this call needs a %zu-byte workspace; the scratch array holds %zu "
                "bytes (qmv_with_workspace takes a larger one)", sizing.need, kScratchBytes);
  Ws ws;
  if (sizing.need > 0) {
    if (int rc = scratch_of_current_device(&ws.ptr)) return rc;
    ws.bytes = kScratchBytes;
  }
  return qmv_impl(x, w_q, scales, biases, y, M, N, K, group_size, bits, transpose, out_dtype, ws, st);
}

int qmv(const uint16_t *x, const uint32_t *w_q, const uint16_t *scales, const uint16_t *biases,
        void *y, int64_t M, int64_t N, int64_t K, int group_size, int bits, int transpose,
        int out_dtype, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws sizing;
  sizing.sizing = true;
  if (int rc = qmv_impl(x, w_q, scales, biases, y, M, N, K, group_size, bits, transpose, out_dtype, sizing, st))
    return rc;
  Ws ws;
  if (sizing.need > 0) {
    // a stream-ordered allocation for this call only, freed on the same
    // stream after the call's kernels (no state kept between calls)
    if (hipMallocAsync(&ws.ptr, sizing.need, st) != hipSuccess) {
      (void)hipGetLastError();
      return fail(QMV_EHIP, "qmv: stream-ordered allocation of the %zu-byte split-K workspace failed "
                  "(qmv_with_workspace takes a caller-owned workspace)", sizing.need);
    }
    ws.bytes = sizing.need;
  }
  const int rc = qmv_impl(x, w_q, scales, biases, y, M, N, K, group_size, bits, transpose, out_dtype, ws, st);
  if (ws.ptr && hipFreeAsync(ws.ptr, st) != hipSuccess && rc == QMV_OK)
    return fail(QMV_EHIP, "qmv: freeing the split-K workspace failed");
  return rc;
}

int qmv_gate_up(const uint16_t *x, const uint32_t *wg, const uint16_t *sg, const uint16_t *bg,
                const uint32_t *wu, const uint16_t *su, const uint16_t *bu, uint16_t *gate_y,
                uint16_t *up_y, int64_t N, int64_t K, int group_size, int bits, void *stream) {
  if (int rc = check_common("qmv_gate_up", N, K, group_size, bits)) return rc;
  if (!x || !wg || !sg || !bg || !wu || !su || !bu || !gate_y || !up_y)
    return fail(QMV_EINVAL, "qmv_gate_up: null pointer argument");
  if (int rc = check_aligned("qmv_gate_up", x, "x")) return rc;
  if (int rc = check_aligned("qmv_gate_up", wg, "wg")) return rc;
  if (int rc = check_aligned("qmv_gate_up", wu, "wu")) return rc;
  if (qmv_lds_bytes(bits, 1, K) > kMaxLds)
    return fail(QMV_EUNSUPPORTED, "qmv_gate_up: K=%lld too large", (long long)K);
  qmvk::QmvArgs a{};
  a.x = x;
  a.mat0 = {wg, sg, bg, gate_y};
  a.mat1 = {wu, su, bu, up_y};
  a.nmat = 2;
  a.N = N;
  a.K = static_cast<int>(K);
  a.M = 1;
  a.gshift = gshift_of(group_size);
  a.out_f32 = 0;
  a.y_ld = N;
  const int rc = launch_qmv_bits<1, qmvk::XIN_PLAIN>(bits, a, static_cast<hipStream_t>(stream));
  return rc ? rc : ok();
}

int qmv_silu_gate_resid(const uint16_t *gate, const uint16_t *up, const uint16_t *x_resid,
                        const uint32_t *w_q, const uint16_t *scales, const uint16_t *biases,
                        void *y, int64_t N, int64_t K, int group_size, int bits, int out_dtype,
                        void *stream) {
  if (int rc = check_common("qmv_silu_gate_resid", N, K, group_size, bits)) return rc;
  if (!gate || !up || !w_q || !scales || !biases || !y)
    return fail(QMV_EINVAL, "qmv_silu_gate_resid: null pointer argument");
  if (out_dtype != QMV_OUT_BF16 && out_dtype != QMV_OUT_F32)
    return fail(QMV_EINVAL, "qmv_silu_gate_resid: out_dtype=%d unknown", out_dtype);
  if (int rc = check_aligned("qmv_silu_gate_resid", gate, "gate")) return rc;
  if (int rc = check_aligned("qmv_silu_gate_resid", up, "up")) return rc;
  if (int rc = check_aligned("qmv_silu_gate_resid", w_q, "w_q")) return rc;
  if (qmv_lds_bytes(8, 1, K) > kMaxLds)
    return fail(QMV_EUNSUPPORTED, "qmv_silu_gate_resid: K=%lld too large", (long long)K);
  qmvk::QmvArgs a{};
  a.x = gate;
  a.up = up;
  a.xres = x_resid;
  a.mat0 = {w_q, scales, biases, y};
  a.mat1 = a.mat0;
  a.nmat = 1;
  a.N = N;
  a.K = static_cast<int>(K);
  a.M = 1;
  a.gshift = gshift_of(group_size);
  a.out_f32 = out_dtype == QMV_OUT_F32;
  a.y_ld = N;
  const int rc = launch_qmv_bits<1, qmvk::XIN_SILU>(bits, a, static_cast<hipStream_t>(stream));
  return rc ? rc : ok();
}

int gather_qmv(const uint16_t *x, int64_t Bx, const uint32_t *w_q, const uint16_t *scales,
               const uint16_t *biases, int64_t E, const uint32_t *lhs_indices,
               const uint32_t *rhs_indices, int64_t P, void *y, int64_t M, int64_t N, int64_t K,
               int group_size, int bits, int transpose, int sorted_indices, int out_dtype,
               void *stream) {
  if (int rc = check_common("gather_qmv", N, K, group_size, bits)) return rc;
  if (!x || !w_q || !scales || !biases || !y) return fail(QMV_EINVAL, "gather_qmv: null pointer argument");
  if (M <= 0 || Bx <= 0 || E <= 0)
    return fail(QMV_EINVAL, "gather_qmv: M=%lld, Bx=%lld, E=%lld must be positive", (long long)M,
                (long long)Bx, (long long)E);
  if (out_dtype != QMV_OUT_BF16 && out_dtype != QMV_OUT_F32)
    return fail(QMV_EINVAL, "gather_qmv: out_dtype=%d unknown", out_dtype);
  if ((lhs_indices == nullptr) != (rhs_indices == nullptr))
    return fail(QMV_EINVAL, "gather_qmv: lhs_indices and rhs_indices must both be given or both NULL");
  if (transpose != 1)
    return fail(QMV_EUNSUPPORTED, "gather_qmv: transpose=0 is not implemented");
  if (!lhs_indices) {
    // no indices: the plain quantized product of x[0] with W[0]
    const int rc = qmv(x, w_q, scales, biases, y, M, N, K, group_size, bits, 1, out_dtype, stream);
    return rc;
  }
  if (P <= 0) return fail(QMV_EINVAL, "gather_qmv: P=%lld must be positive", (long long)P);
  if (int rc = check_aligned("gather_qmv", x, "x")) return rc;
  if (int rc = check_aligned("gather_qmv", w_q, "w_q")) return rc;
  if (qmv_lds_bytes(bits, bits <= 6 ? gather_mv<4>() : gather_mv<8>(), K) > kMaxLds - kGatherStaticLds)
    return fail(QMV_EUNSUPPORTED, "gather_qmv: K=%lld too large", (long long)K);
  if (M > (int64_t(1) << 20) || P > (int64_t(1) << 30))
    return fail(QMV_EUNSUPPORTED, "gather_qmv: M or P too large");
  if (debug_enabled()) {
    if (int rc = check_gather_indices(lhs_indices, rhs_indices, P, Bx, E, static_cast<hipStream_t>(stream)))
      return rc;
  }
  // one expert's words, scales and biases are addressed with 32-bit offsets
  if (N * (K / 32) * bits * 4 + 64 * (K / 32) * bits * 4 >= (int64_t(1) << 31))
    return fail(QMV_EUNSUPPORTED, "gather_qmv: one expert's packed weight must be under 2 GiB");
  qmvk::GatherArgs a{};
  a.x = x;
  a.w = w_q;
  a.s = scales;
  a.b = biases;
  a.lhs = lhs_indices;
  a.rhs = rhs_indices;
  a.P = P;
  a.N = N;
  a.Bx = Bx;
  a.K = static_cast<int>(K);
  a.M = static_cast<int>(M);
  a.gshift = gshift_of(group_size);
  (void)sorted_indices;   // a hint only: the in-kernel routing is order-independent
  a.out_f32 = out_dtype == QMV_OUT_F32;
  a.y = y;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Many tokens per expert: the matrix-core gather (the matrix-core kernel
  // addresses x, and each expert's W, scales and biases, with 32-bit offsets)
  if (P * M >= static_cast<int64_t>(gather_qmm_min()) * E && Bx * M * K * 2 < (int64_t(1) << 32) &&
      N * K * bits / 8 < (int64_t(1) << 32)) {
    qmvk::GatherQmmArgs g{};
    g.x = x;
    g.w = w_q;
    g.s = scales;
    g.b = biases;
    g.lhs = lhs_indices;
    g.rhs = rhs_indices;
    g.P = P;
    g.N = N;
    g.Bx = Bx;
    g.K = static_cast<int>(K);
    g.M = static_cast<int>(M);
    g.out_f32 = out_dtype == QMV_OUT_F32;
    g.y = y;
    const int gs = gshift_of(group_size);
    int rc;
    switch (bits) {
      case 2: rc = launch_gather_qmm_g<2>(gs, g, E, st); break;
      case 3: rc = launch_gather_qmm_g<3>(gs, g, E, st); break;
      case 4: rc = launch_gather_qmm_g<4>(gs, g, E, st); break;
      case 5: rc = launch_gather_qmm_g<5>(gs, g, E, st); break;
      case 6: rc = launch_gather_qmm_g<6>(gs, g, E, st); break;
      default: rc = launch_gather_qmm_g<8>(gs, g, E, st); break;
    }
    return rc ? rc : ok();
  }
  int rc;
  switch (bits) {
    case 2: rc = launch_gather_t<2>(a, E, st); break;
    case 3: rc = launch_gather_t<3>(a, E, st); break;
    case 4: rc = launch_gather_t<4>(a, E, st); break;
    case 5: rc = launch_gather_t<5>(a, E, st); break;
    case 6: rc = launch_gather_t<6>(a, E, st); break;
    default: rc = launch_gather_t<8>(a, E, st); break;
  }
  return rc ? rc : ok();
}

}  // extern "C"
