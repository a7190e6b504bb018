/*
 * qmv.h -- C ABI of libqmv.so: affine group-quantized matrix-vector products
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed (cited by page and section):
 *   An [N, K] weight W is stored as b-bit codes q (b in {2,3,4,5,6,8}) plus one
 *   bf16 scale s and one bf16 bias z per group of `group_size` consecutive
 *   K-elements of a row; the dequantized weight is w_hat = s*q + z
 *   (mlx-cpu 0.30.1 quantized.h, affine_dequantize).  The products use
 *   w_hat exactly; qdot's regrouping y = s*sum(q*x) + z*sum(x) per group is
 *   the same sum (quantized.h, qdot).
 *
 * Layout of a packed weight (quantized.h, affine_quantize / affine_dequantize;
 * mlx/ops.cpp, extract_quantized_matmul_dims):
 *   w_q    uint32 [N, K*bits/32], row-major.  Row n is a little-endian bit
 *          stream: code k occupies bits [bits*k, bits*k + bits), least
 *          significant bit first; stream bit i is bit (i mod 32) of word
 *          (i div 32).  For 3-, 5- and 6-bit codes this is the page's
 *          8-codes-in-3-bytes, 8-in-5 and 4-in-3 byte packs.
 *   scales, biases   bf16 bit patterns (uint16) [N, K/group_size].
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller; the library
 *     never frees or keeps them.  The only allocation is qmv's stream-ordered
 *     split-K workspace, which lives for one call (see qmv).  bf16 values
 *     travel as uint16 bit patterns.  `stream` is a hipStream_t (NULL = the
 *     legacy default stream).
 *   - Calls are asynchronous on `stream`: they enqueue kernels and return.
 *     Results are visible after the stream is synchronized.
 *   - Arguments are validated on the host before any HIP call.  A bad size,
 *     an unsupported bits/group_size, a null required pointer or K not a
 *     multiple of group_size returns QMV_EINVAL; a valid request this build
 *     does not implement returns QMV_EUNSUPPORTED (never a silent slow path,
 *     as the metrale QuantWeights trait asks of its fused defaults); a HIP
 *     launch error returns QMV_EHIP.  qmv_last_error() then describes it.
 *   - bits in {2,3,4,5,6,8}; group_size in {32,64,128}; K % group_size == 0.
 *   - out_dtype QMV_OUT_BF16 rounds each output once, to nearest even;
 *     QMV_OUT_F32 writes the fp32 accumulator (a debugging mode).
 *   - Index arrays are not range-checked on the host (that needs a device
 *     read).  Out-of-range indices give unspecified results but never read
 *     or write outside the buffers: gather_qmv clamps an lhs index to Bx - 1,
 *     and a pair whose rhs index is >= E is routed to no expert, so its
 *     output rows are left unwritten.
 *   - Concurrent calls on different streams are independent.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    QMV_OK = 0,
    QMV_EINVAL = -1,
    QMV_EUNSUPPORTED = -2,
    QMV_EHIP = -3
};

enum { QMV_OUT_BF16 = 0, QMV_OUT_F32 = 1 };

/*
 * qmv_pack -- quantize and pack an fp32 weight on the device
 * (quantized.h, affine_quantize).  Per group, in IEEE fp32 with correctly
 * rounded division and round-half-away-from-zero:
 *   w_min = min(FLT_MAX, min w), w_max = max(0, max w),
 *   s = max((w_max - w_min)/(2^bits - 1), 1e-7), negated unless
 *   |w_min| > |w_max|; edge = that endpoint; q0 = round(edge/s);
 *   if q0 != 0 then s = edge/q0, z = edge, else z = 0;
 *   q = min(round((w - z)/s), 2^bits - 1);  s and z are stored as bf16
 *   (nearest even), the codes use the fp32 values.
 * w: fp32 [N, K], 16-byte aligned.  Outputs: w_q [N, K*bits/32],
 * scales/biases [N, K/group_size].
 */
int qmv_pack(const float *w, int64_t N, int64_t K, int group_size, int bits,
             uint32_t *w_q, uint16_t *scales, uint16_t *biases, void *stream);

/*
 * qmv -- quantized matmul at decode batch sizes (mlx/ops.cpp quantized_matmul;
 * quantized.h qmv_fast / qmv kernels).
 *   transpose = 1: W packed [N, K]; y[m, n] = sum_k x[m, k] * w_hat[n, k].
 *                  K must be a multiple of group_size.  Up to 4 rows of x:
 *                  the W stream is read once per slab of up to 4 rows.  With
 *                  5 or more rows the matrix cores are used (64-row slabs of
 *                  x, W read once per slab) and K is split into slices;
 *                  for 4-bit codes with K = 2048 or 4096 and at most 16
 *                  rows, in one pass with no slices (K split across the
 *                  waves of a workgroup, no workspace).  That threshold (5)
 *                  can be replaced by a positive integer in the environment
 *                  variable QMV_QMM_MIN_M, and QMV_QMF=0 turns the one-pass
 *                  form off (both read once per process), to time the paths
 *                  on one shape.
 *   transpose = 0: W packed [K, N] (groups along N, quantized.h qvm and its
 *                  split-K variant); y[m, n] = sum_k x[m, k] * w_hat[k, n].
 *                  N must be a multiple of group_size; W is read once per
 *                  slab of up to 4 rows of x, and K is split into slices.
 *   Split-K calls write the slices' fp32 partial sums to a workspace and add
 *   them in slice order in a second kernel, so results are reproducible.
 *   qmv takes that workspace as a stream-ordered allocation
 *   (hipMallocAsync) for the call and frees it on the same stream after the
 *   call's kernels (hipFreeAsync); the library keeps no state between
 *   calls.  Callers that cannot allocate use qmv_with_workspace.
 *   qmv_workspace_bytes reports whether a call splits K.
 * x: bf16 [M, K].  y: [M, N], bf16 or fp32 per out_dtype.  M >= 1.
 * x and w_q must be 16-byte aligned (transpose = 1; w_q for transpose = 0).
 */
int qmv(const uint16_t *x, const uint32_t *w_q, const uint16_t *scales,
        const uint16_t *biases, void *y, int64_t M, int64_t N, int64_t K,
        int group_size, int bits, int transpose, int out_dtype, void *stream);

/*
 * qmv_workspace_bytes -- the workspace (bytes) that qmv_with_workspace needs
 * for a call of these sizes: the split-K partial sums, S slices x (rows of x
 * in one slab) x N fp32 values; 0 when the call does not split K.  Validates
 * the sizes like qmv (QMV_EINVAL / QMV_EUNSUPPORTED) and touches no device.
 */
int qmv_workspace_bytes(int64_t M, int64_t N, int64_t K, int group_size,
                        int bits, int transpose, size_t *bytes);

/*
 * qmv_with_workspace -- qmv with a caller-owned device workspace of
 * workspace_bytes bytes (16-byte aligned; NULL allowed when
 * qmv_workspace_bytes reports 0).  QMV_EINVAL if it is smaller than the call
 * needs.  The library allocates nothing.  The workspace is in use until the
 * call's kernels on `stream` have finished: calls that may run at the same
 * time (other streams, graphs replayed concurrently) need workspaces of
 * their own.  A HIP graph that captures this call keeps the workspace
 * pointer.  Results are bit-identical to qmv's.
 */
int qmv_with_workspace(const uint16_t *x, const uint32_t *w_q,
                       const uint16_t *scales, const uint16_t *biases,
                       void *y, int64_t M, int64_t N, int64_t K,
                       int group_size, int bits, int transpose, int out_dtype,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * qmv_noalloc -- qmv for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same arguments and bit-identical results as qmv, but the
 * split-K partial sums go to a static device array of 16 MiB that the
 * library holds on each GPU it runs on until the process ends; no
 * allocation, no free.  A call that needs more than 16 MiB
 * (qmv_workspace_bytes) returns QMV_EINVAL before any HIP call.  Every call
 * on one GPU shares that GPU's array: calls that may overlap on one GPU
 * (different streams, graphs replayed concurrently) race and must be
 * serialized by the caller.  The array needs no clearing between calls
 * (every slice writes its partial sums before they are read).
 */
int qmv_noalloc(const uint16_t *x, const uint32_t *w_q, const uint16_t *scales,
                const uint16_t *biases, void *y, int64_t M, int64_t N,
                int64_t K, int group_size, int bits, int transpose,
                int out_dtype, void *stream);

/*
 * qmv_gate_up -- dual-output matvec over one input in ONE launch
 * (metrale QuantWeights::gemv_gate_up_with, whose default is two gemv calls;
 * the MlxInt8Weight implementation uses a single launch).
 *   gate_y[n] = sum_k w_hat_g[n, k] x[k],  up_y[n] = sum_k w_hat_u[n, k] x[k]
 * x: bf16 [K]; both weights [N, K] with the same bits and group_size;
 * gate_y, up_y: bf16 [N].  Results equal two qmv calls bit for bit.
 */
int qmv_gate_up(const uint16_t *x,
                const uint32_t *wg, const uint16_t *sg, const uint16_t *bg,
                const uint32_t *wu, const uint16_t *su, const uint16_t *bu,
                uint16_t *gate_y, uint16_t *up_y, int64_t N, int64_t K,
                int group_size, int bits, void *stream);

/*
 * qmv_silu_gate_resid -- fused FFN tail (metrale QuantWeights::
 * gemv_silu_gate_resid and gemv_silu_gate):
 *   y[n] = x_resid[n] + sum_k w_hat[n, k] * silu(gate[k]) * up[k],
 *   silu(v) = v / (1 + exp(-v)).
 * gate, up: bf16 [K]; x_resid: bf16 [N] or NULL (then no residual add);
 * W: [N, K]; y: [N] bf16 or fp32.  silu(gate)*up is formed in fp32 and not
 * rounded; the residual is added in fp32 before the single output rounding.
 */
int qmv_silu_gate_resid(const uint16_t *gate, const uint16_t *up,
                        const uint16_t *x_resid, const uint32_t *w_q,
                        const uint16_t *scales, const uint16_t *biases,
                        void *y, int64_t N, int64_t K, int group_size,
                        int bits, int out_dtype, void *stream);

/*
 * gather_qmv -- expert-gathered matvec (mlx.core.gather_qmm; quantized.h
 * adjust_matrix_offsets for the gather kernels):
 *   for p in [0, P):  y[p] (M x N) = x[lhs[p]] (M x K) @ w_hat[rhs[p]]^T
 * x: bf16 [Bx, M, K];  w_q: [E, N, K*bits/32];  scales/biases: [E, N, K/g];
 * lhs_indices, rhs_indices: uint32 [P] (flat batch indices);  y: [P, M, N].
 * Both index arrays NULL: identical to qmv on x[0] and W[0] (mlx/ops.cpp
 * gather_qmm without indices is quantized_matmul); then P is ignored and y is
 * [M, N].  Exactly one NULL is QMV_EINVAL.  sorted_indices = 1 promises rhs is
 * non-decreasing; it may make the call faster and never changes the results
 * (every output is computed with the same arithmetic either way).
 * transpose must be 1 (else QMV_EUNSUPPORTED).  When the routed x vectors
 * average 5 or more per expert (P*M >= 5*E) the matrix cores are used; the
 * environment variable QMV_GATHER_QMM_MIN (a positive integer, read once per
 * process) replaces that 5.
 * One expert's packed weight (N*K*bits/8 bytes) must be under 2 GiB (else
 * QMV_EUNSUPPORTED): it is addressed with 32-bit offsets.
 * Indices must satisfy lhs[p] < Bx and rhs[p] < E (the pages leave checking
 * them to the caller).  Without a check, a pair with rhs[p] >= E is never
 * routed (its rows of y are not written) and lhs[p] >= Bx reads x row
 * Bx - 1; nothing is read out of bounds.  With the environment variable
 * QMV_DEBUG set (non-empty and not "0"; read on every call) the call first
 * checks every index on the device, waits for the stream, and returns
 * QMV_EINVAL if one is out of range; the check is skipped while the stream
 * is being captured into a HIP graph.
 */
int gather_qmv(const uint16_t *x, int64_t Bx, const uint32_t *w_q,
               const uint16_t *scales, const uint16_t *biases, int64_t E,
               const uint32_t *lhs_indices, const uint32_t *rhs_indices,
               int64_t P, void *y, int64_t M, int64_t N, int64_t K,
               int group_size, int bits, int transpose, int sorted_indices,
               int out_dtype, void *stream);

/*
 * qmv_dequantize -- w_hat[n, k] = scales[n, k/g] * q[n, k] + biases[n, k/g]
 * (mlx-metal quantized.h, affine_dequantize; mlx.core.dequantize), with the
 * stored bf16 scale and bias.  out: [N, K], bf16 (QMV_OUT_BF16) or fp32
 * (QMV_OUT_F32).  Each output is the exact value of s*q + z rounded once to
 * nearest even, so it equals the oracle's exact result rounded the same way,
 * bit for bit.  w_q and out must be 16-byte aligned.  Interop and debugging:
 * not part of the matvec path.
 */
int qmv_dequantize(const uint32_t *w_q, const uint16_t *scales,
                   const uint16_t *biases, void *out, int64_t N, int64_t K,
                   int group_size, int bits, int out_dtype, void *stream);

/*
 * qmv_unpack_codes -- debugging export: runs the qmv kernels' own in-register
 * unpacking on w_q [N, K*bits/32] and writes one code per byte, codes [N, K].
 */
int qmv_unpack_codes(const uint32_t *w_q, int64_t N, int64_t K, int bits,
                     uint8_t *codes, void *stream);

/* Message for the last non-QMV_OK return on the calling thread ("" if none). */
const char *qmv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
