/*
 * Plain CPU oracle for the affine group-quantized matrix-vector product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library: every routine below is written from the source pages, in the
 * plainest form that makes it checkable by eye.
 *
 * Sources (cited by page and section; the reader has the pages):
 *   [Q]  mlx-cpu 0.30.1 wheel, mlx/include/mlx/backend/metal/kernels/quantized.h
 *        (diffend.io view): get_pack_factor / get_bytes_per_pack, qdot,
 *        affine_quantize, affine_dequantize, adjust_matrix_offsets (gather).
 *   [OPS] zhangyiss/mlx compare split_logsumexp...trellis-quants, mlx/ops.cpp
 *        hunks: extract_quantized_matmul_dims, quantized_matmul, gather_qmm.
 *   [QW] metrale docs, trait QuantWeights (rendered docs and quant_weights.rs):
 *        gemv, gemv_gate_up_with, gemv_silu_gate, gemv_silu_gate_resid.
 *   [GQ] mlx.core.gather_qmm documentation page.
 *
 * Precision: the quantizer is IEEE fp32, step by step, as [Q] affine_quantize
 * states it; everything after dequantization is fp64.  Build with
 * -ffp-contract=off and without fast-math so that each fp32 operation is one
 * correctly rounded IEEE operation.
 *
 * Every function here has a pin in the CPU test suite (layout against the
 * page's byte formulas, bijection, closed-form quantizer cases, brute-force
 * rational arithmetic, one-hot addressing, silu against a library routine).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32/fp64.  bf16 is the top 16 bits of an fp32; the narrowing   */
/* rounds to nearest, ties to even (the reading of static_cast<T> in [Q]    */
/* affine_quantize for a bfloat16 T).  NaN/Inf inputs are not defined here. */
/* ------------------------------------------------------------------------ */
uint16_t oracle_bf16_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u)))
        keep += 1u;
    return (uint16_t)keep;
}

double oracle_f64_from_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Quantize ([Q] affine_quantize).  One group = g consecutive K-elements of  */
/* one row.  Steps, all in fp32:                                             */
/*   n_bins = 2^bits - 1, eps = 1e-7                                          */
/*   w_min  = min(FLT_MAX, min_i w_i);  w_max = max(0, max_i w_i)             */
/*   scale  = max((w_max - w_min) / n_bins, eps)                              */
/*   side   = |w_min| > |w_max|;  scale = side ? scale : -scale               */
/*   edge   = side ? w_min : w_max                                            */
/*   q0     = round(edge / scale)                                             */
/*   if q0 == 0: bias = 0 (scale kept)   else: scale = edge / q0, bias = edge */
/*   q_i    = (uint8) min(round((w_i - bias) / scale), n_bins)                */
/* The stored scale and bias are the fp32 values narrowed to bf16; the codes */
/* use the unrounded fp32 scale and bias.  round() is half away from zero.   */
/* ------------------------------------------------------------------------ */
static void quantize_group(const float *w, int g, int bits, uint8_t *q,
                           float *scale_out, float *bias_out)
{
    const float n_bins = (float)((1 << bits) - 1);
    const float eps = 1e-7f;

    float w_min = FLT_MAX;
    float w_max = 0.0f;
    for (int i = 0; i < g; i++) {
        if (w[i] < w_min) w_min = w[i];
        if (w[i] > w_max) w_max = w[i];
    }

    float range = w_max - w_min;
    float scale = range / n_bins;
    if (scale < eps) scale = eps;
    int side = fabsf(w_min) > fabsf(w_max);
    if (!side) scale = -scale;
    float edge = side ? w_min : w_max;
    float q0 = roundf(edge / scale);
    float bias;
    if (q0 == 0.0f) {
        bias = 0.0f;
    } else {
        scale = edge / q0;
        bias = edge;
    }

    for (int i = 0; i < g; i++) {
        float diff = w[i] - bias;
        float r = roundf(diff / scale);
        if (r > n_bins) r = n_bins;
        q[i] = (uint8_t)(int)r;
    }
    *scale_out = scale;
    *bias_out = bias;
}

/* w [N,K] fp32 row-major.  codes [N,K] one byte per code.  s32/b32/s16/b16 */
/* [N, K/g].  Any of s32/b32 may be NULL.  Returns 0, or -1 on bad sizes.    */
int oracle_quantize(const float *w, int64_t N, int64_t K, int g, int bits,
                    uint8_t *codes, float *s32, float *b32,
                    uint16_t *s16, uint16_t *b16)
{
    if (N <= 0 || K <= 0 || g <= 0 || K % g != 0 || bits < 1 || bits > 8)
        return -1;
    int64_t groups = K / g;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t j = 0; j < groups; j++) {
            float s, b;
            int64_t base = n * K + j * g;
            quantize_group(w + base, g, bits, codes + base, &s, &b);
            int64_t gi = n * groups + j;
            if (s32) s32[gi] = s;
            if (b32) b32[gi] = b;
            s16[gi] = oracle_bf16_from_f32(s);
            b16[gi] = oracle_bf16_from_f32(b);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Pack / unpack.  Each row is a little-endian bit stream of K*bits bits:    */
/* code k occupies stream bits [bits*k, bits*k + bits), least significant    */
/* bit first; stream bit i is bit (i mod 32) of uint32 word (i div 32).  For */
/* bits in {2,4,8} this is the shift layout of [Q] affine_quantize / the      */
/* per-word reads of affine_dequantize; for 3/5/6 it is the LSB-first byte   */
/* packs (8 codes in 3 bytes, 8 in 5, 4 in 3) that affine_dequantize reads.  */
/* Written one bit at a time on purpose.                                     */
/* ------------------------------------------------------------------------ */
int oracle_pack(const uint8_t *codes, int64_t N, int64_t K, int bits,
                uint32_t *w)
{
    if (N <= 0 || K <= 0 || bits < 1 || bits > 8 || (K * bits) % 32 != 0)
        return -1;
    int64_t words = K * bits / 32;
    memset(w, 0, (size_t)(N * words) * sizeof(uint32_t));
    for (int64_t n = 0; n < N; n++) {
        uint32_t *row = w + n * words;
        for (int64_t k = 0; k < K; k++) {
            unsigned c = codes[n * K + k];
            for (int j = 0; j < bits; j++) {
                if ((c >> j) & 1u) {
                    int64_t bit = k * bits + j;
                    row[bit / 32] |= 1u << (bit % 32);
                }
            }
        }
    }
    return 0;
}

int oracle_unpack(const uint32_t *w, int64_t N, int64_t K, int bits,
                  uint8_t *codes)
{
    if (N <= 0 || K <= 0 || bits < 1 || bits > 8 || (K * bits) % 32 != 0)
        return -1;
    int64_t words = K * bits / 32;
    for (int64_t n = 0; n < N; n++) {
        const uint32_t *row = w + n * words;
        for (int64_t k = 0; k < K; k++) {
            unsigned c = 0;
            for (int j = 0; j < bits; j++) {
                int64_t bit = k * bits + j;
                c |= ((row[bit / 32] >> (bit % 32)) & 1u) << j;
            }
            codes[n * K + k] = (uint8_t)c;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantize ([Q] affine_dequantize): w_hat = scale * q + bias per group,   */
/* with the stored bf16 scale and bias, evaluated exactly in fp64 (8-bit by  */
/* 8-bit significands plus an 8-bit addend fit in 53 bits).                  */
/* ------------------------------------------------------------------------ */
static void dequant_row(const uint32_t *wrow, const uint16_t *srow,
                        const uint16_t *brow, int64_t K, int g, int bits,
                        uint8_t *tmp_codes, double *out)
{
    oracle_unpack(wrow, 1, K, bits, tmp_codes);
    for (int64_t k = 0; k < K; k++) {
        double s = oracle_f64_from_bf16(srow[k / g]);
        double b = oracle_f64_from_bf16(brow[k / g]);
        out[k] = s * (double)tmp_codes[k] + b;
    }
}

int oracle_dequantize(const uint32_t *w, const uint16_t *s, const uint16_t *b,
                      int64_t N, int64_t K, int g, int bits, double *out)
{
    if (N <= 0 || K <= 0 || g <= 0 || K % g != 0 || (K * bits) % 32 != 0)
        return -1;
    int64_t words = K * bits / 32, groups = K / g;
    uint8_t *tmp = (uint8_t *)malloc((size_t)K);
    if (!tmp) return -2;
    for (int64_t n = 0; n < N; n++)
        dequant_row(w + n * words, s + n * groups, b + n * groups, K, g, bits,
                    tmp, out + n * K);
    free(tmp);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* qmv with transpose: y[m,n] = sum_k w_hat[n,k] * x[m,k]  (the plain        */
/* definition of x @ W^T for the dequantized W; [Q] qdot's fold              */
/* scale*sum(q*x) + bias*sum(x) is the same sum regrouped).  x is bf16 bits. */
/* ------------------------------------------------------------------------ */
int oracle_qmv_f64(const uint16_t *x, const uint32_t *w, const uint16_t *s,
                   const uint16_t *b, int64_t M, int64_t N, int64_t K, int g,
                   int bits, double *y)
{
    if (M <= 0 || N <= 0 || K <= 0 || g <= 0 || K % g != 0 ||
        (K * bits) % 32 != 0)
        return -1;
    int64_t words = K * bits / 32, groups = K / g;
    uint8_t *tmp = (uint8_t *)malloc((size_t)K);
    double *row = (double *)malloc((size_t)K * sizeof(double));
    double *xd = (double *)malloc((size_t)(M * K) * sizeof(double));
    if (!tmp || !row || !xd) { free(tmp); free(row); free(xd); return -2; }
    for (int64_t i = 0; i < M * K; i++) xd[i] = oracle_f64_from_bf16(x[i]);
    for (int64_t n = 0; n < N; n++) {
        dequant_row(w + n * words, s + n * groups, b + n * groups, K, g, bits,
                    tmp, row);
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) acc += row[k] * xd[m * K + k];
            y[m * N + n] = acc;
        }
    }
    free(tmp); free(row); free(xd);
    return 0;
}

/* Same product restricted to a list of output rows (for sampled checks at  */
/* full size): y[m, i] = (x @ W^T)[m, rows[i]].                              */
int oracle_qmv_rows_f64(const uint16_t *x, const uint32_t *w,
                        const uint16_t *s, const uint16_t *b, int64_t M,
                        int64_t N, int64_t K, int g, int bits,
                        const int64_t *rows, int64_t R, double *y)
{
    if (M <= 0 || N <= 0 || K <= 0 || g <= 0 || K % g != 0 ||
        (K * bits) % 32 != 0)
        return -1;
    int64_t words = K * bits / 32, groups = K / g;
    uint8_t *tmp = (uint8_t *)malloc((size_t)K);
    double *row = (double *)malloc((size_t)K * sizeof(double));
    if (!tmp || !row) { free(tmp); free(row); return -2; }
    for (int64_t i = 0; i < R; i++) {
        int64_t n = rows[i];
        if (n < 0 || n >= N) { free(tmp); free(row); return -1; }
        dequant_row(w + n * words, s + n * groups, b + n * groups, K, g, bits,
                    tmp, row);
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++)
                acc += row[k] * oracle_f64_from_bf16(x[m * K + k]);
            y[m * R + i] = acc;
        }
    }
    free(tmp); free(row);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* qmv without transpose ([GQ] transpose=False, x @ W): W is [K, N] packed    */
/* along N with groups of g consecutive N-elements; y[m,n] = sum_k x[m,k] *  */
/* w_hat[k,n].                                                                */
/* ------------------------------------------------------------------------ */
int oracle_qvm_f64(const uint16_t *x, const uint32_t *w, const uint16_t *s,
                   const uint16_t *b, int64_t M, int64_t N, int64_t K, int g,
                   int bits, double *y)
{
    if (M <= 0 || N <= 0 || K <= 0 || g <= 0 || N % g != 0 ||
        (N * bits) % 32 != 0)
        return -1;
    int64_t words = N * bits / 32, groups = N / g;
    uint8_t *tmp = (uint8_t *)malloc((size_t)N);
    double *row = (double *)malloc((size_t)N * sizeof(double));
    if (!tmp || !row) { free(tmp); free(row); return -2; }
    for (int64_t i = 0; i < M * N; i++) y[i] = 0.0;
    for (int64_t k = 0; k < K; k++) {
        dequant_row(w + k * words, s + k * groups, b + k * groups, N, g, bits,
                    tmp, row);
        for (int64_t m = 0; m < M; m++) {
            double xv = oracle_f64_from_bf16(x[m * K + k]);
            for (int64_t n = 0; n < N; n++) y[m * N + n] += xv * row[n];
        }
    }
    free(tmp); free(row);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* FFN tail ([QW] gemv_silu_gate / gemv_silu_gate_resid):                     */
/*   h[k] = silu(gate[k]) * up[k],  silu(v) = v / (1 + exp(-v))               */
/*   y[n] = x_resid[n] + sum_k w_hat[n,k] * h[k]   (x_resid NULL: no add)     */
/* gate, up, x_resid are bf16 bits; all arithmetic is fp64.                   */
/* ------------------------------------------------------------------------ */
int oracle_silu_gate_resid_f64(const uint16_t *gate, const uint16_t *up,
                               const uint16_t *x_resid, const uint32_t *w,
                               const uint16_t *s, const uint16_t *b,
                               int64_t N, int64_t K, int g, int bits,
                               double *y)
{
    if (N <= 0 || K <= 0 || g <= 0 || K % g != 0 || (K * bits) % 32 != 0)
        return -1;
    int64_t words = K * bits / 32, groups = K / g;
    uint8_t *tmp = (uint8_t *)malloc((size_t)K);
    double *row = (double *)malloc((size_t)K * sizeof(double));
    double *h = (double *)malloc((size_t)K * sizeof(double));
    if (!tmp || !row || !h) { free(tmp); free(row); free(h); return -2; }
    for (int64_t k = 0; k < K; k++) {
        double gv = oracle_f64_from_bf16(gate[k]);
        double uv = oracle_f64_from_bf16(up[k]);
        h[k] = gv / (1.0 + exp(-gv)) * uv;
    }
    for (int64_t n = 0; n < N; n++) {
        dequant_row(w + n * words, s + n * groups, b + n * groups, K, g, bits,
                    tmp, row);
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++) acc += row[k] * h[k];
        y[n] = (x_resid ? oracle_f64_from_bf16(x_resid[n]) : 0.0) + acc;
    }
    free(tmp); free(row); free(h);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Gather ([Q] adjust_matrix_offsets for the gather kernels; [OPS]          */
/* gather_qmm; [GQ]).  For each flat pair p: x_idx = lhs[p], w_idx = rhs[p]; */
/*   y[p] (M x N) = x[x_idx] (M x K) @ W[w_idx]^T                              */
/* x: [Bx, M, K] bf16; W: [E, N, K*bits/32]; s, b: [E, N, K/g]; y: [P, M, N]. */
/* Returns -3 if an index is out of range.                                   */
/* ------------------------------------------------------------------------ */
int oracle_gather_qmv_f64(const uint16_t *x, int64_t Bx, const uint32_t *w,
                          const uint16_t *s, const uint16_t *b, int64_t E,
                          const uint32_t *lhs, const uint32_t *rhs, int64_t P,
                          int64_t M, int64_t N, int64_t K, int g, int bits,
                          double *y)
{
    if (Bx <= 0 || E <= 0 || P <= 0 || M <= 0 || N <= 0 || K <= 0 || g <= 0 ||
        K % g != 0 || (K * bits) % 32 != 0)
        return -1;
    int64_t wsz = N * (K * bits / 32), ssz = N * (K / g);
    for (int64_t p = 0; p < P; p++) {
        if ((int64_t)lhs[p] >= Bx || (int64_t)rhs[p] >= E) return -3;
        int rc = oracle_qmv_f64(x + (int64_t)lhs[p] * M * K,
                                w + (int64_t)rhs[p] * wsz,
                                s + (int64_t)rhs[p] * ssz,
                                b + (int64_t)rhs[p] * ssz, M, N, K, g, bits,
                                y + p * M * N);
        if (rc) return rc;
    }
    return 0;
}
