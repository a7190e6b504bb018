/*
 * Drives every entry point of the CPU oracle (oracle/qmv_oracle.c) on small
 * seeded inputs, for every bit width and group size, including its error
 * returns, so that a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * sees each code path.  Also checks two page invariants on the way: unpack
 * inverts pack, and the dequantized weight stays within one scale step of
 * the original.  Prints "ok" and exits 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_bf16_from_f32(float f);
double oracle_f64_from_bf16(uint16_t h);
int oracle_quantize(const float *w, int64_t N, int64_t K, int g, int bits, uint8_t *codes,
                    float *s32, float *b32, uint16_t *s16, uint16_t *b16);
int oracle_pack(const uint8_t *codes, int64_t N, int64_t K, int bits, uint32_t *w);
int oracle_unpack(const uint32_t *w, int64_t N, int64_t K, int bits, uint8_t *codes);
int oracle_dequantize(const uint32_t *w, const uint16_t *s, const uint16_t *b, int64_t N, int64_t K,
                      int g, int bits, double *out);
int oracle_qmv_f64(const uint16_t *x, const uint32_t *w, const uint16_t *s, const uint16_t *b,
                   int64_t M, int64_t N, int64_t K, int g, int bits, double *y);
int oracle_qmv_rows_f64(const uint16_t *x, const uint32_t *w, const uint16_t *s, const uint16_t *b,
                        int64_t M, int64_t N, int64_t K, int g, int bits, const int64_t *rows,
                        int64_t R, double *y);
int oracle_qvm_f64(const uint16_t *x, const uint32_t *w, const uint16_t *s, const uint16_t *b,
                   int64_t M, int64_t N, int64_t K, int g, int bits, double *y);
int oracle_silu_gate_resid_f64(const uint16_t *gate, const uint16_t *up, const uint16_t *x_resid,
                               const uint32_t *w, const uint16_t *s, const uint16_t *b, int64_t N,
                               int64_t K, int g, int bits, double *y);
int oracle_gather_qmv_f64(const uint16_t *x, int64_t Bx, const uint32_t *w, const uint16_t *s,
                          const uint16_t *b, int64_t E, const uint32_t *lhs, const uint32_t *rhs,
                          int64_t P, int64_t M, int64_t N, int64_t K, int g, int bits, double *y);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {            /* splitmix64 -> [0, 1) */
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (double)((z ^ (z >> 31)) >> 11) * (1.0 / 9007199254740992.0);
}
static float normalish(void) { return (float)((uniform() + uniform() + uniform() - 1.5) * 0.04); }

static int failures = 0;
#define CHECK(c, ...) do { if (!(c)) { printf(__VA_ARGS__); printf("\n"); failures++; } } while (0)

static void one(int bits, int g) {
  const int64_t N = 3, K = 2 * g, M = 2, E = 3, P = 5, Bx = 4;
  const int64_t words = K * bits / 32, groups = K / g;
  float *w = malloc(sizeof(float) * E * N * K);
  uint8_t *codes = malloc(E * N * K), *codes2 = malloc(E * N * K);
  float *s32 = malloc(sizeof(float) * E * N * groups), *b32 = malloc(sizeof(float) * E * N * groups);
  uint16_t *s16 = malloc(2 * E * N * groups), *b16 = malloc(2 * E * N * groups);
  uint32_t *wq = malloc(4 * E * N * words);
  double *deq = malloc(sizeof(double) * N * K);
  uint16_t *x = malloc(2 * Bx * M * K), *gate = malloc(2 * K), *up = malloc(2 * K), *xr = malloc(2 * N);
  double *y = malloc(sizeof(double) * (P * M * N + K));   /* also qvm's [1, K] */
  for (int64_t i = 0; i < E * N * K; i++) w[i] = normalish();
  for (int64_t i = 0; i < Bx * M * K; i++) x[i] = oracle_bf16_from_f32((float)(uniform() * 2 - 1));
  for (int64_t i = 0; i < K; i++) {
    gate[i] = oracle_bf16_from_f32((float)(uniform() * 4 - 2));
    up[i] = oracle_bf16_from_f32((float)(uniform() * 2 - 1));
  }
  for (int64_t i = 0; i < N; i++) xr[i] = oracle_bf16_from_f32((float)uniform());

  CHECK(oracle_quantize(w, E * N, K, g, bits, codes, s32, b32, s16, b16) == 0, "quantize b%d g%d", bits, g);
  CHECK(oracle_pack(codes, E * N, K, bits, wq) == 0, "pack b%d g%d", bits, g);
  CHECK(oracle_unpack(wq, E * N, K, bits, codes2) == 0, "unpack b%d g%d", bits, g);
  CHECK(memcmp(codes, codes2, E * N * K) == 0, "unpack does not invert pack: b%d g%d", bits, g);
  CHECK(oracle_dequantize(wq, s16, b16, N, K, g, bits, deq) == 0, "dequantize b%d g%d", bits, g);
  for (int64_t n = 0; n < N; n++)
    for (int64_t k = 0; k < K; k++) {
      const double s = fabs(oracle_f64_from_bf16(s16[n * groups + k / g]));
      const double z = fabs(oracle_f64_from_bf16(b16[n * groups + k / g]));
      CHECK(fabs(deq[n * K + k] - w[n * K + k]) <= s + 0.01 * (s * 255 + z) + 1e-12,
            "dequantized weight off by more than a step: b%d g%d n%lld k%lld", bits, g, (long long)n,
            (long long)k);
    }
  CHECK(oracle_qmv_f64(x, wq, s16, b16, M, N, K, g, bits, y) == 0, "qmv b%d g%d", bits, g);
  const int64_t rows[2] = {2, 0};
  CHECK(oracle_qmv_rows_f64(x, wq, s16, b16, M, N, K, g, bits, rows, 2, y) == 0, "qmv_rows b%d g%d", bits, g);
  /* the same words read as transpose = 0 data: W [N, K] quantized along its K */
  CHECK(oracle_qvm_f64(x, wq, s16, b16, 1, K, N, g, bits, y) == 0, "qvm b%d g%d", bits, g);
  CHECK(oracle_silu_gate_resid_f64(gate, up, xr, wq, s16, b16, N, K, g, bits, y) == 0, "silu b%d g%d", bits, g);
  CHECK(oracle_silu_gate_resid_f64(gate, up, NULL, wq, s16, b16, N, K, g, bits, y) == 0, "silu no resid b%d g%d",
        bits, g);
  uint32_t lhs[5], rhs[5];
  for (int p = 0; p < P; p++) { lhs[p] = (uint32_t)(uniform() * Bx); rhs[p] = (uint32_t)(uniform() * E); }
  CHECK(oracle_gather_qmv_f64(x, Bx, wq, s16, b16, E, lhs, rhs, P, M, N, K, g, bits, y) == 0, "gather b%d g%d",
        bits, g);
  rhs[3] = (uint32_t)E;
  CHECK(oracle_gather_qmv_f64(x, Bx, wq, s16, b16, E, lhs, rhs, P, M, N, K, g, bits, y) == -3,
        "gather accepts rhs out of range: b%d g%d", bits, g);
  rhs[3] = 0; lhs[1] = (uint32_t)Bx;
  CHECK(oracle_gather_qmv_f64(x, Bx, wq, s16, b16, E, lhs, rhs, P, M, N, K, g, bits, y) == -3,
        "gather accepts lhs out of range: b%d g%d", bits, g);
  /* bad shapes are refused before any access */
  CHECK(oracle_qmv_f64(x, wq, s16, b16, M, N, K + g / 2, g, bits, y) != 0, "qmv accepts K %% g != 0");
  CHECK(oracle_quantize(w, N, K + g / 2, g, bits, codes, s32, b32, s16, b16) != 0, "quantize accepts K %% g != 0");
  free(w); free(codes); free(codes2); free(s32); free(b32); free(s16); free(b16); free(wq); free(deq);
  free(x); free(gate); free(up); free(xr); free(y);
}

int main(void) {
  const int bits[6] = {2, 3, 4, 5, 6, 8}, groups[3] = {32, 64, 128};
  for (int i = 0; i < 6; i++)
    for (int j = 0; j < 3; j++) one(bits[i], groups[j]);
  if (failures) { printf("%d failures\n", failures); return 1; }
  printf("ok\n");
  return 0;
}
