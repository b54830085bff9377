/*
 * Sanitizer driver for the CPU oracle (test infrastructure only).
 *
 * Built together with nf4_oracle.c under -fsanitize=address,undefined by
 * tests/test_oracle_sanitized.py and run as a plain executable: it calls every
 * entry point of the oracle on small seeded inputs, including the refusal paths
 * and the edge shapes (empty tensors, partial double-quant groups, block sizes
 * that are not powers of two, ranks 1 and odd, the sampled forms), so that an
 * out-of-bounds access, a use of uninitialised heap memory under ASan's poisoning,
 * or undefined arithmetic in the oracle ends the process with a report.  The
 * results themselves are checked elsewhere (the oracle's pins); here only a few
 * self-consistency checks keep every output live.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_nf4_levels(double lv64[16], float lv32[16]);
int orc_nf4_quantize(const float* w, int64_t n, int32_t bs, int32_t dq, int32_t g, uint8_t* packed, float* absmax,
                     uint8_t* absmax_q, float* scale2, uint8_t* codes_out);
int orc_nf4_dequantize(const uint8_t* packed, int64_t n, int32_t bs, int32_t dq, int32_t g, const float* absmax,
                       const uint8_t* absmax_q, const float* scale2, float* out);
void orc_f32_to_bf16(const float* in, uint16_t* out, int64_t n);
void orc_f32_to_f16(const float* in, uint16_t* out, int64_t n);
void orc_bf16_to_f32(const uint16_t* in, float* out, int64_t n);
void orc_f16_to_f32(const uint16_t* in, float* out, int64_t n);
void orc_qlora_fwd(const float* x, const float* W, const float* A, const float* B, const float* bias, int64_t M,
                   int64_t N, int64_t K, int64_t r, double s, double* y);
void orc_qlora_fwd_at(const float* x, const float* W, const float* A, const float* B, const float* bias, int64_t M,
                      int64_t N, int64_t K, int64_t r, double s, const int64_t* ii, const int64_t* jj, int64_t ns,
                      double* out);
void orc_qlora_bwd(const float* x, const float* W, const float* A, const float* B, const float* dY, int64_t M,
                   int64_t N, int64_t K, int64_t r, double s, double* dX, double* dA, double* dB);
void orc_qlora_bwd_dx_at(const float* dY, const float* W, const float* A, const float* B, int64_t M, int64_t N,
                         int64_t K, int64_t r, double s, const int64_t* ii, const int64_t* kk, int64_t ns,
                         double* out);
void orc_qlora_bwd_da_at(const float* x, const float* dY, const float* B, int64_t M, int64_t N, int64_t K, int64_t r,
                         double s, const int64_t* tt, const int64_t* kk, int64_t ns, double* out);
void orc_qlora_bwd_db_at(const float* x, const float* A, const float* dY, int64_t M, int64_t N, int64_t K, int64_t r,
                         double s, const int64_t* nn, const int64_t* tt, int64_t ns, double* out);
void orc_qlora_merge(const float* what, const float* A, const float* B, int64_t N, int64_t K, int64_t r, double s,
                     int32_t kind, void* out);
void orc_round_f64(const double* in, int64_t n, int32_t kind, void* out);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
/* splitmix64 (input generation only) */
static double uniform(void) {
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return (double)(z >> 11) / 9007199254740992.0;
}
static float* fill(int64_t n, double sigma) {
  float* p = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  for (int64_t i = 0; i < n; ++i) p[i] = (float)((uniform() * 2.0 - 1.0) * sigma);
  return p;
}

static int failures = 0;
#define EXPECT(c)                                               \
  do {                                                          \
    if (!(c)) {                                                 \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                               \
    }                                                           \
  } while (0)

static void quant_case(int64_t n, int32_t bs, int32_t dq, int32_t g) {
  float* w = fill(n, 3.0);
  if (n > 2) w[1] = 0.0f;
  const int64_t nb = n / bs, ng = dq ? (nb + g - 1) / g : 0;
  uint8_t* packed = (uint8_t*)malloc((size_t)(n / 2 > 0 ? n / 2 : 1));
  uint8_t* codes = (uint8_t*)malloc((size_t)(n > 0 ? n : 1));
  float* absmax = dq ? NULL : (float*)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(float));
  uint8_t* aq = dq ? (uint8_t*)malloc((size_t)(nb > 0 ? nb : 1)) : NULL;
  float* s2 = dq ? (float*)malloc((size_t)(ng > 0 ? ng : 1) * sizeof(float)) : NULL;
  EXPECT(orc_nf4_quantize(w, n, bs, dq, g, packed, absmax, aq, s2, codes) == 0);
  float* out = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  EXPECT(orc_nf4_dequantize(packed, n, bs, dq, g, absmax, aq, s2, out) == 0);
  for (int64_t i = 0; i < n; ++i) EXPECT(isfinite(out[i]) && codes[i] < 16);
  free(w), free(packed), free(codes), free(absmax), free(aq), free(s2), free(out);
}

static void layer_case(int64_t M, int64_t N, int64_t K, int64_t r, int with_bias) {
  float *x = fill(M * K, 1.0), *W = fill(N * K, 0.02), *A = fill(r * K, 0.3), *B = fill(N * r, 0.01);
  float *dY = fill(M * N, 1.0), *bias = with_bias ? fill(N, 0.1) : NULL;
  const double s = 2.0;
  double* y = (double*)malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(double));
  orc_qlora_fwd(x, W, A, B, bias, M, N, K, r, s, y);
  int64_t ii[5], jj[5], tt[5], kk[5];
  for (int e = 0; e < 5; ++e) {
    ii[e] = (e * 7) % M;
    jj[e] = (e * 11) % N;
    tt[e] = (e * 3) % r;
    kk[e] = (e * 5) % K;
  }
  double at[5];
  orc_qlora_fwd_at(x, W, A, B, bias, M, N, K, r, s, ii, jj, 5, at);
  for (int e = 0; e < 5; ++e) EXPECT(fabs(at[e] - y[ii[e] * N + jj[e]]) <= 1e-9 * (1.0 + fabs(at[e])));
  double* dX = (double*)malloc((size_t)(M * K) * sizeof(double));
  double* dA = (double*)malloc((size_t)(r * K) * sizeof(double));
  double* dB = (double*)malloc((size_t)(N * r) * sizeof(double));
  orc_qlora_bwd(x, W, A, B, dY, M, N, K, r, s, dX, dA, dB);
  orc_qlora_bwd(x, W, A, B, dY, M, N, K, r, s, NULL, dA, NULL);  /* partial requests */
  orc_qlora_bwd_dx_at(dY, W, A, B, M, N, K, r, s, ii, kk, 5, at);
  for (int e = 0; e < 5; ++e) EXPECT(fabs(at[e] - dX[ii[e] * K + kk[e]]) <= 1e-9 * (1.0 + fabs(at[e])));
  orc_qlora_bwd_da_at(x, dY, B, M, N, K, r, s, tt, kk, 5, at);
  for (int e = 0; e < 5; ++e) EXPECT(fabs(at[e] - dA[tt[e] * K + kk[e]]) <= 1e-9 * (1.0 + fabs(at[e])));
  orc_qlora_bwd_db_at(x, A, dY, M, N, K, r, s, jj, tt, 5, at);
  for (int e = 0; e < 5; ++e) EXPECT(fabs(at[e] - dB[jj[e] * r + tt[e]]) <= 1e-9 * (1.0 + fabs(at[e])));
  for (int kind = 0; kind < 3; ++kind) {
    void* out = malloc((size_t)(N * K) * 4);
    orc_qlora_merge(W, A, B, N, K, r, s, kind, out);
    free(out);
  }
  free(x), free(W), free(A), free(B), free(dY), free(bias), free(y), free(dX), free(dA), free(dB);
}

int main(void) {
  double lv64[16];
  float lv32[16];
  orc_nf4_levels(lv64, lv32);
  EXPECT(lv32[0] == -1.0f && lv32[7] == 0.0f && lv32[15] == 1.0f);

  /* block sizes (powers of two and not), partial double-quant groups, one global group */
  quant_case(64 * 64, 64, 0, 1);
  quant_case(64 * 64, 64, 1, 256);
  quant_case(30, 2, 1, 4);
  quant_case(30, 6, 1, 2);
  quant_case(96 * 7, 96, 1, 3);
  quant_case(1000 * 3, 1000, 0, 1);
  quant_case(512, 8, 1, 1000);
  quant_case(0, 64, 1, 256); /* empty */

  /* refusals: odd block, n not a multiple of the block, missing outputs */
  {
    float w[8] = {0};
    uint8_t packed[4], aq[4];
    float am[4], s2[4];
    EXPECT(orc_nf4_quantize(w, 8, 3, 0, 1, packed, am, NULL, NULL, NULL) != 0);
    EXPECT(orc_nf4_quantize(w, 8, 6, 0, 1, packed, am, NULL, NULL, NULL) != 0);
    EXPECT(orc_nf4_quantize(w, 8, 2, 1, 0, packed, NULL, aq, s2, NULL) != 0);
    EXPECT(orc_nf4_quantize(w, 8, 2, 0, 1, packed, NULL, NULL, NULL, NULL) != 0);
    float out[8];
    EXPECT(orc_nf4_dequantize(packed, 8, 3, 0, 1, am, NULL, NULL, out) != 0);
    w[3] = NAN;
    EXPECT(orc_nf4_quantize(w, 8, 2, 0, 1, packed, am, NULL, NULL, NULL) != 0);
  }

  /* dtype conversions, including subnormals, ties, overflow, NaN and infinities */
  {
    float in[12] = {0.0f, -0.0f, 1.0f, 65504.0f, 65520.0f, 1e-8f, -1e-40f, 3.0e38f, INFINITY, -INFINITY, NAN,
                    1.00390625f};
    uint16_t b[12], h[12];
    float back[12];
    orc_f32_to_bf16(in, b, 12);
    orc_f32_to_f16(in, h, 12);
    orc_bf16_to_f32(b, back, 12);
    orc_f16_to_f32(h, back, 12);
    double d[6] = {1.0, 1.0 + 1.0 / 512.0, 65519.99, 1e-300, -2.5, 1e300};
    float f32[6];
    uint16_t u16[6];
    orc_round_f64(d, 6, 0, f32);
    orc_round_f64(d, 6, 1, u16);
    orc_round_f64(d, 6, 2, u16);
  }

  /* the layer: ragged shapes, rank 1, odd rank, with and without bias */
  layer_case(5, 7, 9, 1, 0);
  layer_case(8, 16, 32, 3, 1);
  layer_case(13, 6, 10, 5, 1);

  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer run: ok\n");
  return 0;
}
