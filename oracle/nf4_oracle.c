/*
 * nf4_oracle.c -- the CPU oracle for the QLoRA NF4 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, link or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * do.  It shares no code, header, table or constant with the HIP library.
 *
 * Style: plain scalar C, one loop per definition, no blocking, no fusion.  Every
 * contraction accumulates in IEEE binary64.  Quantities that the method defines in
 * binary32 (the normalised weight, the block scale, the dequantised weight) are
 * computed in binary32 with round-to-nearest-even, because that is the precision
 * the method stores them in.
 *
 * Sources (the pages):
 *   [R]  qlora-rs README -- "Honest capability matrix" (block absmax scales, NF4
 *        pack/unpack, double quant to u8 with one scale-of-scales), "NF4
 *        Quantization" (the 16 printed levels), "Double quantization (simplified)".
 *   [C]  rust_ai_core QLoraConfig docs -- scale() = alpha / r; compute dtype.
 *   [B]  "LoRA and QLoRA, mathematically" -- "NF4: quantizing the frozen base"
 *        (levels at the quantiles of a normal distribution) and eq. (6.3.6).
 *   [E]  qlora-rs src/export.rs -- tests that quantize all-zero and all-one weights
 *        and a 32x32 tensor with block 64 (blocks run over the flattened tensor).
 *
 * Readings taken where the pages are silent:
 *   levels   normalised normal quantiles with offset d = (1-1/30)/2 + (1-1/32)/2,
 *            8 positive and 7 negative quantiles plus an exact zero, divided by
 *            the largest, rounded once to binary32;
 *   nearest  ties between two levels go to the lower code;
 *   nibbles  element 2k is stored in the high nibble of byte k;
 *   zeros    a block whose absmax is 0 gets code 7 (level 0) and scale 0;
 *   DQ       groups of g consecutive block scales; S = fl32(max/255);
 *            q = round-half-even(a/S) evaluated exactly, clamped to [0,255];
 *            the 4-bit codes are always taken against the binary32 absmax.
 *
 * Parity pins: every function here is checked by tests/test_oracle_*.py against
 * the printed level table, closed forms, brute force on small inputs, library
 * routines (scipy ndtri, numpy float16 casts, torch fp64 autograd) and
 * invariants (idempotence, B = 0, linearity in alpha, the merge identity).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_SHAPE (-2)
#define ORC_ERR_NONFINITE (-3)
#define ORC_ERR_NOMEM (-4)

/* ------------------------------------------------------------------------- */
/* Level table: 16 levels at normal quantiles, [B] "NF4: quantizing the frozen
 * base"; printed to three decimals in [R] "NF4 Quantization".                  */
/* ------------------------------------------------------------------------- */

/* Standard normal CDF, written from its definition through erfc. */
static double normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Inverse CDF by bisection: slow, monotone, and accurate to the last few ulps. */
static double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 4000; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (normal_cdf(mid) < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

void orc_nf4_levels(double lv64[16], float lv32[16]) {
  const double d = 0.5 * (1.0 - 1.0 / 30.0) + 0.5 * (1.0 - 1.0 / 32.0);
  const double top = normal_quantile(d);
  int idx = 0;
  /* 7 negative levels: quantiles at d - j(d - 1/2)/7, j = 0..6, negated. */
  for (int j = 0; j <= 6; ++j)
    lv64[idx++] = -normal_quantile(d - j * (d - 0.5) / 7.0) / top;
  lv64[idx++] = 0.0;
  /* 8 positive levels: quantiles at d - j(d - 1/2)/8, j = 7..0 (ascending). */
  for (int j = 7; j >= 0; --j)
    lv64[idx++] = normal_quantile(d - j * (d - 0.5) / 8.0) / top;
  for (int i = 0; i < 16; ++i) lv32[i] = (float)lv64[i];
}

/* ------------------------------------------------------------------------- */
/* Quantize: block absmax [R] matrix; nearest level; two codes per byte.       */
/* ------------------------------------------------------------------------- */

/* code = number of midpoints m_j = (L_j + L_{j+1})/2 strictly below x, i.e. the
 * nearest level with ties to the lower code.  The midpoints are exact in fp64. */
static int nearest_code(float x, const float lv[16]) {
  int c = 0;
  for (int j = 0; j < 15; ++j) {
    double m = ((double)lv[j] + (double)lv[j + 1]) / 2.0;
    if ((double)x > m) ++c;
  }
  return c;
}

int orc_nf4_quantize(const float* w, int64_t n, int32_t bs, int32_t dq, int32_t g,
                     uint8_t* packed, float* absmax, uint8_t* absmax_q, float* scale2,
                     uint8_t* codes_out /* optional, n bytes, one code per byte */) {
  if (!w || !packed || bs <= 0 || n < 0) return ORC_ERR_ARG;
  if (bs % 2 != 0 || n % bs != 0) return ORC_ERR_SHAPE;
  if (dq && (g <= 0 || !absmax_q || !scale2)) return ORC_ERR_ARG;
  if (!dq && !absmax) return ORC_ERR_ARG;
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(w[i])) return ORC_ERR_NONFINITE;

  double lv64[16];
  float lv[16];
  orc_nf4_levels(lv64, lv);

  const int64_t nb = n / bs;
  float* am = dq ? (float*)malloc((size_t)(nb ? nb : 1) * sizeof(float)) : absmax;
  uint8_t* codes = (uint8_t*)malloc((size_t)(n ? n : 1));
  if (!am || !codes) {
    if (dq) free(am);
    free(codes);
    return ORC_ERR_NOMEM;
  }

  for (int64_t b = 0; b < nb; ++b) {
    const float* wb = w + b * bs;
    float a = 0.0f;
    for (int32_t i = 0; i < bs; ++i) {
      float v = fabsf(wb[i]);
      if (v > a) a = v;
    }
    am[b] = a;
    for (int32_t i = 0; i < bs; ++i) {
      /* binary32 division, correctly rounded (C float arithmetic on SSE). */
      float x = (a == 0.0f) ? 0.0f : wb[i] / a;
      codes[b * bs + i] = (uint8_t)nearest_code(x, lv);
    }
  }

  for (int64_t k = 0; k < n / 2; ++k)
    packed[k] = (uint8_t)((codes[2 * k] << 4) | codes[2 * k + 1]);
  if (codes_out) memcpy(codes_out, codes, (size_t)n);

  if (dq) {
    const int64_t ng = (nb + g - 1) / g;
    for (int64_t G = 0; G < ng; ++G) {
      int64_t b0 = G * g, b1 = b0 + g < nb ? b0 + g : nb;
      float c = 0.0f;
      for (int64_t b = b0; b < b1; ++b)
        if (am[b] > c) c = am[b];
      float S = c / 255.0f; /* binary32, correctly rounded */
      scale2[G] = S;
      for (int64_t b = b0; b < b1; ++b) {
        double q = 0.0;
        if (S > 0.0f) {
          /* The fp64 quotient of two binary32 numbers never lands on k + 1/2
           * unless the real quotient does, so this rounding is exact. */
          q = nearbyint((double)am[b] / (double)S);
          if (q < 0.0) q = 0.0;
          if (q > 255.0) q = 255.0;
        }
        absmax_q[b] = (uint8_t)q;
      }
    }
    free(am);
  }
  free(codes);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Dequantize: w_hat = fl32(L[code] * s_hat), s_hat = absmax or fl32(q * S).   */
/* ------------------------------------------------------------------------- */
int orc_nf4_dequantize(const uint8_t* packed, int64_t n, int32_t bs, int32_t dq, int32_t g,
                       const float* absmax, const uint8_t* absmax_q, const float* scale2,
                       float* out) {
  if (!packed || !out || bs <= 0 || n < 0) return ORC_ERR_ARG;
  if (bs % 2 != 0 || n % bs != 0) return ORC_ERR_SHAPE;
  if (dq ? (g <= 0 || !absmax_q || !scale2) : !absmax) return ORC_ERR_ARG;
  double lv64[16];
  float lv[16];
  orc_nf4_levels(lv64, lv);
  for (int64_t i = 0; i < n; ++i) {
    uint8_t byte = packed[i / 2];
    int c = (i % 2 == 0) ? (byte >> 4) : (byte & 15);
    int64_t b = i / bs;
    float s = dq ? (float)absmax_q[b] * scale2[b / g] : absmax[b];
    out[i] = lv[c] * s;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Rounding binary32 -> bf16 / f16, round-to-nearest-even, from the formats'   */
/* definitions.  Used to form the compute-dtype operands.                      */
/* ------------------------------------------------------------------------- */
static uint16_t bf16_from_f32(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) /* NaN */
    return (uint16_t)((u >> 16) | 0x0040u);
  /* Keep the top 16 bits; round on the dropped 16 bits, ties to even. */
  uint32_t dropped = u & 0xffffu, kept = u >> 16;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
  return (uint16_t)kept;
}

static uint16_t f16_from_f32(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if ((u & 0x7f800000u) == 0x7f800000u) /* Inf or NaN */
    return (uint16_t)(sign | 0x7c00u | ((u & 0x007fffffu) ? 0x0200u : 0u));
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  /* Quantum of the f16 grid at a: 2^(e-10) for normals, 2^-24 below 2^-14. */
  int e2;
  frexp(a, &e2); /* a = m * 2^e2, m in [0.5, 1) => floor(log2 a) = e2 - 1 */
  int ex = e2 - 1;
  double quantum = (ex >= -14) ? ldexp(1.0, ex - 10) : ldexp(1.0, -24);
  double k = nearbyint(a / quantum); /* exact scaling, then ties-to-even */
  double r = k * quantum;
  if (r >= 65536.0) return (uint16_t)(sign | 0x7c00u); /* overflow to Inf */
  if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)k); /* subnormal (k <= 1024) */
  int re;
  double rm = frexp(r, &re);
  uint16_t E = (uint16_t)(re - 1 + 15);
  uint16_t M = (uint16_t)((rm * 2.0 - 1.0) * 1024.0);
  return (uint16_t)(sign | (uint16_t)(E << 10) | M);
}

static float f32_from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float f32_from_f16(uint16_t h) {
  int sign = (h >> 15) & 1, E = (h >> 10) & 31, M = h & 1023;
  double v;
  if (E == 31)
    v = M ? NAN : INFINITY;
  else if (E == 0)
    v = ldexp((double)M, -24);
  else
    v = ldexp(1024.0 + M, E - 25);
  return (float)(sign ? -v : v);
}

void orc_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_from_f32(in[i]);
}
void orc_f32_to_f16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_from_f32(in[i]);
}
void orc_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_from_bf16(in[i]);
}
void orc_f16_to_f32(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_from_f16(in[i]);
}

/* ------------------------------------------------------------------------- */
/* Forward and backward of the QLoRA linear layer, fp64.                       */
/* Operands arrive as binary32 arrays that hold the compute-dtype values        */
/* exactly (x~, W~, A~, B~, dY~); every product of two of them is exact in      */
/* fp64.  Shapes: x [M,K], W [N,K], A [r,K], B [N,r], dY [M,N], bias [N].       */
/* s = alpha / r ([C] scale()).                                                */
/* ------------------------------------------------------------------------- */

/* y = x W^T + s (x A^T) B^T + bias   ([R] QuantizedLinear forward; [B] eq. 6.3.6
 * shows the same y as x (W + s B A)^T). */
void orc_qlora_fwd(const float* x, const float* W, const float* A, const float* B,
                   const float* bias, int64_t M, int64_t N, int64_t K, int64_t r, double s,
                   double* y) {
  double* T0 = (double*)malloc((size_t)(M * r > 0 ? M * r : 1) * sizeof(double));
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i)
    for (int64_t t = 0; t < r; ++t) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += (double)x[i * K + k] * (double)A[t * K + k];
      T0[i * r + t] = acc;
    }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      double base = 0.0, lora = 0.0;
      for (int64_t k = 0; k < K; ++k) base += (double)x[i * K + k] * (double)W[j * K + k];
      for (int64_t t = 0; t < r; ++t) lora += T0[i * r + t] * (double)B[j * r + t];
      y[i * N + j] = base + s * lora + (bias ? (double)bias[j] : 0.0);
    }
  free(T0);
}

/* Selected entries y[ii[e], jj[e]] of the same forward, each computed on its own. */
void orc_qlora_fwd_at(const float* x, const float* W, const float* A, const float* B,
                      const float* bias, int64_t M, int64_t N, int64_t K, int64_t r, double s,
                      const int64_t* ii, const int64_t* jj, int64_t ns, double* out) {
  (void)M;
  (void)N;
#pragma omp parallel for schedule(dynamic)
  for (int64_t e = 0; e < ns; ++e) {
    int64_t i = ii[e], j = jj[e];
    double base = 0.0, lora = 0.0;
    for (int64_t k = 0; k < K; ++k) base += (double)x[i * K + k] * (double)W[j * K + k];
    for (int64_t t = 0; t < r; ++t) {
      double T0 = 0.0;
      for (int64_t k = 0; k < K; ++k) T0 += (double)x[i * K + k] * (double)A[t * K + k];
      lora += T0 * (double)B[j * r + t];
    }
    out[e] = base + s * lora + (bias ? (double)bias[j] : 0.0);
  }
}

/* Backward with W frozen ([R] "adapters do update"; [B] LoRA trains A and B only):
 *   T0 = x A^T, dT = s dY B, dX = dY W + dT A, dA = dT^T x, dB = s dY^T T0.   */
void orc_qlora_bwd(const float* x, const float* W, const float* A, const float* B,
                   const float* dY, int64_t M, int64_t N, int64_t K, int64_t r, double s,
                   double* dX, double* dA, double* dB) {
  size_t mr = (size_t)(M * r > 0 ? M * r : 1);
  double* T0 = (double*)malloc(mr * sizeof(double));
  double* dT = (double*)malloc(mr * sizeof(double));
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i)
    for (int64_t t = 0; t < r; ++t) {
      double a = 0.0, b = 0.0;
      for (int64_t k = 0; k < K; ++k) a += (double)x[i * K + k] * (double)A[t * K + k];
      for (int64_t n = 0; n < N; ++n) b += (double)dY[i * N + n] * (double)B[n * r + t];
      T0[i * r + t] = a;
      dT[i * r + t] = s * b;
    }
  if (dX) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
      for (int64_t k = 0; k < K; ++k) {
        double acc = 0.0, lora = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += (double)dY[i * N + n] * (double)W[n * K + k];
        for (int64_t t = 0; t < r; ++t) lora += dT[i * r + t] * (double)A[t * K + k];
        dX[i * K + k] = acc + lora;
      }
  }
  if (dA) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < r; ++t)
      for (int64_t k = 0; k < K; ++k) {
        double acc = 0.0;
        for (int64_t i = 0; i < M; ++i) acc += dT[i * r + t] * (double)x[i * K + k];
        dA[t * K + k] = acc;
      }
  }
  if (dB) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t t = 0; t < r; ++t) {
        double acc = 0.0;
        for (int64_t i = 0; i < M; ++i) acc += (double)dY[i * N + n] * T0[i * r + t];
        dB[n * r + t] = s * acc;
      }
  }
  free(T0);
  free(dT);
}

/* dX[ii[e], kk[e]] computed entry by entry. */
void orc_qlora_bwd_dx_at(const float* dY, const float* W, const float* A, const float* B,
                         int64_t M, int64_t N, int64_t K, int64_t r, double s,
                         const int64_t* ii, const int64_t* kk, int64_t ns, double* out) {
  (void)M;
#pragma omp parallel for schedule(dynamic)
  for (int64_t e = 0; e < ns; ++e) {
    int64_t i = ii[e], k = kk[e];
    double acc = 0.0, lora = 0.0;
    for (int64_t n = 0; n < N; ++n) acc += (double)dY[i * N + n] * (double)W[n * K + k];
    for (int64_t t = 0; t < r; ++t) {
      double dT = 0.0;
      for (int64_t n = 0; n < N; ++n) dT += (double)dY[i * N + n] * (double)B[n * r + t];
      lora += s * dT * (double)A[t * K + k];
    }
    out[e] = acc + lora;
  }
}

/* dA[tt[e], kk[e]] = sum_i dT[i, t] x[i, k]; the column dT[:, t] is computed once
 * per distinct t in the request. */
void orc_qlora_bwd_da_at(const float* x, const float* dY, const float* B, int64_t M, int64_t N,
                         int64_t K, int64_t r, double s, const int64_t* tt, const int64_t* kk,
                         int64_t ns, double* out) {
  double* col = (double*)malloc((size_t)(M > 0 ? M : 1) * sizeof(double));
  for (int64_t t = 0; t < r; ++t) {
    int used = 0;
    for (int64_t e = 0; e < ns; ++e) used |= (tt[e] == t);
    if (!used) continue;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) acc += (double)dY[i * N + n] * (double)B[n * r + t];
      col[i] = s * acc;
    }
    for (int64_t e = 0; e < ns; ++e) {
      if (tt[e] != t) continue;
      double acc = 0.0;
      for (int64_t i = 0; i < M; ++i) acc += col[i] * (double)x[i * K + kk[e]];
      out[e] = acc;
    }
  }
  free(col);
}

/* dB[nn[e], tt[e]] = s sum_i dY[i, n] T0[i, t]; the column T0[:, t] is computed
 * once per distinct t in the request. */
void orc_qlora_bwd_db_at(const float* x, const float* A, const float* dY, int64_t M, int64_t N,
                         int64_t K, int64_t r, double s, const int64_t* nn, const int64_t* tt,
                         int64_t ns, double* out) {
  double* col = (double*)malloc((size_t)(M > 0 ? M : 1) * sizeof(double));
  for (int64_t t = 0; t < r; ++t) {
    int used = 0;
    for (int64_t e = 0; e < ns; ++e) used |= (tt[e] == t);
    if (!used) continue;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += (double)x[i * K + k] * (double)A[t * K + k];
      col[i] = acc;
    }
    for (int64_t e = 0; e < ns; ++e) {
      if (tt[e] != t) continue;
      double acc = 0.0;
      for (int64_t i = 0; i < M; ++i) acc += (double)dY[i * N + nn[e]] * col[i];
      out[e] = s * acc;
    }
  }
  free(col);
}

/* ------------------------------------------------------------------------- */
/* Merge ([B] "The merge math", eq. 6.3.6): W_merged = W_hat + s B A, rounded  */
/* once from the exact (fp64) value to the output dtype; never re-quantized.   */
/* ------------------------------------------------------------------------- */

/* One rounding of a binary64 value to the nearest value with `bits` significant
 * bits whose quantum is at least 2^qmin (ties to even); the result is exact in
 * binary64. */
static double round_sig(double v, int bits, int qmin) {
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  int e;
  frexp(fabs(v), &e); /* |v| = m 2^e, m in [0.5, 1) */
  int q = e - bits;
  if (q < qmin) q = qmin;
  return ldexp(nearbyint(ldexp(v, -q)), q);
}

static uint16_t bf16_from_f64(double v) {
  if (isnan(v)) return 0x7fc0;
  double r = round_sig(v, 8, -133); /* bf16: 8 significant bits, binary32 exponents */
  if (fabs(r) > 3.3895313892515355e38) return (uint16_t)(signbit(v) ? 0xff80 : 0x7f80);
  return bf16_from_f32((float)r); /* exact: r is a bf16 value */
}

static uint16_t f16_from_f64(double v) {
  if (isnan(v)) return 0x7e00;
  double r = round_sig(v, 11, -24); /* f16: 11 significant bits, quantum >= 2^-24 */
  if (fabs(r) > 65504.0) return (uint16_t)(signbit(v) ? 0xfc00 : 0x7c00);
  return f16_from_f32((float)r); /* exact */
}

/* what [N,K] (the binary32 dequantized weight), A [r,K], B [N,r] (adapter values),
 * kind 0: binary32 out, 1: bf16 bits, 2: f16 bits. */
void orc_qlora_merge(const float* what, const float* A, const float* B, int64_t N, int64_t K, int64_t r,
                     double s, int32_t kind, void* out) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0.0;
      for (int64_t t = 0; t < r; ++t) acc += (double)B[n * r + t] * (double)A[t * K + k];
      const double v = (double)what[n * K + k] + s * acc;
      if (kind == 0) ((float*)out)[n * K + k] = (float)v;
      else if (kind == 1) ((uint16_t*)out)[n * K + k] = bf16_from_f64(v);
      else ((uint16_t*)out)[n * K + k] = f16_from_f64(v);
    }
}


/* One rounding of binary64 values to binary32 (kind 0, as float), bf16 (1) or f16 (2)
 * bits: the storage of activations and gradients between the layers of a stack. */
void orc_round_f64(const double* in, int64_t n, int32_t kind, void* out) {
  for (int64_t i = 0; i < n; ++i) {
    if (kind == 0) ((float*)out)[i] = (float)in[i];
    else if (kind == 1) ((uint16_t*)out)[i] = bf16_from_f64(in[i]);
    else ((uint16_t*)out)[i] = f16_from_f64(in[i]);
  }
}
