// gemv.hip -- decode-shaped forward (m <= 16 tokens) of the QLoRA layer on gfx950.
//
// y[m, n] = sum_k x[m, k] W~[n, k] + sum_t T[m, t] B[n, t] (+ bias[n]),
// T = s x A^T, W~ = cd(fl32(L[c] s_b)) (qlora-rs README "Honest capability
// matrix": dequant honours the compute dtype; rust_ai_core QLoraConfig
// scale() = alpha / r).  At m <= 16 the layer moves the packed weight once and
// does at most 32 flops per weight, so it is bound by HBM.
//
// Two launches (bf16 / f16):
//   k_gemv_mfma  split-K over the contraction.  Workgroup (row block of 64, K
//                slice) issues every code load of its slice at once, stages the m
//                token rows of x for the slice in LDS, decodes W~ exactly in
//                registers and lets MFMA 16x16x32 do the token sums (W~ rows as
//                the A operand, x^T as B; tokens past m are zeros).  The LoRA
//                down-projection rides along: the rows of lora_a are r extra
//                (dense) rows of the same product.  Partial sums of every slice go
//                to the workspace with plain stores.
//   k_gemv_epi   adds the slices in slice order (the result does not depend on
//                scheduling), forms T = s x A^T from the extra rows, and writes
//                y = x W~^T + T B^T + bias; the kernel boundary orders it after
//                the partial sums, so no workgroup ever waits on another.
// f32, and shapes the MFMA kernel does not take, run k_lora_t (T = s x A^T) and
// k_gemv (one wavefront per output row on the VALU).
#include <algorithm>

#include "common.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxM = 16;

// T[m, t] = s * sum_k x[m, k] A[t, k]; t0[m, t] = the unscaled sum (optional).
// One workgroup per t: each lane sums 8 consecutive k per step for every token,
// then the workgroup reduces.
template <int CD>
__global__ __launch_bounds__(kThreads) void k_lora_t(const void* __restrict__ x, const void* __restrict__ A,
                                                     int64_t M, int64_t K, int32_t r, float scale,
                                                     float* __restrict__ T, float* __restrict__ t0) {
  __shared__ float red[kThreads / 64][kMaxM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = blockIdx.x;
  float acc[kMaxM];
#pragma unroll
  for (int i = 0; i < kMaxM; ++i) acc[i] = 0.f;
  for (int64_t k = (int64_t)tid * 8; k < K; k += kThreads * 8) {  // K % 8 == 0
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = load_cd<CD>(A, t * K + k + e);
#pragma unroll
    for (int i = 0; i < kMaxM; ++i)
      if (i < M) {
        float v = acc[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) v = fmaf(load_cd<CD>(x, (int64_t)i * K + k + e), a[e], v);
        acc[i] = v;
      }
  }
#pragma unroll
  for (int i = 0; i < kMaxM; ++i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[i] += __shfl_xor(acc[i], off, 64);
    if (lane == 0) red[wave][i] = acc[i];
  }
  __syncthreads();
  if (tid < M) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) v += red[w][tid];
    T[(int64_t)tid * r + t] = v * scale;
    if (t0) t0[(int64_t)tid * r + t] = v;
  }
}

// ---------------------------------------------------------------------------
// MFMA split-K decode GEMV (bf16 / f16).
// ---------------------------------------------------------------------------
constexpr int kRowBlock = 64;   // W rows per workgroup (16 per wave)

struct GemvP {
  Nf4W w;
  const void* x;      // [M, K] cd
  int64_t M;
  const void* A;      // lora_a [r, K] cd: rows n_pad .. n_pad + r of the product
  const void* B;      // lora_b [N, r] cd
  int32_t r;
  float scale;        // s
  const void* bias;   // [N] cd or null
  void* y;            // [M, N] cd
  float* t0;          // [M, r] fp32 x A^T, or null
  float* part;        // [S][16][ld] fp32 partial sums, ld = n_pad + r_pad
  int64_t n_pad, ld;
  int32_t S;          // slices of 512 elements
};

typedef float f32x4v_t __attribute__((__vector_size__(16)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t oob_unless(bool ok, uint32_t off) { return off | ((uint32_t)(!ok) << 31); }

template <int CD>
__device__ __forceinline__ f32x4v_t mfma16(u32x4_t a, u32x4_t b, f32x4v_t c) {
  if constexpr (CD == CD_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

// Lane l of wave w: W row n0 + 16 w + l % 16; in step j of the slice it holds the
// 32 codes at k = kb + 128 j + 32 (l / 16) .. +32, one 16-byte load.  MFMA u of the
// step takes codes 8u .. 8u+8 of them against x at the same k (the 4 x 16-lane
// groups together cover the step's 128 k, in a permuted but consistent order).
// Every load is a buffer load: rows past N (or past r, or tokens past m) read past
// their buffer and return zeros, so the kernel has no per-lane branches.
constexpr int kSlice = 512;               // K elements per slice: 4 steps of 128

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kGemvThreads = 512;  // 8 waves: row group w % 4 (16 rows), slice half w / 4 (2 steps)

template <int CD, int DQ>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_mfma(GemvP p, Nf4Tables tab) {
  // the level pair of every code byte (element 2b in the high nibble, 2b + 1 in the low
  // one): one 8-byte LDS read per two codes
  __shared__ __attribute__((aligned(16))) float2 s_pair[256];
  __shared__ __attribute__((aligned(16))) uint16_t xs[kMaxM][kSlice + 8];  // +16 B per row: no bank conflicts
  // the codes of the slice, [64 rows][256 bytes]; 16-byte chunk c of row r sits at
  // chunk c ^ (r % 16), so the 16 rows a read instruction touches hit 16 bank groups
  __shared__ __attribute__((aligned(1024))) uint8_t cs[kRowBlock * kSlice / 2];
  __shared__ f32x4v_t red[4][64];  // second-half sums, per row group and lane
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave & 3, half = wave >> 2;
  if (tid < 256) s_pair[tid] = make_float2(tab.lv[tid >> 4], tab.lv[tid & 15]);
  const Nf4W& w = p.w;
  const int64_t K = w.cols, N = w.rows;
  const int64_t n0 = (int64_t)blockIdx.x * kRowBlock;
  const bool lora = n0 >= p.n_pad;  // a block of lora_a rows (uniform per workgroup)
  const int sl = blockIdx.y;
  const int64_t kb = (int64_t)sl * kSlice;
  const int q = lane >> 4, rl = lane & 15;
  const int64_t row = n0 + 16 * grp + rl;  // column of the partial sums

  // x for the slice first (thread: token tid / 32, 16-byte chunks tid % 32 + 32 j)
  const int xm = tid >> 5, xc = tid & 31;
  const rsrc_t rx = make_rsrc(p.x, p.M * K * 2);
  u32x4_t xv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    xv[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                            rx, (int)((xm * K + kb + 8 * (xc + 32 * j)) * 2), 0, 0));

  // four accumulators (one per MFMA of a step) keep the MFMAs independent
  f32x4v_t acc[4] = {};
  if (lora) {
    // dense rows t = row - n_pad of lora_a, in the same k order as the codes
    const int64_t t = row - p.n_pad;
    const rsrc_t ra = make_rsrc(p.A, (int64_t)p.r * K * 2);
    u32x4_t av[2][4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        av[jj][u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                        ra, (int)oob_unless(t < p.r, (uint32_t)((t * K + kb + 128 * (2 * half + jj) + 32 * q + 8 * u) * 2)),
                        0, 0));
#pragma unroll
    for (int j = 0; j < 2; ++j) *(u32x4_t*)&xs[xm][8 * (xc + 32 * j)] = xv[j];
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc[u] = mfma16<CD>(av[jj][u], *(const u32x4_t*)&xs[rl][128 * (2 * half + jj) + 32 * q + 8 * u], acc[u]);
  } else {
    const bool rok = row < N;
    const rsrc_t rc = make_rsrc(w.codes, N * K / 2);
    const int64_t nb = N * K / w.bs;
    const rsrc_t rq = DQ ? make_rsrc(w.absmax_q, nb) : make_rsrc(w.absmax, nb * 4);
    const rsrc_t rs = make_rsrc(DQ ? (const void*)w.scale2 : (const void*)w.absmax,
                                DQ ? (((nb - 1) >> w.g_shift) + 1) * 4 : nb * 4);
    // codes: DMA instruction i of wave w fills rows 4 (8 i + w) .. +4, 256 bytes each:
    // lane l lands in physical chunk l % 16 of row l / 16 and fetches the logical
    // chunk that maps there (rows past N read past the buffer: zeros)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 4 * (8 * i + wave) + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      const int64_t grow = n0 + r;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rc, (lds_void*)(cs + (8 * i + wave) * 1024), 16,
          (int)oob_unless(grow < N, (uint32_t)((grow * K + kb) / 2 + 16 * c)), 0, 0, 0);
    }
    uint32_t sq[2];
    float sf[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int64_t e = row * K + kb + 128 * (2 * half + jj) + 32 * q;  // 32 codes in one block (bs >= 32)
      const uint32_t b = (uint32_t)(e >> w.bs_shift);
      if constexpr (DQ) {
        sq[jj] = __builtin_amdgcn_raw_buffer_load_b8(rq, (int)oob_unless(rok, b), 0, 0);
        sf[jj] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rs, (int)oob_unless(rok, (b >> w.g_shift) * 4), 0, 0));
      } else {
        sf[jj] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rq, (int)oob_unless(rok, b * 4), 0, 0));
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) *(u32x4_t*)&xs[xm][8 * (xc + 32 * j)] = xv[j];
    __builtin_amdgcn_s_waitcnt(((DQ ? 4 : 2) & 15) | (7 << 4) | (15 << 8));  // the DMA (the scales may fly)
    __syncthreads();
    const int crow = (16 * grp + rl) * (kSlice / 2);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * half + jj;
      const u32x4_t cw = *(const u32x4_t*)(cs + crow + 16 * ((4 * j + q) ^ rl));
      const float s = DQ ? (float)sq[jj] * sf[jj] : sf[jj];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t word = cw[u];
        u32x4_t a;
#pragma unroll
        for (int b = 0; b < 4; ++b) {  // byte b: element 2b in the high nibble, 2b + 1 in the low one
          const float2 lv2 = *(const float2*)((const char*)s_pair + (byte_of(word, b) << 3));
          a[b] = pack2<CD>(fl32_mul(lv2.x, s), fl32_mul(lv2.y, s));
        }
        acc[u] = mfma16<CD>(a, *(const u32x4_t*)&xs[rl][128 * j + 32 * q + 8 * u], acc[u]);
      }
    }
  }

  // sum of the four accumulators and the two halves; then the partial sums
  // D[row 16 g + 4 q + v][token rl] of this slice
  f32x4v_t v = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  if (half) red[grp][lane] = v;
  __syncthreads();
  if (half) return;
  v += red[grp][lane];
  if (rl < p.M) *(f32x4v_t*)(p.part + ((int64_t)sl * kMaxM + rl) * p.ld + n0 + 16 * grp + 4 * q) = v;
}

// y[m, n] = sum over slices of the partials + T[m, :] . B[n, :] + bias[n], with
// T = s (sum over slices of the lora_a rows).  Workgroup (256 columns, token m)
// forms T[m, :] in LDS; the workgroups of column block 0 also write t0 = x A^T
// when asked.  For r <= 64, r % 8 == 0 every global load of a thread (its
// column's S partial sums, bias, lora_b row, and its share of the r x S partial
// sums of T) is issued before the first is used, so the kernel waits on memory
// once; T's slices are then added in slice order through LDS.  Other ranks take
// the same sums in two dependent rounds.
template <int CD, int S>
__global__ __launch_bounds__(kThreads) void k_gemv_epi(GemvP p) {
  extern __shared__ float s_t[];  // [r] sums, then (fast path) [S][64] staged partial sums
  const int tid = threadIdx.x;
  const int m = blockIdx.y;
  const int64_t N = p.w.rows;
  const float* pm = p.part + (int64_t)m * p.ld;
  const int64_t ss = (int64_t)kMaxM * p.ld;
  const int64_t n = (int64_t)blockIdx.x * kThreads + tid;
  const int64_t nc = n < N ? n : N - 1;  // clamped: every lane loads, out-of-range lanes store nothing
  float v = 0.f, lora = 0.f;
  if (p.r <= 64 && (p.r & 7) == 0) {
    float pv[S];
#pragma unroll
    for (int i = 0; i < S; ++i) pv[i] = pm[i * ss + nc];
    // bias through a buffer of zero size when absent: the load returns 0, no branch
    const rsrc_t rb = make_rsrc(p.bias, p.bias ? N * 2 : 0);
    const uint32_t braw = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(nc * 2), 0, 0);
    const rsrc_t rB = make_rsrc(p.B, N * p.r * 2);
    u32x4_t bv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      bv[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              rB, (int)(uint32_t)(q * 8 < p.r ? (nc * p.r + 8 * q) * 2 : 0), 0, 0));
    // T's partial sums: slice i = tid / 64 + 4 k, rank column t = tid % 64
    const int t = tid & 63;
    float tp[(S + 3) / 4];
#pragma unroll
    for (int k = 0; k < (S + 3) / 4; ++k) {
      const int i = (tid >> 6) + 4 * k;
      tp[k] = pm[(i < S ? i : 0) * ss + p.n_pad + (t < p.r ? t : 0)];
    }
#pragma unroll
    for (int k = 0; k < (S + 3) / 4; ++k) {
      const int i = (tid >> 6) + 4 * k;
      if (i < S) s_t[64 + i * 64 + t] = tp[k];
    }
    __syncthreads();
    if (tid < p.r) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < S; ++i) sum += s_t[64 + i * 64 + tid];
      s_t[tid] = sum * p.scale;
      if (p.t0 && blockIdx.x == 0) p.t0[(int64_t)m * p.r + tid] = sum;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q * 8 < p.r) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          lora = fmaf(s_t[8 * q + e], from_cd16<CD>((uint16_t)(bv[q][e >> 1] >> (16 * (e & 1)))), lora);
      }
#pragma unroll
    for (int i = 0; i < S; ++i) v += pv[i];
    v += lora + (p.bias ? from_cd16<CD>((uint16_t)braw) : 0.f);
  } else {
    for (int t = tid; t < p.r; t += kThreads) {
      float tv[S];
#pragma unroll
      for (int i = 0; i < S; ++i) tv[i] = pm[i * ss + p.n_pad + t];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < S; ++i) sum += tv[i];
      s_t[t] = sum * p.scale;
      if (p.t0 && blockIdx.x == 0) p.t0[(int64_t)m * p.r + t] = sum;
    }
    __syncthreads();
    float pv[S];
#pragma unroll
    for (int i = 0; i < S; ++i) pv[i] = pm[i * ss + nc];
    const float bias = p.bias ? load_cd<CD>(p.bias, nc) : 0.f;
    for (int t = 0; t < p.r; ++t) lora = fmaf(s_t[t], load_cd<CD>(p.B, nc * p.r + t), lora);
#pragma unroll
    for (int i = 0; i < S; ++i) v += pv[i];
    v += lora + bias;
  }
  if (n < N) store_cd<CD>(p.y, m * N + n, v);
}

// VALU decode GEMV: one wavefront per output row (f32, and other shapes).
template <int CD>
__global__ __launch_bounds__(kThreads) void k_gemv(Nf4W w, const void* __restrict__ x, int64_t M,
                                                   const float* __restrict__ T,
                                                   const void* __restrict__ B, int32_t r,
                                                   const void* __restrict__ bias, void* __restrict__ y,
                                                   Nf4Tables tab) {
  __shared__ float s_lv[16];
  if (threadIdx.x < 16) s_lv[threadIdx.x] = tab.lv[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (n >= w.rows) return;
  const int64_t K = w.cols;
  float acc[kMaxM];
#pragma unroll
  for (int i = 0; i < kMaxM; ++i) acc[i] = 0.f;

  for (int64_t c = lane; c < K / 32; c += 64) {
    const int64_t k0 = c * 32;
    const int64_t e = n * K + k0;
    u32x4_t v = *(const u32x4_t*)(w.codes + e / 2);
    const float s = block_scale(w, block_of(w, e));
    float wt[32];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t code = (v[d] >> ((j >> 1) * 8 + ((j & 1) ? 0 : 4))) & 15u;
        float f = fl32_mul(s_lv[code], s);
        if constexpr (CD != CD_F32) f = from_cd16<CD>(to_cd16<CD>(f));
        wt[d * 8 + j] = f;
      }
#pragma unroll
    for (int i = 0; i < kMaxM; ++i) {
      if (i < M) {
        float a = acc[i];
#pragma unroll
        for (int j = 0; j < 32; ++j) a = fmaf(load_cd<CD>(x, (int64_t)i * K + k0 + j), wt[j], a);
        acc[i] = a;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxM; ++i)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[i] += __shfl_xor(acc[i], off, 64);

  if (lane < M) {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxM; ++i)
      if (i == lane) v = acc[i];
    float lora = 0.f;
    for (int t = 0; t < r; ++t) lora = fmaf(T[(int64_t)lane * r + t], load_cd<CD>(B, n * r + t), lora);
    v += lora;
    if (bias) v += load_cd<CD>(bias, n);
    store_cd<CD>(y, (int64_t)lane * w.rows + n, v);
  }
}

// Split of the contraction into S slices of 512 elements (S in {1, 2, 4, 8, 16}).
struct GemvPlan {
  bool mfma;
  int32_t S;
  int64_t n_pad, r_pad, ld, off_part, total;
};
GemvPlan plan_gemv(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd) {
  GemvPlan P = {};
  P.S = (int32_t)(cols / kSlice);
  P.mfma = (cd == CD_BF16 || cd == CD_F16) && rows > 0 && cols % kSlice == 0 &&
           (P.S == 1 || P.S == 2 || P.S == 4 || P.S == 8 || P.S == 16);
  P.n_pad = round_up(rows, kRowBlock);
  P.r_pad = round_up(r, kRowBlock);
  P.ld = P.n_pad + P.r_pad;
  P.off_part = round_up(m * r * 4, 256);  // T for the VALU path
  P.total = P.off_part + (P.mfma ? round_up((int64_t)P.S * kMaxM * P.ld * 4, 256) : 0);
  return P;
}

template <int CD>
int gemv_forward_t(const LayerCall& c, void* y, float* t_save) {
  const GemvPlan P = plan_gemv(c.m, c.w.rows, c.w.cols, c.r, c.cd);
  const bool mfma = P.mfma && c.w.bs_shift >= 5 && (!c.w.dq || c.w.g_shift >= 0) &&
                    c.w.rows * c.w.cols / 2 < 0x7fff0000LL;
  char* ws = (char*)c.ws;
  if constexpr (CD != CD_F32) {
    if (mfma) {
      GemvP p = {};
      p.w = c.w;
      p.x = c.x;
      p.M = c.m;
      p.A = c.lora_a;
      p.B = c.lora_b;
      p.r = c.r;
      p.scale = c.scale;
      p.bias = c.bias;
      p.y = y;
      p.t0 = t_save;
      p.part = (float*)(ws + P.off_part);
      p.n_pad = P.n_pad;
      p.ld = P.ld;
      p.S = P.S;
      {
        ProfScope prof(QLORA_K_GEMV, c.stream);
        const dim3 grid((unsigned)(P.ld / kRowBlock), (unsigned)P.S);
        if (c.w.dq) k_gemv_mfma<CD, 1><<<grid, dim3(kGemvThreads), 0, c.stream>>>(p, host_tables());
        else k_gemv_mfma<CD, 0><<<grid, dim3(kGemvThreads), 0, c.stream>>>(p, host_tables());
        int rc = check_launch("k_gemv_mfma");
        if (rc) return rc;
      }
      ProfScope prof(QLORA_K_REDUCE, c.stream);
      const size_t lds = (size_t)(c.r <= 64 && c.r % 8 == 0 ? 64 * (1 + P.S) : c.r) * sizeof(float);
      if (lds > 65536) return set_error(QLORA_ERR_UNSUPPORTED, "decode: rank %d too large", c.r);
      const dim3 eg((unsigned)ceil_div(c.w.rows, kThreads), (unsigned)c.m);
      switch (P.S) {
        case 1: k_gemv_epi<CD, 1><<<eg, dim3(kThreads), lds, c.stream>>>(p); break;
        case 2: k_gemv_epi<CD, 2><<<eg, dim3(kThreads), lds, c.stream>>>(p); break;
        case 4: k_gemv_epi<CD, 4><<<eg, dim3(kThreads), lds, c.stream>>>(p); break;
        case 8: k_gemv_epi<CD, 8><<<eg, dim3(kThreads), lds, c.stream>>>(p); break;
        default: k_gemv_epi<CD, 16><<<eg, dim3(kThreads), lds, c.stream>>>(p); break;
      }
      return check_launch("k_gemv_epi");
    }
  }
  float* T = (float*)ws;
  {
    ProfScope prof(QLORA_K_LORA_DOWN, c.stream);
    k_lora_t<CD><<<dim3((unsigned)c.r), dim3(kThreads), 0, c.stream>>>(c.x, c.lora_a, c.m, c.w.cols, c.r, c.scale,
                                                                         T, t_save);
    int rc = check_launch("k_lora_t");
    if (rc) return rc;
  }
  ProfScope prof(QLORA_K_GEMV, c.stream);
  k_gemv<CD><<<dim3((unsigned)ceil_div(c.w.rows, kThreads / 64)), dim3(kThreads), 0, c.stream>>>(
      c.w, c.x, c.m, T, c.lora_b, c.r, c.bias, y, host_tables());
  return check_launch("k_gemv");
}

}  // namespace

size_t gemv_workspace_bytes(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd) {
  return (size_t)plan_gemv(m, rows, cols, r, cd).total;
}

int gemv_forward(const LayerCall& c, void* y, float* t_save) {
  switch (c.cd) {
    case CD_BF16: return gemv_forward_t<CD_BF16>(c, y, t_save);
    case CD_F16: return gemv_forward_t<CD_F16>(c, y, t_save);
    case CD_F32: return gemv_forward_t<CD_F32>(c, y, t_save);
  }
  return set_error(QLORA_ERR_DTYPE, "forward: bad compute dtype %d", c.cd);
}

}  // namespace qnf4
