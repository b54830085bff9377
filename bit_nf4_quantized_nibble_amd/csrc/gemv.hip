// gemv.hip -- decode-shaped forward (m <= 16 tokens) of the QLoRA layer on gfx950.
//
// y[m, n] = sum_k x[m, k] W~[n, k] + sum_t T[m, t] B[n, t] (+ bias[n]),
// T = s x A^T, W~ = cd(fl32(L[c] s_b)) (qlora-rs README "Honest capability
// matrix": dequant honours the compute dtype; rust_ai_core QLoraConfig
// scale() = alpha / r).  At m <= 16 the layer moves the packed weight once and
// does at most 32 flops per weight, so it is bound by HBM.
//
// Two launches (bf16 / f16):
//   k_gemv_k     split-K over the contraction.  Workgroup (row block of 32, slice
//                of 1024) issues every load of its tile at once, decodes W~ exactly
//                and lets MFMA 16x16x32 do the token sums (W~ rows as the A
//                operand, x^T as B; tokens past m are zeros).  The LoRA
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

// Split-K decode GEMV.  Workgroup = 4 waves on a tile of 32 W rows x 1024
// contraction elements (slice sl); wave w takes the sub-slice [kb + 256 w,
// kb + 256 (w + 1)) of the 32 rows (two row groups of 16), so the x fragments a lane
// loads are its own and serve both row groups.  MFMA 16x16x32: W~ [16 rows x 32 k]
// as A, x^T [32 k x 16 tokens] as B (tokens past m read as zeros).  Lane l
// (q = l / 16, rl = l % 16) in sub-step s of row group g holds row 16 g + rl and the
// 32 codes of chunk q + 4 s (of the sub-slice's eight 32-code chunks); MFMA u takes
// codes 8 u .. 8 u + 8 of them, and x is loaded in the same permuted k order.
// Memory: each wave loads its codes as 8 rows x 128 contiguous bytes per
// instruction (two per row group) and transposes them to the MFMA layout through
// its own LDS region, so no wave waits for another until the final sum.  Every load
// is issued before the first wait, in the order the decode needs them (row group
// 0's codes, the block scales, x, row group 1's codes), since a wave sees its loads
// complete in issue order.  Each weight decodes exactly to W~ = cd(fl32(L[c] s_b))
// (one 8-byte LDS read of a level pair per code byte); the four waves' partial sums
// are added in wave order through LDS.  Rows past N (and lora_a rows past r) read
// past their buffers: zeros, no branch.
constexpr int kRows = 32;      // W rows per workgroup
constexpr int kSliceK = 1024;  // contraction elements per slice
constexpr int kWaveK = 256;    // contraction elements per wave
constexpr int kGemvThreads = 256;

// Chunk (16 bytes = 32 codes) c of tile row r in a wave's [32 rows][128 bytes] LDS
// tile: rows r and r + 2 share banks, so the chunk index is XORed with (r / 2) % 8.
__device__ __forceinline__ int tile_off(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }

template <int CD, int DQ, int NBK>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_k(GemvP p, Nf4Tables tab) {
  __shared__ __attribute__((aligned(16))) float2 s_pair[256];
  __shared__ float s_sc[4][kRows][8];  // per wave: block scales [row][block within the sub-slice]
  __shared__ __attribute__((aligned(16))) unsigned char s_codes[4][kRows * 128];  // per wave, swizzled
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, rl = lane & 15;
  const Nf4W& w = p.w;
  const int64_t K = w.cols, N = w.rows;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const bool lora = n0 >= p.n_pad;  // a block of lora_a rows (uniform per workgroup)
  const int sl = blockIdx.y;
  const int64_t kw = (int64_t)sl * kSliceK + kWaveK * wave;  // the wave's sub-slice
  const rsrc_t rx = make_rsrc(p.x, p.M * K * 2);
  u32x4_t xv[2][4];  // x of token rl: sub-step s, MFMA u -> k = kw + 32 (q + 4 s) + 8 u
  f32x4v_t acc[2] = {};

  if (lora) {
    // dense rows t = row - n_pad of lora_a in the same k order; only the row groups
    // that hold rows below r
    const int groups = (int)min<int64_t>(2, (p.r - (n0 - p.n_pad) + 15) / 16);
    const rsrc_t ra = make_rsrc(p.A, (int64_t)p.r * K * 2);
    u32x4_t av[2][2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t t = n0 + 16 * g + rl - p.n_pad;
          av[g][st][u] = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                           ra, (int)oob_unless(t < p.r && g < groups, (uint32_t)((t * K + kw + 32 * (q + 4 * st) + 8 * u) * 2)),
                           0, 0));
        }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        xv[st][u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rx, (int)((rl * K + kw + 32 * (q + 4 * st) + 8 * u) * 2), 0, 0));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[g] = mfma16<CD>(av[g][st][u], xv[st][u], acc[g]);
  } else {
    const rsrc_t rc = make_rsrc(w.codes, N * K / 2);
    // codes: instruction i loads tile rows 8 i + lane / 8, 16-byte chunk lane % 8
    u32x4_t cw[4];
    auto load_codes = [&](int i) {
      const int64_t grow = n0 + 8 * i + (lane >> 3);
      cw[i] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                       rc, (int)oob_unless(grow < N, (uint32_t)((grow * K + kw) / 2 + 16 * (lane & 7))), 0, 0));
    };
    load_codes(0);
    load_codes(1);
    // block scales of the wave's tile: lane l < 32 takes row l, blocks b0 .. b0 + nbk
    // of the sub-slice (bs >= 32: nbk <= 8, a power of two dividing b0), as one
    // naturally aligned load of the nbk u8 (or fp32) scales and one fp32 load per
    // second-level group they touch
    const int64_t nb = N * K / w.bs;
    const rsrc_t rq = DQ ? make_rsrc(w.absmax_q, nb) : make_rsrc(w.absmax, nb * 4);
    const int64_t srow = n0 + (lane & 31);
    const uint32_t b0 = (uint32_t)((srow * K + kw) >> w.bs_shift);  // a multiple of NBK
    const bool sok = lane < kRows && srow < N;
    uint32_t sraw[NBK];  // DQ: the u8 scales packed little-endian; else the fp32 scales
    uint32_t sf[NBK];    // DQ: second-level scale of each group touched (ngr <= NBK)
    const int ngr = (w.g_shift >= 31 || NBK <= (1 << w.g_shift)) ? 1 : NBK >> w.g_shift;
    if constexpr (DQ) {
      const uint32_t off = oob_unless(sok, b0);
      if constexpr (NBK == 1) sraw[0] = __builtin_amdgcn_raw_buffer_load_b8(rq, (int)off, 0, 0);
      else if constexpr (NBK == 2) sraw[0] = __builtin_amdgcn_raw_buffer_load_b16(rq, (int)off, 0, 0);
      else if constexpr (NBK == 4) sraw[0] = __builtin_amdgcn_raw_buffer_load_b32(rq, (int)off, 0, 0);
      else {
        const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rq, (int)off, 0, 0));
        sraw[0] = v[0];
        sraw[1] = v[1];
      }
      const rsrc_t rs = make_rsrc(w.scale2, (((nb - 1) >> w.g_shift) + 1) * 4);
      sf[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)oob_unless(sok, (b0 >> w.g_shift) * 4), 0, 0);
#pragma unroll
      for (int j = 1; j < NBK; ++j) sf[j] = 0u;
      if (ngr > 1) {  // groups smaller than the sub-slice (uniform; rare)
#pragma unroll
        for (int j = 1; j < NBK; ++j)
          sf[j] = __builtin_amdgcn_raw_buffer_load_b32(
              rs, (int)oob_unless(sok && j < ngr, ((b0 >> w.g_shift) + j) * 4), 0, 0);
      }
    } else {
      const uint32_t off = oob_unless(sok, b0 * 4);
      if constexpr (NBK == 1) sraw[0] = __builtin_amdgcn_raw_buffer_load_b32(rq, (int)off, 0, 0);
      else if constexpr (NBK == 2) {
        const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rq, (int)off, 0, 0));
        sraw[0] = v[0];
        sraw[1] = v[1];
      } else {
#pragma unroll
        for (int h = 0; h < NBK / 4; ++h) {
          const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                            rq, (int)oob_unless(sok, b0 * 4 + 16 * h), 0, 0));
#pragma unroll
          for (int e = 0; e < 4; ++e) sraw[4 * h + e] = v[e];
        }
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        xv[st][u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rx, (int)((rl * K + kw + 32 * (q + 4 * st) + 8 * u) * 2), 0, 0));
    load_codes(2);
    load_codes(3);
    __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first wait
    // level pair of code byte tid (element 2b in the high nibble), from the kernel
    // arguments
    {
      float lhi = tab.lv[0], llo = tab.lv[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        lhi = (tid >> 4) == i ? tab.lv[i] : lhi;
        llo = (tid & 15) == i ? tab.lv[i] : llo;
      }
      s_pair[tid] = make_float2(lhi, llo);
    }
    __syncthreads();  // the level pairs (everything after is the wave's own)
    unsigned char* tile = s_codes[wave];
    if (lane < kRows) {
#pragma unroll
      for (int j = 0; j < NBK; ++j) {
        if constexpr (DQ) {
          const uint32_t qb = byte_of(sraw[j >> 2], j & 3);
          const int gi = ngr == 1 ? 0 : (j >> w.g_shift);
          float s2 = __uint_as_float(sf[0]);
#pragma unroll
          for (int k = 1; k < NBK; ++k) s2 = k == gi ? __uint_as_float(sf[k]) : s2;
          s_sc[wave][lane][j] = fl32_mul((float)qb, s2);
        } else {
          s_sc[wave][lane][j] = __uint_as_float(sraw[j]);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      // rows 16 g .. 16 g + 15 arrived with instructions 2 g and 2 g + 1
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *(u32x4_t*)(tile + tile_off(16 * g + 8 * h + (lane >> 3), lane & 7)) = cw[2 * g + h];
      __builtin_amdgcn_wave_barrier();  // LDS operations of one wave complete in order
      u32x4_t cv[2];
      float sc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int c = q + 4 * st;
        cv[st] = *(const u32x4_t*)(tile + tile_off(16 * g + rl, c));
        sc[st] = s_sc[wave][16 * g + rl][NBK == 1 ? 0 : (32 * c) >> w.bs_shift];
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float2 lv2[4][4];  // the 16 level pairs of the chunk, requested before the first use
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int b = 0; b < 4; ++b) lv2[u][b] = *(const float2*)((const char*)s_pair + (byte_of(cv[st][u], b) << 3));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          u32x4_t a;
#pragma unroll
          for (int b = 0; b < 4; ++b) a[b] = pack2<CD>(fl32_mul(lv2[u][b].x, sc[st]), fl32_mul(lv2[u][b].y, sc[st]));
          acc[g] = mfma16<CD>(a, xv[st][u], acc[g]);
        }
      }
    }
  }

  // acc[g] = D[rows 16 g + 4 q .. +3][token rl] of this wave's sub-slice; waves 0 and
  // 1 add the four waves' sums of row groups 0 and 1, in wave order
  f32x4v_t* red = (f32x4v_t*)&s_codes[0][0];  // [wave][group][lane]
  __syncthreads();
#pragma unroll
  for (int g = 0; g < 2; ++g) red[(wave * 2 + g) * 64 + lane] = acc[g];
  __syncthreads();
  if (wave < 2) {
    const int g = wave;
    const f32x4v_t v = (red[g * 64 + lane] + red[(2 + g) * 64 + lane]) + (red[(4 + g) * 64 + lane] + red[(6 + g) * 64 + lane]);
    if (rl < p.M) *(f32x4v_t*)(p.part + ((int64_t)sl * kMaxM + rl) * p.ld + n0 + 16 * g + 4 * q) = v;
  }
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

// Split of the contraction into S slices of 1024 elements (S in {1, 2, 4, 8, 16}).
struct GemvPlan {
  bool mfma;
  int32_t S;
  int64_t n_pad, r_pad, ld, off_part, total;
};
GemvPlan plan_gemv(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd) {
  GemvPlan P = {};
  P.S = (int32_t)(cols / kSliceK);
  P.mfma = (cd == CD_BF16 || cd == CD_F16) && rows > 0 && cols % kSliceK == 0 &&
           (P.S == 1 || P.S == 2 || P.S == 4 || P.S == 8 || P.S == 16);
  P.n_pad = round_up(rows, kRows);
  P.r_pad = round_up(r, kRows);
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
        const dim3 grid((unsigned)(P.ld / kRows), (unsigned)P.S);
        const int nbk = c.w.bs_shift >= 8 ? 1 : 1 << (8 - c.w.bs_shift);  // blocks per 256-element sub-slice
        switch (nbk * 2 + (c.w.dq ? 1 : 0)) {
          case 2: k_gemv_k<CD, 0, 1><<<grid, dim3(kGemvThreads), 0, c.stream>>>(p, host_tables()); break;
          case 3: k_gemv_k<CD, 1, 1><<<grid, dim3(kGemvThreads), 0, c.stream>>>(p, host_tables()); break;
          case 4: k_gemv_k<CD, 0, 2><<<grid, dim3(kGemvThreads), 0, c.stream>>>(p, host_tables()); break;
          case 5: k_gemv_k<CD, 1, 2><<<grid, dim3(kGemvThreads), 0, c.stream>>>(p, host_tables()); break;
          case 8: k_gemv_k<CD, 0, 4><<<grid, dim3(kGemvThreads), 0, c.stream>>>(p, host_tables()); break;
          case 9: k_gemv_k<CD, 1, 4><<<grid, dim3(kGemvThreads), 0, c.stream>>>(p, host_tables()); break;
          case 16: k_gemv_k<CD, 0, 8><<<grid, dim3(kGemvThreads), 0, c.stream>>>(p, host_tables()); break;
          default: k_gemv_k<CD, 1, 8><<<grid, dim3(kGemvThreads), 0, c.stream>>>(p, host_tables()); break;
        }
        int rc = check_launch("k_gemv_k");
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
