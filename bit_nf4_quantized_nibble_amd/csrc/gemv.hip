// gemv.hip -- decode-shaped forward (up to 64 tokens) of the QLoRA layer on gfx950.
//
// y[m, n] = sum_k x[m, k] W~[n, k] + sum_t T[m, t] B[n, t] (+ bias[n]),
// T = s x A^T, W~ = cd(fl32(L[c] s_b)) (qlora-rs README "Honest capability
// matrix": dequant honours the compute dtype; rust_ai_core QLoraConfig
// scale() = alpha / r).  At a few tokens the layer moves the packed weight once and
// does at most 2 m flops per weight, so it is bound by HBM and by the decode.
//
// Two launches (bf16 / f16, cols a multiple of 1024):
//   k_gemv_k     split-K over the contraction.  Workgroup (row block of 32, slice
//                of 1024) issues every load of its tile at once, decodes W~ exactly
//                and lets MFMA 16x16x32 do the token sums (W~ rows as the A
//                operand, x^T as B; tokens past m are zeros), each decoded
//                fragment feeding up to four 16-token column groups.  With two or
//                more token groups and many row tiles a workgroup loops over row
//                tiles, keeping its x fragments in registers and requesting each
//                tile's codes before it decodes the previous one.  The LoRA
//                down-projection rides along: the rows of lora_a are r extra
//                (dense) rows of the same product.  Partial sums of every slice go
//                to the workspace with plain stores.
//   k_gemv_epi   adds the slices in slice order (the result does not depend on
//                scheduling), forms T = s x A^T from the extra rows, and writes
//                y = x W~^T + T B^T + bias; the kernel boundary orders it after
//                the partial sums, so no workgroup ever waits on another.
// f32, and shapes the MFMA kernel does not take (at most 16 tokens), run k_lora_t
// (T = s x A^T) and k_gemv (one wavefront per output row on the VALU).
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
  void* y;            // [M, ldy] cd
  int64_t ldy;        // row stride of y (>= N)
  float* t0;          // [M, r] fp32 x A^T, or null
  float* part;        // [S][mp][ld] fp32 partial sums, ld = n_pad + r_pad, mp = m rounded up to 16
  int64_t n_pad, ld, mp;
  int32_t S;          // slices of 1024 elements
  int32_t G;          // workgroups (per slice) on W tiles; the ones after take lora_a row blocks
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
// as A, x^T [32 k x 16 tokens] as B (tokens past m read as zeros).  The k order is
// permuted (the sum does not depend on it): MFMA u of sub-step s takes the
// sub-slice's 32-code chunk 4 s + u, lane l (q = l / 16, rl = l % 16) its codes
// 8 q .. 8 q + 8 for row 16 g + rl, so one x load instruction reads 64 contiguous
// bytes of each token.  Memory: each wave loads its codes as 8 rows x 128
// contiguous bytes per instruction (two per row group) and transposes them to the
// MFMA layout through its own LDS region (a 4 x 4 word transpose within each
// group of four chunks), so no wave waits for another until the final sum.  Every load
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

// The loads of one W tile (32 rows x the wave's 256-element sub-slice) a lane issues.
template <int NBK>
struct TileRegs {
  u32x4_t cw[4];       // codes: instruction i holds tile row 8 i + lane / 8, 16-byte chunk lane % 8
  uint32_t sraw[NBK];  // DQ: the u8 block scales packed little-endian; else the fp32 scales
  uint32_t sf[NBK];    // DQ: the second-level scale of each group the row's blocks touch
};

// Per-lane constants of a wave's view of its sub-slice.
struct WaveView {
  int lane, wave, q, rl;
  int64_t K, N, kw;  // kw: first contraction element of the wave's sub-slice
  int ngr;           // second-level groups a row's blocks touch in the sub-slice (1 unless groups are small)
};

template <int NBK>
__device__ __forceinline__ void issue_codes(const GemvP& p, const WaveView& v, int64_t n0, int i, TileRegs<NBK>& t) {
  const rsrc_t rc = make_rsrc(p.w.codes, v.N * v.K / 2);
  const int64_t grow = n0 + 8 * i + (v.lane >> 3);
  t.cw[i] = __builtin_bit_cast(
      u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                   rc, (int)oob_unless(grow < v.N, (uint32_t)((grow * v.K + v.kw) / 2 + 16 * (v.lane & 7))), 0, 0));
}

// Block scales of the wave's tile: lane l < 32 takes row l, blocks b0 .. b0 + NBK of
// the sub-slice (bs >= 32: NBK <= 8, a power of two dividing b0), as one naturally
// aligned load of the NBK u8 (or fp32) scales and one fp32 load per second-level
// group they touch.
template <int DQ, int NBK>
__device__ __forceinline__ void issue_scales(const GemvP& p, const WaveView& v, int64_t n0, TileRegs<NBK>& t) {
  const Nf4W& w = p.w;
  const int64_t nb = v.N * v.K / w.bs;
  const rsrc_t rq = DQ ? make_rsrc(w.absmax_q, nb) : make_rsrc(w.absmax, nb * 4);
  const int64_t srow = n0 + (v.lane & 31);
  const uint32_t b0 = (uint32_t)((srow * v.K + v.kw) >> w.bs_shift);  // a multiple of NBK
  const bool sok = v.lane < kRows && srow < v.N;
  if constexpr (DQ) {
    const uint32_t off = oob_unless(sok, b0);
    if constexpr (NBK == 1) t.sraw[0] = __builtin_amdgcn_raw_buffer_load_b8(rq, (int)off, 0, 0);
    else if constexpr (NBK == 2) t.sraw[0] = __builtin_amdgcn_raw_buffer_load_b16(rq, (int)off, 0, 0);
    else if constexpr (NBK == 4) t.sraw[0] = __builtin_amdgcn_raw_buffer_load_b32(rq, (int)off, 0, 0);
    else {
      const u32x2_t u = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rq, (int)off, 0, 0));
      t.sraw[0] = u[0];
      t.sraw[1] = u[1];
    }
    const rsrc_t rs = make_rsrc(w.scale2, (((nb - 1) >> w.g_shift) + 1) * 4);
    t.sf[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)oob_unless(sok, (b0 >> w.g_shift) * 4), 0, 0);
#pragma unroll
    for (int j = 1; j < NBK; ++j) t.sf[j] = 0u;
    if (v.ngr > 1) {  // groups smaller than the sub-slice (uniform; rare)
#pragma unroll
      for (int j = 1; j < NBK; ++j)
        t.sf[j] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, (int)oob_unless(sok && j < v.ngr, ((b0 >> w.g_shift) + j) * 4), 0, 0);
    }
  } else {
    const uint32_t off = oob_unless(sok, b0 * 4);
    if constexpr (NBK == 1) t.sraw[0] = __builtin_amdgcn_raw_buffer_load_b32(rq, (int)off, 0, 0);
    else if constexpr (NBK == 2) {
      const u32x2_t u = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rq, (int)off, 0, 0));
      t.sraw[0] = u[0];
      t.sraw[1] = u[1];
    } else {
#pragma unroll
      for (int h = 0; h < NBK / 4; ++h) {
        const u32x4_t u = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rq, (int)oob_unless(sok, b0 * 4 + 16 * h), 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) t.sraw[4 * h + e] = u[e];
      }
    }
  }
}

template <int DQ, int NBK>
__device__ __forceinline__ void issue_tile(const GemvP& p, const WaveView& v, int64_t n0, TileRegs<NBK>& t) {
  issue_codes(p, v, n0, 0, t);
  issue_codes(p, v, n0, 1, t);
  issue_scales<DQ>(p, v, n0, t);
  issue_codes(p, v, n0, 2, t);
  issue_codes(p, v, n0, 3, t);
}

// x of token 16 tg + rl for the wave's sub-slice: sub-step s, MFMA u -> k = kw +
// 32 (u + 4 s) + 8 q (tokens past m read as zeros).
template <int MT>
__device__ __forceinline__ void load_x(const GemvP& p, const WaveView& v, u32x4_t (&xv)[MT][2][4]) {
  const rsrc_t rx = make_rsrc(p.x, p.M * v.K * 2);
#pragma unroll
  for (int tg = 0; tg < MT; ++tg)
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        xv[tg][st][u] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         rx, (int)(((16 * tg + v.rl) * v.K + v.kw + 32 * (u + 4 * st) + 8 * v.q) * 2), 0, 0));
}

// acc[g][tg] += W~[rows 16 g .. +16 of the tile, the wave's sub-slice] x^T for the
// tile whose loads t holds.  sc_w: the wave's [32][8] block-scale region, tile: its
// [32][128-byte] code tile (both the wave's own).
template <int CD, int DQ, int NBK, int MT>
__device__ __forceinline__ void decode_mfma(const GemvP& p, const WaveView& v, const TileRegs<NBK>& t,
                                            float (*sc_w)[8], unsigned char* tile, const float2* s_pair,
                                            const u32x4_t (&xv)[MT][2][4], f32x4v_t (&acc)[2][MT]) {
  const int lane = v.lane, q = v.q, rl = v.rl;
  if (lane < kRows) {
#pragma unroll
    for (int j = 0; j < NBK; ++j) {
      if constexpr (DQ) {
        const uint32_t qb = byte_of(t.sraw[j >> 2], j & 3);
        const int gi = v.ngr == 1 ? 0 : (j >> p.w.g_shift);
        float s2 = __uint_as_float(t.sf[0]);
#pragma unroll
        for (int k = 1; k < NBK; ++k) s2 = k == gi ? __uint_as_float(t.sf[k]) : s2;
        sc_w[lane][j] = fl32_mul((float)qb, s2);
      } else {
        sc_w[lane][j] = __uint_as_float(t.sraw[j]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    // rows 16 g .. 16 g + 15 arrived with instructions 2 g and 2 g + 1; word e of
    // chunk c goes to word c % 4 of slot 4 (c / 4) + e: slot 4 s + q then holds codes
    // 8 q .. 8 q + 8 of chunks 4 s .. 4 s + 3
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * g + 8 * h + (lane >> 3), c = lane & 7;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *(uint32_t*)(tile + tile_off(row, 4 * (c >> 2) + e) + 4 * (c & 3)) = t.cw[2 * g + h][e];
    }
    __builtin_amdgcn_wave_barrier();  // LDS operations of one wave complete in order
    u32x4_t cv[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) cv[st] = *(const u32x4_t*)(tile + tile_off(16 * g + rl, q + 4 * st));
    // the row's block scales; chunk c lies in block c NBK / 8 of the sub-slice
    float scv[NBK];
    {
      const float* src = &sc_w[16 * g + rl][0];
      if constexpr (NBK >= 4) {
#pragma unroll
        for (int h = 0; h < NBK / 4; ++h) {
          const float4 f = *(const float4*)(src + 4 * h);
          scv[4 * h] = f.x, scv[4 * h + 1] = f.y, scv[4 * h + 2] = f.z, scv[4 * h + 3] = f.w;
        }
      } else if constexpr (NBK == 2) {
        const float2 f = *(const float2*)src;
        scv[0] = f.x, scv[1] = f.y;
      } else {
        scv[0] = src[0];
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float2 lv2[4][4];  // the 16 level pairs of the sub-step, requested before the first use
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int b = 0; b < 4; ++b) lv2[u][b] = *(const float2*)((const char*)s_pair + byte_x8(cv[st][u], b));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float sc = scv[((4 * st + u) * NBK) >> 3];
        u32x4_t a;
#pragma unroll
        for (int b = 0; b < 4; ++b) a[b] = pack2<CD>(fl32_mul(lv2[u][b].x, sc), fl32_mul(lv2[u][b].y, sc));
#pragma unroll
        for (int tg = 0; tg < MT; ++tg) acc[g][tg] = mfma16<CD>(a, xv[tg][st][u], acc[g][tg]);
      }
    }
  }
}

// acc[g][tg] = D[rows 16 g + 4 q .. +3][token 16 tg + rl] of this wave's sub-slice;
// waves 0 and 1 add the four waves' sums of row groups 0 and 1 in wave order and
// store them as slice sl's partial sums of rows n0 .. n0 + 31.  red: [wave][group]
// [token group][lane], a buffer of its own (the next tile's code writes may start
// while waves 0 and 1 still read it).
template <int MT>
__device__ __forceinline__ void reduce_store(const GemvP& p, const WaveView& v, f32x4v_t (&acc)[2][MT],
                                             f32x4v_t* red, int sl, int64_t n0) {
  __syncthreads();  // the previous tile's readers are done with red
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int tg = 0; tg < MT; ++tg) red[((v.wave * 2 + g) * MT + tg) * 64 + v.lane] = acc[g][tg];
  __syncthreads();
  if (v.wave < 2) {
    const int g = v.wave;
#pragma unroll
    for (int tg = 0; tg < MT; ++tg) {
      auto at = [&](int ww) { return red[((ww * 2 + g) * MT + tg) * 64 + v.lane]; };
      const f32x4v_t s = (at(0) + at(1)) + (at(2) + at(3));
      const int tok = 16 * tg + v.rl;
      if (tok < p.M) *(f32x4v_t*)(p.part + ((int64_t)sl * p.mp + tok) * p.ld + n0 + 16 * g + 4 * v.q) = s;
    }
  }
}

// Split-K GEMV kernel.  Workgroups x < p.G take W tiles: tile blockIdx.x alone
// (LOOP = 0), or tiles blockIdx.x, blockIdx.x + G, ... (LOOP = 1: the wave's x
// fragments stay in registers for every tile, and each tile's codes and scales are
// requested before the previous tile is decoded); workgroups from G on take one
// 32-row block of lora_a each.
template <int CD, int DQ, int NBK, int MT, int LOOP>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_k(GemvP p, Nf4Tables tab) {
  __shared__ __attribute__((aligned(16))) float2 s_pair[256];
  __shared__ __attribute__((aligned(16))) float s_sc[4][kRows][8];  // per wave: block scales [row][block of the sub-slice]
  __shared__ __attribute__((aligned(16))) unsigned char s_tile[4 * kRows * 128];  // per wave: swizzled code tile
  __shared__ f32x4v_t s_red[4 * 2 * MT * 64];
  WaveView v;
  const int tid = threadIdx.x;
  v.lane = tid & 63;
  v.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  v.q = v.lane >> 4;
  v.rl = v.lane & 15;
  v.K = p.w.cols;
  v.N = p.w.rows;
  const int sl = blockIdx.y;
  v.kw = (int64_t)sl * kSliceK + kWaveK * v.wave;
  v.ngr = (p.w.g_shift >= 31 || NBK <= (1 << p.w.g_shift)) ? 1 : NBK >> p.w.g_shift;
  const int G = (int)p.G;
  u32x4_t xv[MT][2][4];
  f32x4v_t acc[2][MT];

  if ((int)blockIdx.x >= G) {
    // dense rows t = row - n_pad of lora_a in the same k order; only the row groups
    // that hold rows below r
    const int64_t n0 = p.n_pad + (int64_t)(blockIdx.x - G) * kRows;
    const int groups = (int)min<int64_t>(2, (p.r - (n0 - p.n_pad) + 15) / 16);
    const rsrc_t ra = make_rsrc(p.A, (int64_t)p.r * v.K * 2);
    u32x4_t av[2][2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t t = n0 + 16 * g + v.rl - p.n_pad;
          av[g][st][u] = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                           ra, (int)oob_unless(t < p.r && g < groups,
                                               (uint32_t)((t * v.K + v.kw + 32 * (u + 4 * st) + 8 * v.q) * 2)),
                           0, 0));
        }
    load_x<MT>(p, v, xv);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int tg = 0; tg < MT; ++tg) acc[g][tg] = f32x4v_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int tg = 0; tg < MT; ++tg) acc[g][tg] = mfma16<CD>(av[g][st][u], xv[tg][st][u], acc[g][tg]);
    reduce_store<MT>(p, v, acc, s_red, sl, n0);
    return;
  }

  float (*sc_w)[8] = s_sc[v.wave];
  unsigned char* tile = s_tile + v.wave * (kRows * 128);
  auto run_tile = [&](const TileRegs<NBK>& t, int64_t n0) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int tg = 0; tg < MT; ++tg) acc[g][tg] = f32x4v_t{0.f, 0.f, 0.f, 0.f};
    decode_mfma<CD, DQ, NBK, MT>(p, v, t, sc_w, tile, s_pair, xv, acc);
    reduce_store<MT>(p, v, acc, s_red, sl, n0);
  };
  if constexpr (!LOOP) {
    // every load in flight before the first wait, in the order the decode needs them
    // (row group 0's codes, the block scales, x, row group 1's codes): a wave sees its
    // loads complete in issue order
    const int64_t n0 = (int64_t)blockIdx.x * kRows;
    TileRegs<NBK> t;
    issue_codes(p, v, n0, 0, t);
    issue_codes(p, v, n0, 1, t);
    issue_scales<DQ>(p, v, n0, t);
    load_x<MT>(p, v, xv);
    issue_codes(p, v, n0, 2, t);
    issue_codes(p, v, n0, 3, t);
    __builtin_amdgcn_sched_barrier(0);
    s_pair[tid] = level_pair(tab, tid);  // level pair of code byte tid
    __syncthreads();                     // the level pairs (everything after is the wave's own)
    run_tile(t, n0);
  } else {
    // tiles rt = blockIdx.x + G i of the n_tiles weight tiles, two register sets in turn
    const int nt = (int)(p.n_pad / kRows);
    int rt = blockIdx.x;
    TileRegs<NBK> ta, tb;
    load_x<MT>(p, v, xv);
    issue_tile<DQ>(p, v, (int64_t)rt * kRows, ta);
    s_pair[tid] = level_pair(tab, tid);
    __syncthreads();
    while (true) {
      const int rb = rt + G;
      if (rb < nt) issue_tile<DQ>(p, v, (int64_t)rb * kRows, tb);
      run_tile(ta, (int64_t)rt * kRows);
      if (rb >= nt) break;
      rt = rb + G;
      if (rt < nt) issue_tile<DQ>(p, v, (int64_t)rt * kRows, ta);
      run_tile(tb, (int64_t)rb * kRows);
      if (rt >= nt) break;
    }
  }
}

// y[m, n] = sum over slices of the partials + T[m, :] . B[n, :] + bias[n], with
// T = s (sum over slices of the lora_a rows).  Workgroup (256 columns, TB tokens):
// the thread of column n loads its lora_b row once and serves the TB tokens with
// it; thread (j, t) forms T[m0 + j, t] into LDS (the workgroups of column block 0
// also write t0 = x A^T when asked).  With r <= 64, r % 8 == 0 and S <= SM, every
// global load of a thread (its T partial sums, lora_b row, bias, and the TB x S
// partial sums of its column) is issued before the first is used, so the kernel
// waits on memory once.  Every sum over slices runs in slice order, so the result
// does not depend on scheduling.
template <int CD, int TB, int SM>
__global__ __launch_bounds__(kThreads) void k_gemv_epi(GemvP p) {
  extern __shared__ __attribute__((aligned(16))) float s_t[];  // [TB][r]
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * TB;
  const int nt = (int)min<int64_t>(TB, p.M - m0);
  const int64_t N = p.w.rows;
  const int S = p.S;
  const int64_t ss = p.mp * p.ld;
  const int64_t n = (int64_t)blockIdx.x * kThreads + tid;
  const int64_t nc = n < N ? n : N - 1;  // clamped: every lane loads, out-of-range lanes store nothing
  const float* pm0 = p.part + m0 * p.ld;
  constexpr int kTE = TB * 64 > kThreads ? TB * 64 / kThreads : 1;  // elements of T per thread (r <= 64)
  const bool fast = p.r <= 64 && (p.r & 7) == 0 && S <= SM;  // uniform
  if (fast) {
    const rsrc_t rB = make_rsrc(p.B, N * p.r * 2);
    u32x4_t bv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      bv[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              rB, (int)(uint32_t)(q * 8 < p.r ? (nc * p.r + 8 * q) * 2 : 0), 0, 0));
    // bias through a buffer of zero size when absent: the load returns 0, no branch
    const rsrc_t rb = make_rsrc(p.bias, p.bias ? N * 2 : 0);
    const uint32_t braw = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(nc * 2), 0, 0);
    // partial sums through a buffer: slices past S and tokens past m read as 0 with
    // no branch, so every load is in flight before the first wait
    const rsrc_t rp = make_rsrc(p.part, (int64_t)S * ss * 4);
    const uint32_t base = (uint32_t)(m0 * p.ld);
    uint32_t tp[kTE][SM], pv[TB][SM];
    int jt[kTE], tt[kTE];
    bool has_t[kTE];
#pragma unroll
    for (int h = 0; h < kTE; ++h) {  // element tid + 256 h of T's TB x r block
      const int e = tid + kThreads * h;
      jt[h] = e / p.r, tt[h] = e - jt[h] * p.r;
      has_t[h] = e < TB * p.r && jt[h] < nt;
#pragma unroll
      for (int i = 0; i < SM; ++i)
        tp[h][i] = __builtin_amdgcn_raw_buffer_load_b32(
            rp, (int)oob_unless(has_t[h] && i < S, (uint32_t)((i * ss + base + jt[h] * p.ld + p.n_pad + tt[h]) * 4)),
            0, 0);
    }
#pragma unroll
    for (int j = 0; j < TB; ++j)
#pragma unroll
      for (int i = 0; i < SM; ++i)
        pv[j][i] = __builtin_amdgcn_raw_buffer_load_b32(
            rp, (int)oob_unless(j < nt && i < S, (uint32_t)((i * ss + base + j * p.ld + nc) * 4)), 0, 0);
#pragma unroll
    for (int h = 0; h < kTE; ++h)
      if (has_t[h]) {
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < SM; ++i) sum += __uint_as_float(tp[h][i]);
        s_t[jt[h] * p.r + tt[h]] = sum * p.scale;
        if (p.t0 && blockIdx.x == 0) p.t0[(m0 + jt[h]) * p.r + tt[h]] = sum;
      }
    __syncthreads();
    float bf[64];
#pragma unroll
    for (int e = 0; e < 64; ++e) bf[e] = from_cd16<CD>((uint16_t)(bv[e >> 3][(e & 7) >> 1] >> (16 * (e & 1))));
    const float bias = p.bias ? from_cd16<CD>((uint16_t)braw) : 0.f;
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      if (j < nt) {
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < SM; ++i) v += __uint_as_float(pv[j][i]);
        float lora = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q * 8 < p.r) {
            // r % 8 == 0: two aligned 16-byte reads of T's row
            const float4 t0v = *(const float4*)&s_t[j * p.r + 8 * q];
            const float4 t1v = *(const float4*)&s_t[j * p.r + 8 * q + 4];
            const float tv[8] = {t0v.x, t0v.y, t0v.z, t0v.w, t1v.x, t1v.y, t1v.z, t1v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) lora = fmaf(tv[e], bf[8 * q + e], lora);
          }
        if (n < N) store_cd<CD>(p.y, (m0 + j) * p.ldy + n, v + lora + bias);
      }
    }
    return;
  }
  // any rank and slice count: the same sums in dependent rounds
  auto slice_sum = [&](const float* base) {
    float v = 0.f;
    for (int i = 0; i < S; ++i) v += base[(int64_t)i * ss];
    return v;
  };
  for (int e = tid; e < TB * p.r; e += kThreads) {
    const int j = e / p.r, t = e - j * p.r;
    if (j < nt) {
      const float sum = slice_sum(pm0 + (int64_t)j * p.ld + p.n_pad + t);
      s_t[j * p.r + t] = sum * p.scale;
      if (p.t0 && blockIdx.x == 0) p.t0[(m0 + j) * p.r + t] = sum;
    }
  }
  __syncthreads();
  const float bias = p.bias ? load_cd<CD>(p.bias, nc) : 0.f;
  for (int j = 0; j < nt; ++j) {
    const float v = slice_sum(pm0 + (int64_t)j * p.ld + nc);
    float lora = 0.f;
    for (int t = 0; t < p.r; ++t) lora = fmaf(s_t[j * p.r + t], load_cd<CD>(p.B, nc * p.r + t), lora);
    if (n < N) store_cd<CD>(p.y, (m0 + j) * p.ldy + n, v + lora + bias);
  }
}

// VALU decode GEMV: one wavefront per output row (f32, and other shapes).
template <int CD>
__global__ __launch_bounds__(kThreads) void k_gemv(Nf4W w, const void* __restrict__ x, int64_t M,
                                                   const float* __restrict__ T,
                                                   const void* __restrict__ B, int32_t r,
                                                   const void* __restrict__ bias, void* __restrict__ y,
                                                   int64_t ldy, Nf4Tables tab) {
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
    store_cd<CD>(y, (int64_t)lane * ldy + n, v);
  }
}

// Split of the contraction into S = cols / 1024 slices of 1024 elements.
struct GemvPlan {
  bool mfma;
  int32_t S;
  int64_t n_pad, r_pad, ld, mp, off_part, total;
};
GemvPlan plan_gemv(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd) {
  GemvPlan P = {};
  P.S = (int32_t)(cols / kSliceK);
  P.mfma = (cd == CD_BF16 || cd == CD_F16) && rows > 0 && cols % kSliceK == 0 && P.S >= 1;
  P.n_pad = round_up(rows, kRows);
  P.r_pad = round_up(r, kRows);
  P.ld = P.n_pad + P.r_pad;
  P.mp = round_up(m, 16);
  P.off_part = round_up(m * r * 4, 256);  // T for the VALU path
  P.total = P.off_part + (P.mfma ? round_up((int64_t)P.S * P.mp * P.ld * 4, 256) : 0);
  return P;
}

template <int CD, int DQ, int NBK, int LOOP>
void launch_gemv_mt(const GemvP& p, dim3 grid, int mt, hipStream_t st) {
  const dim3 blk(kGemvThreads);
  if (mt == 1) k_gemv_k<CD, DQ, NBK, 1, LOOP><<<grid, blk, 0, st>>>(p, host_tables());
  else if (mt == 2) k_gemv_k<CD, DQ, NBK, 2, LOOP><<<grid, blk, 0, st>>>(p, host_tables());
  else k_gemv_k<CD, DQ, NBK, 4, LOOP><<<grid, blk, 0, st>>>(p, host_tables());
}
template <int CD, int DQ, int LOOP>
void launch_gemv_nbk(const GemvP& p, dim3 grid, int nbk, int mt, hipStream_t st) {
  if (nbk == 1) launch_gemv_mt<CD, DQ, 1, LOOP>(p, grid, mt, st);
  else if (nbk == 2) launch_gemv_mt<CD, DQ, 2, LOOP>(p, grid, mt, st);
  else if (nbk == 4) launch_gemv_mt<CD, DQ, 4, LOOP>(p, grid, mt, st);
  else launch_gemv_mt<CD, DQ, 8, LOOP>(p, grid, mt, st);
}
template <int CD>
void launch_gemv_k(const GemvP& p, dim3 grid, bool dq, bool loop, int nbk, int mt, hipStream_t st) {
  if (dq && loop) launch_gemv_nbk<CD, 1, 1>(p, grid, nbk, mt, st);
  else if (dq) launch_gemv_nbk<CD, 1, 0>(p, grid, nbk, mt, st);
  else if (loop) launch_gemv_nbk<CD, 0, 1>(p, grid, nbk, mt, st);
  else launch_gemv_nbk<CD, 0, 0>(p, grid, nbk, mt, st);
}

// Workgroups the looping form aims at: as many as fit at once (256 CUs x the
// looping kernel's workgroups per CU: 3, 2, 1 for 1, 2, 4 token groups by its
// registers).
inline int64_t gemv_loop_slots(int mt) { return 256 * (mt == 1 ? 3 : mt == 2 ? 2 : 1); }

// Whether the split-K MFMA form takes the call (bf16 / f16, cols a multiple of
// 1024, a power-of-two block of at least 32, a power-of-two
// or single second-level group, codes under 2 GiB, at most 64 tokens).
bool mfma_form_ok(const LayerCall& c) {
  const GemvPlan P = plan_gemv(c.m, c.w.rows, c.w.cols, c.r, c.cd);
  return P.mfma && c.m <= 64 && c.w.bs_shift >= 5 && (!c.w.dq || c.w.g_shift >= 0) &&
         c.w.rows * c.w.cols / 2 < 0x7fff0000LL && c.m * c.w.cols * 2 < 0x7fff0000LL &&
         (int64_t)P.S * P.mp * P.ld * 4 < 0x7fff0000LL;
}

template <int CD>
int gemv_forward_t(const LayerCall& c, void* y, float* t_save) {
  const GemvPlan P = plan_gemv(c.m, c.w.rows, c.w.cols, c.r, c.cd);
  const bool mfma = mfma_form_ok(c);
  if (!mfma && c.m > kMaxM) return set_error(QLORA_ERR_UNSUPPORTED, "decode: %lld tokens need the MFMA form", (long long)c.m);
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
      p.ldy = c.ldy ? c.ldy : c.w.rows;
      p.t0 = t_save;
      p.part = (float*)(ws + P.off_part);
      p.n_pad = P.n_pad;
      p.ld = P.ld;
      p.mp = P.mp;
      p.S = P.S;
      {
        ProfScope prof(QLORA_K_GEMV, c.stream);
        const int nbk = c.w.bs_shift >= 8 ? 1 : 1 << (8 - c.w.bs_shift);  // blocks per 256-element sub-slice
        const int mt = (int)(P.mp / 16);  // token groups of 16 (1, 2 or 4)
        const int64_t nt = P.n_pad / kRows, lt = P.r_pad / kRows;  // W tiles, lora_a row blocks
        const int64_t slots = gemv_loop_slots(mt), g_loop = std::max<int64_t>(1, slots / P.S);
        // measured: the looping form wins with two or more token groups (x re-reads
        // dominate), at most 8 slices and at least 3 tiles per workgroup; at one
        // token group many independent workgroups hide latency better
        const bool loop = mt >= 2 && P.S <= 8 && nt >= 3 * g_loop;
        p.G = (int32_t)(loop ? g_loop : nt);
        const dim3 grid((unsigned)(p.G + lt), (unsigned)P.S);
        launch_gemv_k<CD>(p, grid, c.w.dq, loop, nbk, mt, c.stream);
        int rc = check_launch("k_gemv_k");
        if (rc) return rc;
      }
      ProfScope prof(QLORA_K_REDUCE, c.stream);
      // tokens per epilogue workgroup (T's rows for them sit in LDS): one up to 16
      // tokens (the most workgroups; re-reading lora_b is cheap), above that 8 when
      // the slices are few enough to hold 8 x S partial sums in registers, else 4
      int tb = c.m <= 16 ? 1 : P.S <= 8 ? 8 : 4;
      if ((size_t)tb * c.r * sizeof(float) > 65536) tb = 1;
      const size_t lds = (size_t)tb * c.r * sizeof(float);
      if (lds > 65536) return set_error(QLORA_ERR_UNSUPPORTED, "decode: rank %d too large", c.r);
      const dim3 eg((unsigned)ceil_div(c.w.rows, kThreads), (unsigned)ceil_div(c.m, tb));
      const dim3 eb(kThreads);
      if (tb == 1 && P.S <= 4) k_gemv_epi<CD, 1, 4><<<eg, eb, lds, c.stream>>>(p);
      else if (tb == 1) k_gemv_epi<CD, 1, 16><<<eg, eb, lds, c.stream>>>(p);
      else if (tb == 8 && P.S <= 4) k_gemv_epi<CD, 8, 4><<<eg, eb, lds, c.stream>>>(p);
      else if (tb == 8) k_gemv_epi<CD, 8, 8><<<eg, eb, lds, c.stream>>>(p);
      else if (P.S <= 4) k_gemv_epi<CD, 4, 4><<<eg, eb, lds, c.stream>>>(p);
      else k_gemv_epi<CD, 4, 16><<<eg, eb, lds, c.stream>>>(p);  // S > 16: the general rounds
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
      c.w, c.x, c.m, T, c.lora_b, c.r, c.bias, y, c.ldy ? c.ldy : c.w.rows, host_tables());
  return check_launch("k_gemv");
}

}  // namespace

bool gemv_mfma_ok(const LayerCall& c) { return mfma_form_ok(c); }

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
