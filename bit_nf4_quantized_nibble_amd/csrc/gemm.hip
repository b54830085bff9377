// gemm.hip -- MFMA tile engine for the QLoRA layer on gfx950, and the forward /
// backward launchers built on it.
//
// One kernel template computes C[i, j] = sum_k A'[i, k] B'[j, k] over up to two
// contraction segments, where each operand tile is staged in LDS as
// [tile index][contraction] (contraction contiguous, 128 bytes per row) by one of
// these loaders:
//   LK_ROWS      source already [index][contraction] in the compute dtype
//   LK_COLS      source [contraction][index]: transposed while staging
//   LK_COLS_F32  the same from an fp32 source, rounded to the compute dtype
//   LK_NF4_ROWS  NF4 codes of W [rows][cols] decoded to W~ along a row (forward)
//   LK_NF4_COLS  the same, transposed so the contraction runs over rows (dX)
// Decoding is the dequantization of the method, fl32(L[c] * s_b), rounded to the
// compute dtype: the operand the GEMM sees is exactly W~ = cd(deq(W)).
//
// Forward (fused dequant-GEMM, "LoRA and QLoRA, mathematically", "Tooling": the
// NF4 dequant and the LoRA matmul in one kernel):
//   T  = s x A^T                      (prologue, split-K + fixed-order reduction)
//   y  = [x | T] [W~ | B]^T + bias    (one accumulator: the LoRA term is r extra
//                                      contraction steps after the K loop)
// Backward (base frozen; qlora-rs README "Honest capability matrix", "Training"):
//   dT = s dY B,  dX = [dY | dT] [W~ ; A],  dA = dT^T x,  dB = s dY^T T0
// Reductions over a split contraction write fp32 partials and sum them in a
// fixed order, so every result is deterministic.
#include <string.h>

#include <algorithm>

#include "common.h"

namespace qnf4 {


namespace {

constexpr int kThreads = 256;
constexpr int ROWB = 128 + 16;  // LDS row pitch in bytes (128 data + 16 pad)

template <int CD>
struct Cfg {
  static constexpr int ES = (CD == CD_F32) ? 4 : 2;  // element bytes
  static constexpr int BK = 128 / ES;                // contraction elements per stage
  static constexpr int EPC = 16 / ES;                // elements per 16-byte chunk
};

enum LoadKind { LK_ROWS = 0, LK_COLS = 1, LK_COLS_F32 = 2, LK_NF4_ROWS = 3, LK_NF4_COLS = 4, LK_NONE = 5 };
enum EpiKind { EPI_CD = 0, EPI_F32_PARTIAL = 1 };

struct Opnd {
  const void* p;
  int64_t ld;    // leading dimension of the source, in elements
  int64_t nidx;  // extent along the tile index
  int64_t kmax;  // extent along the contraction
  int vec;       // 16-byte vector loads are aligned and allowed
};

struct GemmParams {
  Opnd a1, b1, a2, b2;
  Nf4W w;
  int64_t k1, k1_chunk, k2;
  int64_t M, N;  // output extent
  void* out;
  int64_t ldo;
  int64_t split_stride;  // elements between fp32 partials of consecutive splits
  const void* bias;
  float out_scale;
};

// ---------------------------------------------------------------- loaders
template <int CD>
__device__ __forceinline__ uint32_t raw_elem(const void* p, int64_t i) {
  if constexpr (CD == CD_F32) return ((const uint32_t*)p)[i];
  else return ((const uint16_t*)p)[i];
}

// 16 bytes of compute-dtype elements p[i .. i+EPC), zero beyond `avail`.
template <int CD>
__device__ __forceinline__ u32x4_t load_chunk(const void* p, int64_t i, int64_t avail, int vec) {
  constexpr int EPC = Cfg<CD>::EPC;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (avail <= 0) return v;
  if (vec && avail >= EPC) return *(const u32x4_t*)((const char*)p + i * Cfg<CD>::ES);
  if constexpr (CD == CD_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < avail) v[e] = raw_elem<CD>(p, i + e);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < avail) v[e >> 1] |= raw_elem<CD>(p, i + e) << ((e & 1) * 16);
  }
  return v;
}

// Decode 32 NF4 weights (16 bytes of codes) starting at flat element index e.
template <int CD>
__device__ __forceinline__ void decode32(const Nf4W& w, int64_t e, const float* s_lv, float (&f)[32]) {
  u32x4_t v = *(const u32x4_t*)(w.codes + e / 2);
  const float s = block_scale(w, block_of(w, e));
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t c = (v[d] >> ((j >> 1) * 8 + ((j & 1) ? 0 : 4))) & 15u;
      f[d * 8 + j] = fl32_mul(s_lv[c], s);
    }
  }
}

// Decode the (up to) 32 weights of W row `row` at columns k0 .. k0+31 for any even
// block size and any cols: one code byte and one block scale per element, zero past
// the row's end (blocks may cross rows: the block is that of the flat index).
__device__ __forceinline__ void decode32_any(const Nf4W& w, int64_t row, int64_t k0, const float* s_lv,
                                             float (&f)[32]) {
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    f[e] = 0.f;
    const int64_t k = k0 + e;
    if (k < w.cols) {
      const int64_t flat = row * w.cols + k;
      const uint32_t byte = w.codes[flat >> 1];
      const uint32_t c = (flat & 1) ? (byte & 15u) : (byte >> 4);  // element 2j in the high nibble
      f[e] = fl32_mul(s_lv[c], block_scale(w, block_of(w, flat)));
    }
  }
}

// decode32 needs each 32-element chunk inside one block with 16-byte aligned codes:
// a block size and a row length that are multiples of 32.
__device__ __forceinline__ bool chunks32(const Nf4W& w) { return (w.bs & 31) == 0 && (w.cols & 31) == 0; }

template <int CD, int LK, int BR>
__device__ __forceinline__ void load_tile(char* lds, const Opnd& o, const Nf4W& w, const float* s_lv,
                                          int64_t i0, int64_t k0, int tid) {
  constexpr int ES = Cfg<CD>::ES, BK = Cfg<CD>::BK, EPC = Cfg<CD>::EPC;
  if constexpr (LK == LK_ROWS) {
    // BR rows x 8 chunks of 16 bytes.
    for (int q = tid; q < BR * 8; q += kThreads) {
      const int row = q >> 3, c = q & 7;
      const int64_t gi = i0 + row, gk = k0 + c * EPC;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (gi < o.nidx) v = load_chunk<CD>(o.p, gi * o.ld + gk, o.kmax - gk, o.vec);
      *(u32x4_t*)(lds + row * ROWB + c * 16) = v;
    }
  } else if constexpr (LK == LK_COLS) {
    // Source [k][index]: a chunk is EPC consecutive indices at one k.
    constexpr int CPK = BR / EPC;
    for (int q = tid; q < BK * CPK; q += kThreads) {
      const int kr = q / CPK, cc = q % CPK;
      const int64_t gk = k0 + kr, gi = i0 + (int64_t)cc * EPC;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (gk < o.kmax) v = load_chunk<CD>(o.p, gk * o.ld + gi, o.nidx - gi, o.vec);
      if constexpr (CD == CD_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) *(uint32_t*)(lds + (cc * 4 + e) * ROWB + kr * 4) = v[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *(uint16_t*)(lds + (cc * 8 + e) * ROWB + kr * 2) = (uint16_t)(v[e >> 1] >> ((e & 1) * 16));
      }
    }
  } else if constexpr (LK == LK_COLS_F32) {
    // fp32 source [k][index], 4 indices per chunk, rounded to the compute dtype.
    constexpr int CPK = BR / 4;
    for (int q = tid; q < BK * CPK; q += kThreads) {
      const int kr = q / CPK, cc = q % CPK;
      const int64_t gk = k0 + kr, gi = i0 + (int64_t)cc * 4;
      float f[4] = {0.f, 0.f, 0.f, 0.f};
      if (gk < o.kmax) {
        const float* src = (const float*)o.p + gk * o.ld + gi;
        if (o.vec && gi + 4 <= o.nidx) {
          f32x4_t t = *(const f32x4_t*)src;
          f[0] = t[0]; f[1] = t[1]; f[2] = t[2]; f[3] = t[3];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gi + e < o.nidx) f[e] = src[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (CD == CD_F32)
          *(float*)(lds + (cc * 4 + e) * ROWB + kr * 4) = f[e];
        else
          *(uint16_t*)(lds + (cc * 4 + e) * ROWB + kr * 2) = to_cd16<CD>(f[e]);
      }
    }
  } else if constexpr (LK == LK_NF4_ROWS) {
    // W rows are the tile index, W columns the contraction.  One chunk = 32 weights.
    constexpr int CPR = BK / 32;
    for (int q = tid; q < BR * CPR; q += kThreads) {
      const int row = q / CPR, c = q % CPR;
      const int64_t gi = i0 + row, gk = k0 + 32 * c;
      char* dst = lds + row * ROWB + c * 32 * ES;
      if (gi < w.rows && gk < w.cols) {
        float f[32];
        if (chunks32(w)) decode32<CD>(w, gi * w.cols + gk, s_lv, f);
        else decode32_any(w, gi, gk, s_lv, f);
        if constexpr (CD == CD_F32) {
#pragma unroll
          for (int d = 0; d < 8; ++d)
            *(f32x4_t*)(dst + d * 16) = f32x4_t{f[4 * d], f[4 * d + 1], f[4 * d + 2], f[4 * d + 3]};
        } else {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            u32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = pack2<CD>(f[8 * d + 2 * e], f[8 * d + 2 * e + 1]);
            *(u32x4_t*)(dst + d * 16) = v;
          }
        }
      } else {
#pragma unroll
        for (int d = 0; d < 32 * ES / 16; ++d) *(u32x4_t*)(dst + d * 16) = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  } else if constexpr (LK == LK_NF4_COLS) {
    // W columns are the tile index, W rows the contraction (dX = dY W~).
    constexpr int CPR = BR / 32;
    for (int q = tid; q < BK * CPR; q += kThreads) {
      const int nr = q / CPR, c = q % CPR;
      const int64_t gn = k0 + nr, gk = i0 + 32 * c;
      float f[32];
      if (gn < w.rows && gk < w.cols) {
        if (chunks32(w)) decode32<CD>(w, gn * w.cols + gk, s_lv, f);
        else decode32_any(w, gn, gk, s_lv, f);
      } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) f[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        if constexpr (CD == CD_F32)
          *(float*)(lds + (32 * c + e) * ROWB + nr * 4) = f[e];
        else
          *(uint16_t*)(lds + (32 * c + e) * ROWB + nr * 2) = to_cd16<CD>(f[e]);
      }
    }
  }
}

// ---------------------------------------------------------------- MFMA
template <int CD>
__device__ __forceinline__ f32x16_t mfma16(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (CD == CD_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// One LDS stage: wave tile (32 TM) x (32 TN) at (wm, wn).  Lane l feeds row
// (l % 32) and contraction elements [8 (l / 32), 8 (l / 32) + 8) of each
// 16-element step to both operands, so A and B pair up on the same k.
template <int CD, int TM, int TN>
__device__ __forceinline__ void mma_stage(f32x16_t (&acc)[TM][TN], const char* As, const char* Bs,
                                          int wm, int wn, int lane) {
  const int r = lane & 31, h = lane >> 5;
  if constexpr (CD != CD_F32) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = *(const u32x4_t*)(As + (wm + 32 * i + r) * ROWB + (16 * ks + 8 * h) * 2);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = *(const u32x4_t*)(Bs + (wn + 32 * j + r) * ROWB + (16 * ks + 8 * h) * 2);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16<CD>(a[i], b[j], acc[i][j]);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f32x4_t a[TM][2], b[TN][2];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          a[i][u] = *(const f32x4_t*)(As + (wm + 32 * i + r) * ROWB + (16 * ks + 8 * h + 4 * u) * 4);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          b[j][u] = *(const f32x4_t*)(Bs + (wn + 32 * j + r) * ROWB + (16 * ks + 8 * h + 4 * u) * 4);
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s >> 2][s & 3], b[j][s >> 2][s & 3],
                                                             acc[i][j], 0, 0, 0);
    }
  }
}

// Row of element v of a 32x32 MFMA accumulator held by lane-half h.
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// ---------------------------------------------------------------- kernel
template <int CD, int BM, int BN, int LA1, int LB1, int LA2, int LB2, int EPI>
__global__ __launch_bounds__(kThreads) void k_gemm(GemmParams p, Nf4Tables tab) {
  constexpr int BK = Cfg<CD>::BK;
  constexpr int TM = BM / 64, TN = BN / 64;
  __shared__ __attribute__((aligned(16))) char As[BM * ROWB];
  __shared__ __attribute__((aligned(16))) char Bs[BN * ROWB];
  __shared__ float s_lv[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 16) s_lv[tid] = tab.lv[tid];
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int z = blockIdx.z;
  const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  __syncthreads();

  const int64_t kb = (int64_t)z * p.k1_chunk;
  const int64_t ke = (kb + p.k1_chunk < p.k1) ? kb + p.k1_chunk : p.k1;
  for (int64_t k = kb; k < ke; k += BK) {
    load_tile<CD, LA1, BM>(As, p.a1, p.w, s_lv, m0, k, tid);
    load_tile<CD, LB1, BN>(Bs, p.b1, p.w, s_lv, n0, k, tid);
    __syncthreads();
    mma_stage<CD, TM, TN>(acc, As, Bs, wm, wn, lane);
    __syncthreads();
  }
  if constexpr (LA2 != LK_NONE) {
    if (z == 0) {
      for (int64_t k = 0; k < p.k2; k += BK) {
        load_tile<CD, LA2, BM>(As, p.a2, p.w, s_lv, m0, k, tid);
        load_tile<CD, LB2, BN>(Bs, p.b2, p.w, s_lv, n0, k, tid);
        __syncthreads();
        mma_stage<CD, TM, TN>(acc, As, Bs, wm, wn, lane);
        __syncthreads();
      }
    }
  }

  const int h = lane >> 5, cl = lane & 31;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm + 32 * i + acc_row(v, h);
        const int64_t col = n0 + wn + 32 * j + cl;
        if (row < p.M && col < p.N) {
          float val = acc[i][j][v] * p.out_scale;
          if constexpr (EPI == EPI_CD) {
            if (p.bias) val += load_cd<CD>(p.bias, col);
            store_cd<CD>(p.out, row * p.ldo + col, val);
          } else {
            ((float*)p.out)[(int64_t)z * p.split_stride + row * p.ldo + col] = val;
          }
        }
      }
}

// out32[i, j] = sc32 * sum_z part[z, i, j] (fixed order); outcd[i, j] = cd(sccd * sum)
// over a padded [rows, ldcd] layout whose padding is zero-filled.
template <int CD>
__global__ __launch_bounds__(kThreads) void k_reduce(const float* __restrict__ part, int S, int64_t stride,
                                                     int64_t rows, int64_t cols, float sc32,
                                                     float* __restrict__ out32, float sccd,
                                                     void* __restrict__ outcd, int64_t ldcd) {
  const int64_t width = (outcd && ldcd > cols) ? ldcd : cols;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= rows * width) return;
  const int64_t i = idx / width, j = idx % width;
  if (j >= cols) {
    store_cd<CD>(outcd, i * ldcd + j, 0.f);
    return;
  }
  float sum = 0.f;
  for (int z = 0; z < S; ++z) sum += part[(int64_t)z * stride + i * cols + j];
  if (out32) out32[i * cols + j] = sum * sc32;
  if (outcd) store_cd<CD>(outcd, i * ldcd + j, sum * sccd);
}

// ---------------------------------------------------------------- host helpers
template <int CD>
Opnd opnd(const void* p, int64_t ld, int64_t nidx, int64_t kmax, int es = Cfg<CD>::ES) {
  Opnd o;
  o.p = p;
  o.ld = ld;
  o.nidx = nidx;
  o.kmax = kmax;
  o.vec = (((uintptr_t)p % 16) == 0) && ((ld * es) % 16 == 0);
  return o;
}

struct Split {
  int S;
  int64_t chunk;
};

// Split a contraction of length k over S workgroups so the grid has >= ~512 of them.
Split choose_split(int64_t tiles, int64_t k, int bk) {
  int64_t steps = ceil_div(k, bk);
  int64_t S = ceil_div(512, tiles > 0 ? tiles : 1);
  if (S > steps) S = steps;
  if (S > 64) S = 64;
  if (S < 1) S = 1;
  int64_t chunk = round_up(ceil_div(k, S), bk);
  Split sp;
  sp.S = (int)ceil_div(k, chunk);
  sp.chunk = chunk;
  return sp;
}

constexpr int64_t kAlign = 256;
inline int64_t al(int64_t b) { return round_up(b, kAlign); }

// Whether a call takes the dequantize-then-GEMM path, from its shape and flags
// alone (the workspace query must agree with the launch).  The launch also needs
// dense256_ok; when that fails the copy's workspace is simply unused.  Unless a
// path flag decides, every call above the fused forward's range (below) that the
// GEMV does not take goes this way: with each weight read from HBM, writing W~ once
// and running the dense GEMM is as fast as the fused kernels or faster from 1024
// tokens up (q_proj and gate_proj shapes, r 64, bf16); the fused kernels also need
// no rows x cols copy in the workspace.
// Internal plan flag: W~ comes from the caller (cached-dequant forward), so the
// workspace holds no copy of it.
constexpr int32_t kFlagCachedW = 1 << 20;

// Forward calls of at most this many tokens with no path flag take the fused kernel
// when its eight-wave form applies (rank a multiple of 8): there, decoding each W
// tile once per 256 tokens costs less than writing W~ and reading it back (q + gate
// forward at 128 / 256 / 512 tokens: 0.095 / 0.109 / 0.150 ms fused against
// 0.112 / 0.135 / 0.158 ms; at 1024 tokens 0.201 against 0.198).
constexpr int64_t kFusedFwdMaxM = 768;

bool dense_path(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd, int32_t flags, bool dx) {
  if (cd != CD_BF16 && cd != CD_F16) return false;
  if (cols % 64 || (dx && rows % 64)) return false;
  if (flags & QLORA_FLAG_FUSED) return false;
  if (!dx && !(flags & (QLORA_FLAG_DEQUANT_GEMM | kFlagCachedW)) && m <= kFusedFwdMaxM && r % 8 == 0) return false;
  return true;
}

// Whether the 256 x 256 GEMMs (dense or fused) may take a call of this dtype: their
// cut last round needs its slices' partial sums in the workspace.
inline bool big_tiles(int cd) { return cd == CD_BF16 || cd == CD_F16; }

// Layers whose block size is a multiple of 32 dividing cols, with cols a multiple
// of 64 (fast_layout), take the tiled kernels (decode GEMV, rank-product kernels,
// 256 x 256 GEMMs).  Every other layer the quantize call accepts (any even block
// size, any cols, blocks that run across rows) takes the generic tile engine for
// all of its products, decoding W per element.  The workspace queries do not know
// the block size; they always cover the generic engine's needs.

// Workspace plan shared by the size query and the launchers.
struct FwdPlan {
  int64_t r_pad;
  Split st;
  bool dense;
  DenseSplit dsp;  // cut of the 256 x 256 GEMM's last round (dense or fused)
  int64_t off_tcd, off_part, off_wd, off_xm, off_split, total;
};
FwdPlan plan_fwd(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd, int32_t flags) {
  FwdPlan P;
  const int es = cd_bytes(cd), bk = 128 / es;
  P.r_pad = round_up(r, 8);
  P.st = choose_split(ceil_div(m, 128) * ceil_div(r, 64), cols, bk);
  P.off_tcd = 0;
  P.off_part = al(m * P.r_pad * es);
  int64_t part = (int64_t)P.st.S * m * r * 4;
  if (skinny_ok(cd, r)) part = std::max<int64_t>(part, (int64_t)skinny_part_bytes(m, cols));
  P.off_wd = P.off_part + al(part);
  P.dense = dense_path(m, rows, cols, r, cd, flags, false);
  P.off_xm = P.off_wd + (P.dense && !(flags & kFlagCachedW) ? al(rows * cols * es) : 0);  // x M with LoRA dropout
  P.off_split = P.off_xm + ((flags & QLORA_FLAG_DROPOUT) ? al(m * cols * es) : 0);
  P.dsp = dense_split(m, rows, cols, !P.dense);
  P.total = P.off_split + (big_tiles(cd) ? al(dense_split_bytes(P.dsp)) : 0);
  return P;
}

struct BwdPlan {
  int64_t r_pad;
  Split st, sdt, sda, sdb;
  bool dense;
  bool sk, sk_n;       // the skinny kernels take the rank products (dT and dB also need rows % 8)
  int64_t n_pad, m_pad;  // contractions rounded up to whole 64-element stages
  DenseSplit dsp;        // cut of the 256 x 256 dX GEMM's last round (dense or fused)
  int64_t off_t0, off_dt, off_dtcd, off_bt, off_dtt, off_t0t, off_part, off_part2, off_wdt, off_xm, off_zero, off_split,
      off_at, total;
};
BwdPlan plan_bwd(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd, int32_t flags) {
  BwdPlan P;
  const int es = cd_bytes(cd), bk = 128 / es;
  P.r_pad = round_up(r, 8);
  P.st = choose_split(ceil_div(m, 128) * ceil_div(r, 64), cols, bk);
  P.sdt = choose_split(ceil_div(m, 128) * ceil_div(r, 64), rows, bk);
  P.sda = choose_split(ceil_div(r, 64) * ceil_div(cols, 128), m, bk);
  P.sdb = choose_split(ceil_div(rows, 128) * ceil_div(r, 64), m, bk);
  P.sk = skinny_ok(cd, r);
  P.sk_n = P.sk && rows % 8 == 0;
  P.n_pad = round_up(rows, 64);
  P.m_pad = round_up(m, 64);
  P.off_t0 = 0;
  P.off_dt = P.off_t0 + al(m * r * 4);
  P.off_dtcd = P.off_dt + al(m * r * 4);
  P.off_bt = P.off_dtcd + al(m * P.r_pad * es);
  P.off_dtt = P.off_bt + (P.sk_n && r % 8 ? al(r * P.n_pad * es) : 0);  // B^T only when lora_b cannot be read as stored
  P.off_t0t = P.off_dtt + (P.sk ? al(r * P.m_pad * es) : 0);
  P.off_part = P.off_t0t + (P.sk_n ? al(r * P.m_pad * es) : 0);
  int64_t part = (int64_t)P.st.S * m * r * 4;
  part = std::max<int64_t>(part, (int64_t)P.sdt.S * m * r * 4);
  part = std::max<int64_t>(part, (int64_t)P.sda.S * r * cols * 4);
  part = std::max<int64_t>(part, (int64_t)P.sdb.S * rows * r * 4);
  if (P.sk) {
    part = std::max<int64_t>(part, (int64_t)skinny_part_bytes(m, cols));        // T0
    part = std::max<int64_t>(part, (int64_t)skinny_part_bytes(cols, P.m_pad));  // dA
  }
  if (P.sk_n) {
    part = std::max<int64_t>(part, (int64_t)skinny_part_bytes(m, P.n_pad));     // dT
    part = std::max<int64_t>(part, (int64_t)skinny_part_bytes(rows, P.m_pad));  // dB
  }
  // dB's partial sums live beside dA's so that one launch reduces both
  P.off_part2 = P.off_part + al(part);
  P.off_wdt = P.off_part2 + (P.sk_n ? al((int64_t)skinny_part_bytes(rows, P.m_pad)) : 0);
  P.dense = dense_path(m, rows, cols, r, cd, flags, true);
  // with LoRA dropout: x M, and a zero [m, r_pad] operand for the base-only dX GEMM
  P.off_xm = P.off_wdt + (P.dense ? al(rows * cols * es) : 0);
  const bool drop = (flags & QLORA_FLAG_DROPOUT) != 0;
  P.off_zero = P.off_xm + (drop ? al(m * cols * es) : 0);
  P.off_split = P.off_zero + (drop ? al(m * P.r_pad * es) : 0);
  P.dsp = dense_split(m, cols, rows, !P.dense);
  // A^T [cols][r_pad] in cd: the W-side rows of the dense dX GEMM's low-rank tail
  P.off_at = P.off_split + (big_tiles(cd) ? al(dense_split_bytes(P.dsp)) : 0);
  P.total = P.off_at + (P.dense ? al(cols * P.r_pad * es) : 0);
  return P;
}

template <int CD>
int run_reduce(const float* part, const Split& sp, int64_t rows, int64_t cols, float sc32, float* out32,
               float sccd, void* outcd, int64_t ldcd, hipStream_t s) {
  const int64_t width = (outcd && ldcd > cols) ? ldcd : cols;
  const int64_t n = rows * width;
  if (n == 0) return QLORA_OK;
  ProfScope prof(QLORA_K_REDUCE, s);
  k_reduce<CD><<<dim3((unsigned)ceil_div(n, kThreads)), dim3(kThreads), 0, s>>>(
      part, sp.S, rows * cols, rows, cols, sc32, out32, sccd, outcd, ldcd);
  return check_launch("k_reduce");
}

template <int CD, int BM, int BN, int LA1, int LB1, int LA2, int LB2, int EPI>
int run_gemm(GemmParams& p, int S, int kind, hipStream_t s) {
  dim3 grid((unsigned)ceil_div(p.N, BN), (unsigned)ceil_div(p.M, BM), (unsigned)S);
  ProfScope prof(kind, s);
  k_gemm<CD, BM, BN, LA1, LB1, LA2, LB2, EPI><<<grid, dim3(kThreads), 0, s>>>(p, host_tables());
  return check_launch("k_gemm");
}

GemmParams base_params(const LayerCall& c) {
  GemmParams p = {};
  p.w = c.w;
  p.out_scale = 1.0f;
  return p;
}

// T0 (or s T0) = x A^T as fp32 partials, reduced into out32 (scale sc32) and a
// compute-dtype copy outcd [m, r_pad] (scale sccd).
template <int CD>
int lora_down(const LayerCall& c, const void* lx, const Split& sp, float* part, float* out32, float sc32,
              void* outcd, float sccd, int64_t r_pad) {
  const int64_t K = c.w.cols;
  GemmParams p = base_params(c);
  p.a1 = opnd<CD>(lx, K, c.m, K);
  p.b1 = opnd<CD>(c.lora_a, K, c.r, K);
  p.k1 = K;
  p.k1_chunk = sp.chunk;
  p.M = c.m;
  p.N = c.r;
  p.out = part;
  p.ldo = c.r;
  p.split_stride = c.m * c.r;
  int rc = run_gemm<CD, 128, 64, LK_ROWS, LK_ROWS, LK_NONE, LK_NONE, EPI_F32_PARTIAL>(p, sp.S, QLORA_K_LORA_DOWN, c.stream);
  if (rc) return rc;
  return run_reduce<CD>(part, sp, c.m, c.r, sc32, out32, sccd, outcd, r_pad, c.stream);
}

template <int CD>
int forward_gemm(const LayerCall& c, void* y, float* t_save) {
  const int64_t M = c.m, N = c.w.rows, K = c.w.cols;
  FwdPlan P = plan_fwd(M, N, K, c.r, CD, c.flags);
  char* ws = (char*)c.ws;
  void* tcd = ws + P.off_tcd;
  float* part = (float*)(ws + P.off_part);
  int rc;
  const bool fast = fast_layout(c.w);
  // input of the low-rank branch: x, or x M with LoRA dropout
  const void* lx = c.x;
  if (c.drop_mask) {
    if ((rc = apply_mask(CD, c.x, c.drop_mask, M * K, ws + P.off_xm, c.stream))) return rc;
    lx = ws + P.off_xm;
  }
  // T0 = x A^T (fp32, saved on request) and T = s T0 in cd for the GEMM's tail.  On
  // the dequantize-then-GEMM path the reduction of the skinny kernel's slices rides
  // on the dequantize launch.
  const bool dense = fast && P.dense && dense256_ok(c, false);
  SkRed red;
  bool red_pending = false;
  if (fast && skinny_ok(CD, c.r)) {
    int S;
    if ((rc = skinny(CD, false, lx, K, M, c.lora_a, K, M, c.r, K, part, &S, c.stream, QLORA_K_LORA_DOWN))) return rc;
    red.part = part;
    red.S = S;
    red.P = M;
    red.R = c.r;
    red.out32 = t_save;
    red.sccd = c.scale;
    red.outcd = tcd;
    red.ldcd = P.r_pad;
    if (dense) red_pending = true;
    else if ((rc = skinny_reduce_jobs(CD, red, nullptr, c.stream))) return rc;
  } else if ((rc = lora_down<CD>(c, lx, P.st, part, t_save, 1.0f, tcd, c.scale, P.r_pad))) {
    return rc;
  }
  if (dense) {
    void* wd = ws + P.off_wd;
    if ((rc = dequant_into(c.w, CD, wd, false, c.stream, red_pending ? &red : nullptr))) return rc;
    return dense256_forward(c, wd, tcd, P.r_pad, y, P.dsp, ws + P.off_split);
  }
  if (fast && fused256_ok(c, false)) return fused256_forward(c, tcd, P.r_pad, y, P.dsp, ws + P.off_split);

  GemmParams p = base_params(c);
  p.a1 = opnd<CD>(c.x, K, M, K);
  p.b1 = opnd<CD>(nullptr, 0, N, K);
  p.k1 = K;
  p.k1_chunk = round_up(K, Cfg<CD>::BK);
  p.a2 = opnd<CD>(tcd, P.r_pad, M, P.r_pad);
  p.b2 = opnd<CD>(c.lora_b, c.r, N, c.r);
  p.k2 = P.r_pad;
  p.M = M;
  p.N = N;
  p.out = y;
  p.ldo = N;
  p.bias = c.bias;
  return run_gemm<CD, 128, 128, LK_ROWS, LK_NF4_ROWS, LK_ROWS, LK_ROWS, EPI_CD>(p, 1, QLORA_K_FWD_GEMM, c.stream);
}

template <int CD>
int backward_gemm(const LayerCall& c, const void* dy, const float* t_saved, void* dx, float* d_a,
                  float* d_b) {
  const int64_t M = c.m, N = c.w.rows, K = c.w.cols, r = c.r;
  BwdPlan P = plan_bwd(M, N, K, c.r, CD, c.flags);
  const bool fast = fast_layout(c.w);
  if (!fast) P.sk = P.sk_n = P.dense = false;  // the generic engine for every product (see fast_layout)
  char* ws = (char*)c.ws;
  float* t0 = (float*)(ws + P.off_t0);
  float* dt = (float*)(ws + P.off_dt);
  void* dtcd = ws + P.off_dtcd;
  float* part = (float*)(ws + P.off_part);
  int rc;
  // input of the low-rank branch: x, or x M with LoRA dropout
  const void* lx = c.x;
  if (c.drop_mask) {
    if ((rc = apply_mask(CD, c.x, c.drop_mask, M * K, ws + P.off_xm, c.stream))) return rc;
    lx = ws + P.off_xm;
  }

  // T0 = x A^T (recomputed unless the forward saved it).
  const float* T0 = t_saved;
  if (!T0) {
    if (P.sk) {
      int S;
      if ((rc = skinny(CD, false, lx, K, M, c.lora_a, K, M, r, K, part, &S, c.stream, QLORA_K_LORA_DOWN))) return rc;
      if ((rc = skinny_reduce(CD, part, S, M, r, 1.0f, t0, false, 0.f, nullptr, 0, c.stream))) return rc;
    } else if ((rc = lora_down<CD>(c, lx, P.st, part, t0, 1.0f, nullptr, 0.f, 0))) {
      return rc;
    }
    T0 = t0;
  }

  // dT = s dY B  -> fp32 [M, r] and a compute-dtype copy [M, r_pad].  On the skinny
  // path the same launch writes the operands of dA and dB: dT^T [r][m_pad] (the cd
  // copy transposed) and T0^T [r][m_pad] rounded to cd, both zero past M.
  void* dtt = ws + P.off_dtt;
  void* t0t = ws + P.off_t0t;
  // A^T [K][r_pad] (zero past r) for the low-rank tail of the dense dX GEMM; its
  // transpose shares a launch with B^T's on the skinny path.
  const bool dense_dx = dx && P.dense && dense256_ok(c, true);
  void* at = dense_dx ? (void*)(ws + P.off_at) : nullptr;
  TransposeSpec ta;
  ta.src = c.lora_a;
  ta.ld_src = K;
  ta.rows = r;
  ta.cols = K;
  ta.dst = at;
  ta.ld_dst = P.r_pad;
  SkRed red_dt;  // the dT reduction, launched here or riding on W~^T's dequantize
  bool red_dt_pending = false;
  if (P.sk_n) {
    // dY against lora_b: read as stored when r is a multiple of 8 (A^T's transpose
    // rides on the same launch), else against a transposed copy B^T [r][n_pad], zero
    // past N
    SkSpec sd;
    sd.a = dy;
    sd.lda = N;
    sd.arows = M;
    sd.P = M;
    sd.R = r;
    sd.Kc = P.n_pad;
    const TransposeSpec* ride = nullptr;
    if (r % 8 == 0) {
      sd.b = c.lora_b;
      sd.ldb = r;
      sd.bt = true;
      sd.brows = N;
      ride = at ? &ta : nullptr;
    } else {
      void* bt = ws + P.off_bt;
      TransposeSpec tb;
      tb.src = c.lora_b;
      tb.ld_src = r;
      tb.rows = N;
      tb.cols = r;
      tb.dst = bt;
      tb.ld_dst = P.n_pad;
      if ((rc = transpose_jobs(CD, tb, at ? &ta : nullptr, c.stream))) return rc;
      sd.b = bt;
      sd.ldb = P.n_pad;
    }
    int S;
    if ((rc = skinny_jobs(CD, false, sd, part, &S, nullptr, nullptr, nullptr, c.stream, QLORA_K_BWD_DT, ride)))
      return rc;
    red_dt.part = part;
    red_dt.S = S;
    red_dt.P = M;
    red_dt.R = r;
    red_dt.sc32 = c.scale;
    red_dt.out32 = dt;
    red_dt.sccd = c.scale;
    red_dt.outcd = dtcd;
    red_dt.ldcd = P.r_pad;
    red_dt.outt = dtt;
    red_dt.ldt = P.m_pad;
    red_dt.side = T0;
    red_dt.side_t = t0t;
    if (dense_dx) red_dt_pending = true;
    else if ((rc = skinny_reduce_jobs(CD, red_dt, nullptr, c.stream))) return rc;
  } else {
    if (at && (rc = transpose_jobs(CD, ta, nullptr, c.stream))) return rc;
    GemmParams p = base_params(c);
    p.a1 = opnd<CD>(dy, N, M, N);
    p.b1 = opnd<CD>(c.lora_b, r, r, N);  // source [n][t]: transposed while staging
    p.k1 = N;
    p.k1_chunk = P.sdt.chunk;
    p.M = M;
    p.N = r;
    p.out = part;
    p.ldo = r;
    p.split_stride = M * r;
    rc = run_gemm<CD, 128, 64, LK_ROWS, LK_COLS, LK_NONE, LK_NONE, EPI_F32_PARTIAL>(p, P.sdt.S, QLORA_K_BWD_DT, c.stream);
    if (rc) return rc;
    rc = run_reduce<CD>(part, P.sdt, M, r, c.scale, dt, c.scale, dtcd, P.r_pad, c.stream);
    if (rc) return rc;
  }

  // dX = dY W~ + dT A (the contraction runs over W's rows): W~^T written once and a
  // dense GEMM, or the fused dequant.  With LoRA dropout the GEMM gets a zero dT
  // (base product only) and the masked low-rank term is added afterwards.
  const void* dt_gemm = dtcd;
  if (dx && c.drop_mask) {
    if ((rc = zero_fill(ws + P.off_zero, M * P.r_pad * cd_bytes(CD), c.stream))) return rc;
    dt_gemm = ws + P.off_zero;
  }
  if (dense_dx) {
    void* wdt = ws + P.off_wdt;
    if ((rc = dequant_into(c.w, CD, wdt, true, c.stream, red_dt_pending ? &red_dt : nullptr))) return rc;
    if ((rc = dense256_dx(c, dy, wdt, dt_gemm, P.r_pad, dx, P.dsp, ws + P.off_split, at))) return rc;
  } else if (dx && fast && fused256_ok(c, true)) {
    rc = fused256_dx(c, dy, dt_gemm, P.r_pad, dx, P.dsp, ws + P.off_split);
    if (rc) return rc;
  } else if (dx) {
    GemmParams p = base_params(c);
    p.a1 = opnd<CD>(dy, N, M, N);
    p.b1 = opnd<CD>(nullptr, 0, K, N);
    p.k1 = N;
    p.k1_chunk = round_up(N, Cfg<CD>::BK);
    p.a2 = opnd<CD>(dt_gemm, P.r_pad, M, P.r_pad);
    p.b2 = opnd<CD>(c.lora_a, K, K, r);  // source [t][k]: transposed while staging
    p.k2 = P.r_pad;
    p.M = M;
    p.N = K;
    p.out = dx;
    p.ldo = K;
    rc = run_gemm<CD, 128, 128, LK_ROWS, LK_NF4_COLS, LK_ROWS, LK_COLS, EPI_CD>(p, 1, QLORA_K_BWD_DX, c.stream);
    if (rc) return rc;
  }
  if (dx && c.drop_mask &&
      (rc = rank_add_masked(CD, dx, c.drop_mask, dtcd, P.r_pad, c.lora_a, r, M, K, c.stream)))
    return rc;

  // dA = dT^T x and dB = s dY^T T0 (contractions over tokens): on the skinny path
  // both products, then one launch that reduces both.
  if (P.sk_n) {
    float* part2 = (float*)(ws + P.off_part2);
    int Sa, Sb;
    SkSpec pa, pb;  // dA: x^T against dT^T;  dB: dY^T against T0^T (one launch)
    pa.a = lx;
    pa.lda = K;
    pa.arows = M;
    pa.b = dtt;
    pa.ldb = P.m_pad;
    pa.P = K;
    pa.R = r;
    pa.Kc = P.m_pad;
    pb.a = dy;
    pb.lda = N;
    pb.arows = M;
    pb.b = t0t;
    pb.ldb = P.m_pad;
    pb.P = N;
    pb.R = r;
    pb.Kc = P.m_pad;
    if ((rc = skinny_jobs(CD, true, pa, part, &Sa, &pb, part2, &Sb, c.stream, QLORA_K_BWD_DA))) return rc;
    SkRed ra, rb;
    ra.part = part;
    ra.S = Sa;
    ra.P = K;
    ra.R = r;
    ra.out32 = d_a;
    ra.trans = true;
    rb.part = part2;
    rb.S = Sb;
    rb.P = N;
    rb.R = r;
    rb.sc32 = c.scale;
    rb.out32 = d_b;
    return skinny_reduce_jobs(CD, ra, &rb, c.stream);
  }
  // dA = dT^T x  (contraction over tokens).
  if (P.sk) {
    // dT^T [r][m_pad] in cd (the operand the dX uses), zero past M
    if ((rc = transpose_small(CD, dtcd, false, P.r_pad, M, r, 1.0f, dtt, P.m_pad, c.stream))) return rc;
    int S;
    if ((rc = skinny(CD, true, lx, K, M, dtt, P.m_pad, K, r, P.m_pad, part, &S, c.stream, QLORA_K_BWD_DA))) return rc;
    if ((rc = skinny_reduce(CD, part, S, K, r, 1.0f, d_a, true, 0.f, nullptr, 0, c.stream))) return rc;
  } else {
    GemmParams p = base_params(c);
    p.a1 = opnd<CD>(dtcd, P.r_pad, r, M);  // source [m][t]
    p.b1 = opnd<CD>(lx, K, K, M);          // source [m][k]
    p.k1 = M;
    p.k1_chunk = P.sda.chunk;
    p.M = r;
    p.N = K;
    p.out = part;
    p.ldo = K;
    p.split_stride = r * K;
    rc = run_gemm<CD, 64, 128, LK_COLS, LK_COLS, LK_NONE, LK_NONE, EPI_F32_PARTIAL>(p, P.sda.S, QLORA_K_BWD_DA, c.stream);
    if (rc) return rc;
    rc = run_reduce<CD>(part, P.sda, r, K, 1.0f, d_a, 0.f, nullptr, 0, c.stream);
    if (rc) return rc;
  }

  // dB = s dY^T T0  (contraction over tokens; the skinny case returned above).
  {
    GemmParams p = base_params(c);
    p.a1 = opnd<CD>(dy, N, N, M);         // source [m][n]
    p.b1 = opnd<CD>(T0, r, r, M, 4);      // fp32 source [m][t]
    p.k1 = M;
    p.k1_chunk = P.sdb.chunk;
    p.M = N;
    p.N = r;
    p.out = part;
    p.ldo = r;
    p.split_stride = N * r;
    rc = run_gemm<CD, 128, 64, LK_COLS, LK_COLS_F32, LK_NONE, LK_NONE, EPI_F32_PARTIAL>(p, P.sdb.S, QLORA_K_BWD_DB, c.stream);
    if (rc) return rc;
    rc = run_reduce<CD>(part, P.sdb, N, r, c.scale, d_b, 0.f, nullptr, 0, c.stream);
    if (rc) return rc;
  }
  return QLORA_OK;
}

// Forward with W~ [rows][cols] in cd that the caller dequantized once and keeps
// (cached-dequant mode): T = s x A^T by the rank-product kernels, then the dense
// 256 x 256 GEMM reads W~ where it lies.
template <int CD>
int forward_cached_t(const LayerCall& c, const void* wd, void* y, float* t_save) {
  const int64_t M = c.m, N = c.w.rows, K = c.w.cols;
  const FwdPlan P = plan_fwd(M, N, K, c.r, CD, c.flags | kFlagCachedW);
  char* ws = (char*)c.ws;
  void* tcd = ws + P.off_tcd;
  float* part = (float*)(ws + P.off_part);
  int rc;
  if (skinny_ok(CD, c.r)) {
    int S;
    if ((rc = skinny(CD, false, c.x, K, M, c.lora_a, K, M, c.r, K, part, &S, c.stream, QLORA_K_LORA_DOWN))) return rc;
    SkRed red;
    red.part = part;
    red.S = S;
    red.P = M;
    red.R = c.r;
    red.out32 = t_save;
    red.sccd = c.scale;
    red.outcd = tcd;
    red.ldcd = P.r_pad;
    if ((rc = skinny_reduce_jobs(CD, red, nullptr, c.stream))) return rc;
  } else if ((rc = lora_down<CD>(c, c.x, P.st, part, t_save, 1.0f, tcd, c.scale, P.r_pad))) {
    return rc;
  }
  return dense256_forward(c, wd, tcd, P.r_pad, y, P.dsp, ws + P.off_split);
}

}  // namespace

size_t cached_fwd_workspace_bytes(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd) {
  return (size_t)plan_fwd(m, rows, cols, r, cd, QLORA_FLAG_DEQUANT_GEMM | kFlagCachedW).total;
}

int launch_forward_cached(const LayerCall& c, const void* wd, void* y, float* t_save) {
  if (c.cd == CD_BF16) return forward_cached_t<CD_BF16>(c, wd, y, t_save);
  if (c.cd == CD_F16) return forward_cached_t<CD_F16>(c, wd, y, t_save);
  return set_error(QLORA_ERR_DTYPE, "linear_fwd_cached: compute dtype must be bf16 or f16");
}

int gemv_forward(const LayerCall& c, void* y, float* t_save);  // gemv.hip
size_t gemv_workspace_bytes(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd);
bool gemv_mfma_ok(const LayerCall& c);
// The decode GEMV takes every call of at most 16 tokens (on the VALU where its MFMA
// form does not apply), and calls of 17 to 64 tokens that carry no path flag when
// its MFMA form applies (one decode of W~ serves up to four 16-token column groups).
constexpr int64_t kGemvMaxM = 16, kGemvMfmaMaxM = 64;
inline bool gemv_candidate(int64_t m, int32_t flags) {
  if (flags & QLORA_FLAG_DROPOUT) return false;
  return m <= kGemvMaxM || (m <= kGemvMfmaMaxM && !(flags & (QLORA_FLAG_FUSED | QLORA_FLAG_DEQUANT_GEMM)));
}

size_t fwd_workspace_bytes(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd, int32_t flags) {
  // A GEMV candidate may still run on the GEMM path (a layout the GEMV does not take:
  // the query does not see the block size): room for both.  At most 16 tokens the
  // GEMM path is the generic engine, which needs only T and the rank-product partial
  // sums (the start of its plan).
  const FwdPlan P = plan_fwd(m, rows, cols, r, cd, flags);
  if (!gemv_candidate(m, flags)) return (size_t)P.total;
  return std::max(gemv_workspace_bytes(m, rows, cols, r, cd), (size_t)(m <= kGemvMaxM ? P.off_wd : P.total));
}

size_t bwd_workspace_bytes(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd, int32_t flags) {
  return (size_t)plan_bwd(m, rows, cols, r, cd, flags).total;
}

bool gemv_route(const LayerCall& c) {
  return !c.drop_mask && fast_layout(c.w) && gemv_candidate(c.m, c.flags) && (c.m <= kGemvMaxM || gemv_mfma_ok(c));
}

int launch_forward(const LayerCall& c, void* y, float* t_save) {
  if (gemv_route(c)) return gemv_forward(c, y, t_save);
  switch (c.cd) {
    case CD_BF16: return forward_gemm<CD_BF16>(c, y, t_save);
    case CD_F16: return forward_gemm<CD_F16>(c, y, t_save);
    case CD_F32: return forward_gemm<CD_F32>(c, y, t_save);
  }
  return set_error(QLORA_ERR_DTYPE, "forward: bad compute dtype %d", c.cd);
}

int launch_backward(const LayerCall& c, const void* dy, const float* t_saved, void* dx, float* d_a,
                    float* d_b) {
  switch (c.cd) {
    case CD_BF16: return backward_gemm<CD_BF16>(c, dy, t_saved, dx, d_a, d_b);
    case CD_F16: return backward_gemm<CD_F16>(c, dy, t_saved, dx, d_a, d_b);
    case CD_F32: return backward_gemm<CD_F32>(c, dy, t_saved, dx, d_a, d_b);
  }
  return set_error(QLORA_ERR_DTYPE, "backward: bad compute dtype %d", c.cd);
}

}  // namespace qnf4
