// gemm256.hip -- the two big fused dequant-GEMMs of the QLoRA layer (bf16 / f16
// compute) on gfx950:
//
//   forward  y  = [x | T] [W~ | B]^T (+ bias)     T = s x A^T, W~ = cd(fl32(L[c] s_b))
//   dX       dX = [dY | dT] [W~ ; A]              dT = s dY B
//
// ("LoRA and QLoRA, mathematically", "Tooling": the NF4 dequant and the LoRA matmul
// fused in one kernel; the backward keeps W frozen, qlora-rs README "Honest
// capability matrix").
//
// Tile 256 x 256 per workgroup, 4 waves in 2 x 2, each owning a 128 x 128 block
// of the output as 4 x 4 MFMA 32x32x16 tiles (256 fp32 accumulators per lane, in
// the accumulation registers).  The contraction advances 64 elements per stage;
// both operand tiles live in LDS as [tile index][contraction] rows of 128 bytes
// (+16 bytes pad so that the 16-byte fragment reads of 16 consecutive rows hit
// distinct banks), double buffered (2 x 72 KiB).
//
// Pipeline (one wave per SIMD, so all latency hiding is explicit):
//   * global data for a stage is fetched two stages ahead into one of two
//     register sets, with buffer loads (32-bit offsets, out-of-range reads
//     return zero, so ragged tails need no branches);
//   * while the 64 MFMAs of stage k run from LDS buffer k % 2, the lanes decode
//     the NF4 codes of stage k+1 and write both tiles of that stage into the other
//     buffer, a quarter per 16-element MFMA step; fragments for the next MFMA
//     step are read while the current one issues.
//
// NF4 decode (the method's dequantization, exact): code c -> fl32(L[c] * s_b) ->
// compute dtype; L sits in LDS (16 words in 16 banks: conflict-free lookups).
//   forward: lane t owns row t of the W tile: 64 codes (32 bytes) per stage;
//   dX:      the contraction runs over W's rows, so a lane decodes an 8 x 8 block
//            (8 rows x one 32-bit word of codes) and packs pairs from adjacent
//            rows, writing 16-byte runs of the transposed tile [k][n].
// The workgroup -> tile map keeps the tiles that run concurrently on one XCD
// (workgroups b, b + 8, ... share an XCD) in the same row block, so their common
// activation tile stays in that XCD's L2.
#include "common.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int TILE = 256;
constexpr int BK = 64;                    // contraction elements per stage (16-bit dtypes)
constexpr int ROWB = 128;                 // LDS row: 64 elements, 8 chunks of 16 bytes (swizzled)
constexpr int TILE_BYTES = TILE * ROWB;   // 32 KiB per operand tile
constexpr int LV_OFF = 4 * TILE_BYTES;    // the 16-entry level table sits after the 4 tiles

enum Mode { MODE_FWD = 0, MODE_DX = 1 };

struct Big {
  const void* a1;     // [M, ld_a1] cd: x (fwd) or dY (dX)
  int64_t ld_a1;
  const void* a2;     // [M, r_pad] cd: T (fwd) or dT (dX)
  int64_t r_pad;
  const void* b2;     // fwd: lora_b [N, r]; dX: lora_a [r, K]
  Nf4W w;
  int64_t M;
  int64_t NB;         // output columns: N (fwd) or K (dX)
  int64_t K1;         // main contraction: K (fwd) or N (dX)
  int32_t r;
  int32_t tiles_m, tiles_n;
  void* out;          // [M, NB] cd
  const void* bias;   // [NB] cd (fwd) or null
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4_t ld128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t ld8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}
// Out-of-range offset: the top bit puts it past every buffer (all are < 2 GiB).
__device__ __forceinline__ uint32_t oob_unless(bool ok, uint32_t off) {
  return off | ((uint32_t)(!ok) << 31);
}

// LDS layout of a tile: row r holds contraction elements [0, 64) as 8 chunks of
// 16 bytes; logical chunk c sits at physical chunk c ^ swz(r).  Reads of one
// chunk from 16 consecutive rows then touch every 4-bank group once, whether the
// LDS serves 8 lanes over 32 banks or 16 lanes over 64 banks.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int chunk_addr(int row, int c) { return row * ROWB + ((c ^ swz(row)) << 4); }

__device__ __forceinline__ void tile_of(const Big& p, int& tm, int& tn) {
  const int b = blockIdx.x;
  const int T = p.tiles_m * p.tiles_n;
  int t = b;
  if ((T & 7) == 0) t = (b & 7) * (T >> 3) + (b >> 3);  // XCD-contiguous chunks
  tm = t / p.tiles_n;
  tn = t % p.tiles_n;
}

// The NF4 codes (and raw block scales) a lane fetches for one stage.
struct CodeRegs {
  u32x4_t c[2];   // fwd: 32 bytes of codes of W row tid
  uint32_t cw[8]; // dX: one word of codes from each of 8 W rows
  uint32_t sq[8]; // u8 block scale (double quant) as loaded
  float sf[8];    // second-level scale (double quant) or the fp32 absmax
};

template <int DQ>
__device__ __forceinline__ float scale_of(const CodeRegs& R, int i) {
  if constexpr (DQ) return (float)R.sq[i] * R.sf[i];
  else return R.sf[i];
}

// Per-lane constant parts of the addresses (all byte offsets fit in 31 bits).
struct Lane {
  uint32_t a_off[8];     // activation: global byte offset of the chunk this lane copies, stage 0
  uint32_t a_col[8];     // its element column within a stage (tail check)
  uint32_t w_row;        // fwd: this lane's W row; dX: first of its 8 W rows within a stage
  uint32_t w_col;        // dX: first of this lane's 8 W columns
  uint32_t row_bytes;    // bytes of codes per W row (cols / 2)
  uint32_t row_blocks;   // blocks per W row (cols / block_size)
};

// Activation tile of stage kt straight from global memory into LDS buffer `dst`:
// instruction i of wave w fills rows 8 (4 i + w) .. +8; lane l lands in physical
// chunk l % 8 of row l / 8 and so fetches the logical chunk that maps there.
template <int MODE>
__device__ __forceinline__ void fetch_a(const Big& p, const Lane& L, rsrc_t ra, char* dst, int wave, uint32_t kt) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool ok = MODE == MODE_FWD || kt * BK + L.a_col[i] < (uint32_t)p.K1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dst + (4 * i + wave) * 1024), 16,
                                             (int)oob_unless(ok, L.a_off[i] + kt * (BK * 2)), 0, 0, 0);
  }
}

template <int MODE, int DQ>
__device__ __forceinline__ void fetch_w(CodeRegs& R, const Big& p, const Lane& L, rsrc_t rc, rsrc_t rq,
                                        rsrc_t rs, uint32_t kt) {
  const Nf4W& w = p.w;
  const uint32_t bsh = (uint32_t)w.bs_shift, gsh = (uint32_t)w.g_shift;
  if constexpr (MODE == MODE_FWD) {
    const bool ok = L.w_row < (uint32_t)w.rows;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t col = kt * BK + 32 * j;
      R.c[j] = ld128(rc, oob_unless(ok, L.w_row * L.row_bytes + col / 2));
      const uint32_t b = L.w_row * L.row_blocks + (col >> bsh);
      if constexpr (DQ) {
        R.sq[j] = ld8(rq, oob_unless(ok, b));
        R.sf[j] = __uint_as_float(ld32(rs, oob_unless(ok, (b >> gsh) * 4)));
      } else {
        R.sf[j] = __uint_as_float(ld32(rq, oob_unless(ok, b * 4)));
      }
    }
  } else {
    const bool col_ok = L.w_col < (uint32_t)w.cols;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t n = kt * BK + L.w_row + i;
      const bool ok = col_ok && n < (uint32_t)w.rows;
      R.cw[i] = ld32(rc, oob_unless(ok, n * L.row_bytes + L.w_col / 2));
      const uint32_t b = n * L.row_blocks + (L.w_col >> bsh);
      if constexpr (DQ) {
        R.sq[i] = ld8(rq, oob_unless(ok, b));
        R.sf[i] = __uint_as_float(ld32(rs, oob_unless(ok, (b >> gsh) * 4)));
      } else {
        R.sf[i] = __uint_as_float(ld32(rq, oob_unless(ok, b * 4)));
      }
    }
  }
}

// Level lookup: a = 4 * code (byte address into the 16-word table).
__device__ __forceinline__ float lv_at(const char* lds, uint32_t a) {
  return *(const float*)(lds + LV_OFF + a);
}

// The NF4 decode of one quarter (16 weights per lane) runs in two halves so that
// the level lookups of quarter q + 1 are in flight while quarter q finishes:
//   lookup: 16 reads of the level table (byte address = 4 * code);
//   finish: fl32(level * scale) -> compute dtype -> 2 chunks into the W tile.
template <int MODE>
__device__ __forceinline__ void lookup_quarter(const CodeRegs& R, const char* lds, int qtr, float (&lv)[16]) {
  if constexpr (MODE == MODE_FWD) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t word = R.c[qtr >> 1][2 * (qtr & 1) + d];
      const uint32_t hi4 = (word >> 2) & 0x3c3c3c3cu;  // 4 * high nibble of each byte
      const uint32_t lo4 = (word << 2) & 0x3c3c3c3cu;  // 4 * low nibble of each byte
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // byte e: element 2e in the high nibble, 2e + 1 in the low one
        lv[8 * d + 2 * e] = lv_at(lds, (hi4 >> (8 * e)) & 0xffu);
        lv[8 * d + 2 * e + 1] = lv_at(lds, (lo4 >> (8 * e)) & 0xffu);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * qtr + u;  // column of the 8 x 8 block
      const uint32_t sh = 8 * (j >> 1) + ((j & 1) ? 0 : 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) lv[8 * u + i] = lv_at(lds, ((R.cw[i] >> sh) & 15u) * 4);
    }
  }
}

template <int CD, int MODE, int DQ>
__device__ __forceinline__ void finish_quarter(const CodeRegs& R, const float (&lv)[16], char* Bs, int tid,
                                               int qtr) {
  if constexpr (MODE == MODE_FWD) {
    const float s = scale_of<DQ>(R, qtr >> 1);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      u32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack2<CD>(fl32_mul(lv[8 * d + 2 * e], s), fl32_mul(lv[8 * d + 2 * e + 1], s));
      *(u32x4_t*)(Bs + chunk_addr(tid, 2 * qtr + d)) = o;
    }
  } else {
    const int ng = tid & 7, kg = tid >> 3;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * qtr + u;
      u32x4_t o;
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2)
        o[p2] = pack2<CD>(fl32_mul(lv[8 * u + 2 * p2], scale_of<DQ>(R, 2 * p2)),
                          fl32_mul(lv[8 * u + 2 * p2 + 1], scale_of<DQ>(R, 2 * p2 + 1)));
      *(u32x4_t*)(Bs + chunk_addr(kg * 8 + j, ng)) = o;
    }
  }
}

template <int CD, int MODE, int DQ>
__device__ __forceinline__ void decode_quarter(const CodeRegs& R, const char* lds, char* Bs, int tid, int qtr) {
  float lv[16];
  lookup_quarter<MODE>(R, lds, qtr, lv);
  finish_quarter<CD, MODE, DQ>(R, lv, Bs, tid, qtr);
}

// s_waitcnt vmcnt(n) (expcnt / lgkmcnt left alone).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Number of vector loads fetch_w issues (they follow the activation DMA of a stage).
template <int MODE, int DQ>
constexpr int fetch_w_loads() {
  return MODE == MODE_FWD ? (DQ ? 6 : 4) : (DQ ? 24 : 16);
}

template <int CD>
__device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (CD == CD_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

struct Frags {
  u32x4_t a[4], b[4];
};

// Fragments of 16-element step ks: lane (row l % 32, half l / 32) reads logical
// chunk 2 ks + half of rows wm + 32 i + l % 32 (A) and wn + 32 j + l % 32 (B).
__device__ __forceinline__ void read_frags(Frags& F, const char* As, const char* Bs, int a_row, int b_row,
                                           int xr, int h, int ks) {
  const int cphys = ((2 * ks + h) ^ xr) << 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) F.a[i] = *(const u32x4_t*)(As + (a_row + 32 * i) * ROWB + cphys);
#pragma unroll
  for (int j = 0; j < 4; ++j) F.b[j] = *(const u32x4_t*)(Bs + (b_row + 32 * j) * ROWB + cphys);
}

template <int CD>
__device__ __forceinline__ void mfma16(f32x16_t (&acc)[4][4], const Frags& F) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mfma<CD>(F.a[i], F.b[j], acc[i][j]);
}

// Interleave hints: after each MFMA, a few VALU / LDS instructions of the decode.
__device__ __forceinline__ void interleave_hints() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // 3 VALU
  }
  __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);    // the 2 LDS writes
}

// One stage: 64 MFMAs from LDS buffer `cur`; meanwhile the NF4 codes of the next
// stage (registers R) are decoded into the other buffer, a quarter per step.
template <int CD, int MODE, int DQ>
__device__ __forceinline__ void stage(f32x16_t (&acc)[4][4], char* lds, int cur, const CodeRegs& R, int a_row,
                                      int b_row, int xr, int h, int tid) {
  char* As = lds + cur * TILE_BYTES;
  char* Bs = lds + (2 + cur) * TILE_BYTES;
  char* Bn = lds + (2 + (cur ^ 1)) * TILE_BYTES;
  Frags F[2];
  float lv[2][16];
  read_frags(F[0], As, Bs, a_row, b_row, xr, h, 0);
  lookup_quarter<MODE>(R, lds, 0, lv[0]);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks < 3) {
      read_frags(F[(ks + 1) & 1], As, Bs, a_row, b_row, xr, h, ks + 1);
      lookup_quarter<MODE>(R, lds, ks + 1, lv[(ks + 1) & 1]);
    }
    mfma16<CD>(acc, F[ks & 1]);
    finish_quarter<CD, MODE, DQ>(R, lv[ks & 1], Bn, tid, ks);
    interleave_hints();
  }
}

template <int CD, int MODE, int DQ>
__global__ __launch_bounds__(kThreads, 1) void k_fused256(Big p, Nf4Tables tab) {
  // [A0 | A1 | B0 | B1 | levels]
  __shared__ __attribute__((aligned(1024))) char lds[4 * TILE_BYTES + 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 16) *(float*)(lds + LV_OFF + 4 * tid) = tab.lv[tid];
  int tm, tn;
  tile_of(p, tm, tn);
  const int64_t m0 = (int64_t)tm * TILE, n0 = (int64_t)tn * TILE;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const int h = lane >> 5;
  const int a_row = wm + (lane & 31), b_row = wn + (lane & 31);
  const int xr = swz(lane & 31);  // swizzle of every row this lane reads (rows differ by 32)

  const Nf4W& w = p.w;
  const rsrc_t ra = make_rsrc(p.a1, p.M * p.ld_a1 * 2);
  const rsrc_t rc = make_rsrc(w.codes, w.rows * w.cols / 2);
  const int64_t nb = w.rows * w.cols / w.bs;
  const rsrc_t rq = DQ ? make_rsrc(w.absmax_q, nb) : make_rsrc(w.absmax, nb * 4);
  const rsrc_t rs = make_rsrc(DQ ? (const void*)w.scale2 : (const void*)w.absmax,
                              DQ ? ((nb + w.g - 1) / w.g) * 4 : nb * 4);

  Lane L;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 8 * (4 * i + wave) + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    L.a_col[i] = 8 * c;
    L.a_off[i] = (uint32_t)(((m0 + row) * p.ld_a1 + 8 * c) * 2);
  }
  L.row_bytes = (uint32_t)(w.cols / 2);
  L.row_blocks = (uint32_t)(w.cols >> w.bs_shift);
  if constexpr (MODE == MODE_FWD) {
    L.w_row = (uint32_t)(n0 + tid);
    L.w_col = 0;
  } else {
    L.w_row = (uint32_t)((tid & 7) * 8);
    L.w_col = (uint32_t)(n0 + (tid >> 3) * 8);
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const uint32_t KT = (uint32_t)((p.K1 + BK - 1) / BK);
  CodeRegs R0, R1;
  fetch_a<MODE>(p, L, ra, lds, wave, 0);
  fetch_w<MODE, DQ>(R0, p, L, rc, rq, rs, 0);
  fetch_w<MODE, DQ>(R1, p, L, rc, rq, rs, 1);
  __syncthreads();  // level table
#pragma unroll
  for (int q = 0; q < 4; ++q) decode_quarter<CD, MODE, DQ>(R0, lds, lds + 2 * TILE_BYTES, tid, q);
  fetch_w<MODE, DQ>(R0, p, L, rc, rq, rs, 2);
  wait_vmcnt<fetch_w_loads<MODE, DQ>()>();  // the activation tile of stage 0 has landed in LDS
  __syncthreads();

  // Stage kt reads buffer kt % 2, prefetches the activations of stage kt + 1 into
  // the other buffer and decodes its codes (fetched two stages ahead) there.
  uint32_t kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    fetch_a<MODE>(p, L, ra, lds + TILE_BYTES, wave, kt + 1);
    stage<CD, MODE, DQ>(acc, lds, 0, R1, a_row, b_row, xr, h, tid);
    fetch_w<MODE, DQ>(R1, p, L, rc, rq, rs, kt + 3);
    wait_vmcnt<fetch_w_loads<MODE, DQ>()>();  // this stage's activation DMA has landed
    __syncthreads();
    fetch_a<MODE>(p, L, ra, lds, wave, kt + 2);
    stage<CD, MODE, DQ>(acc, lds, 1, R0, a_row, b_row, xr, h, tid);
    fetch_w<MODE, DQ>(R0, p, L, rc, rq, rs, kt + 4);
    wait_vmcnt<fetch_w_loads<MODE, DQ>()>();
    __syncthreads();
  }
  if (kt < KT) {
    stage<CD, MODE, DQ>(acc, lds, 0, R1, a_row, b_row, xr, h, tid);
    __syncthreads();
  }

  // LoRA segment: r_pad more contraction steps with [T | B] (fwd) or [dT | A] (dX).
  char* As0 = lds;
  char* Bs0 = lds + 2 * TILE_BYTES;
  for (int64_t k = 0; k < p.r_pad; k += BK) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + kThreads * i;
      const int row = q >> 3, c = q & 7;
      const int64_t grow = m0 + row, col = k + c * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (grow < p.M && col < p.r_pad) v = *(const u32x4_t*)((const uint16_t*)p.a2 + grow * p.r_pad + col);
      *(u32x4_t*)(As0 + chunk_addr(row, c)) = v;
    }
    if constexpr (MODE == MODE_FWD) {
      // lora_b rows [n][t] as they are
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = tid + kThreads * i;
        const int row = q >> 3, c = q & 7;
        const int64_t grow = n0 + row, col = k + c * 8;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (grow < p.NB) {
          const uint16_t* src = (const uint16_t*)p.b2 + grow * p.r + col;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col + e < p.r) v[e >> 1] |= (uint32_t)src[e] << ((e & 1) * 16);
        }
        *(u32x4_t*)(Bs0 + chunk_addr(row, c)) = v;
      }
    } else {
      // lora_a [t][k] staged as [k][t]: one 8 x 8 block per lane, transposed with permutes
      const int tg = tid & 7, kg = tid >> 3;
      u32x4_t in[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t t = k + tg * 8 + i, col = n0 + kg * 8;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (t < p.r) {
          const uint16_t* src = (const uint16_t*)p.b2 + t * p.NB + col;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col + e < p.NB) v[e >> 1] |= (uint32_t)src[e] << ((e & 1) * 16);
        }
        in[i] = v;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x4_t o;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) o[q2] = __builtin_amdgcn_perm(in[2 * q2 + 1][j >> 1], in[2 * q2][j >> 1], sel);
        *(u32x4_t*)(Bs0 + chunk_addr(kg * 8 + j, tg)) = o;
      }
    }
    __syncthreads();
    Frags F;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      read_frags(F, As0, Bs0, a_row, b_row, xr, h, ks);
      mfma16<CD>(acc, F);
    }
    __syncthreads();
  }

  // Epilogue: fp32 accumulators (+ bias) -> compute dtype.
  const int cl = lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t col = n0 + wn + 32 * j + cl;
    if (col >= p.NB) continue;
    const float bias = p.bias ? load_cd<CD>(p.bias, col) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row < p.M) store_cd<CD>(p.out, row * p.NB + col, acc[i][j][v] + bias);
      }
  }
}

template <int CD, int MODE>
int run(const Big& b, hipStream_t s, int kind) {
  const int64_t tiles = (int64_t)b.tiles_m * b.tiles_n;
  ProfScope prof(kind, s);
  if (b.w.dq)
    k_fused256<CD, MODE, 1><<<dim3((unsigned)tiles), dim3(kThreads), 0, s>>>(b, host_tables());
  else
    k_fused256<CD, MODE, 0><<<dim3((unsigned)tiles), dim3(kThreads), 0, s>>>(b, host_tables());
  return check_launch(MODE == MODE_FWD ? "k_fused256<fwd>" : "k_fused256<dx>");
}

bool fits_buffers(const LayerCall& c, int64_t a1_bytes) {
  const int64_t lim = 0x7fff0000LL;
  const int64_t nb = c.w.rows * c.w.cols / c.w.bs;
  return a1_bytes < lim && c.w.rows * c.w.cols / 2 < lim && nb * 4 < lim;
}

}  // namespace

// Whether the 256-tile kernels take this layer (else the generic tile engine does).
bool fused256_ok(const LayerCall& c, bool dx) {
  if (c.cd != CD_BF16 && c.cd != CD_F16) return false;
  if (c.w.bs_shift < 0 || (c.w.dq && c.w.g_shift < 0)) return false;
  if (dx) return (c.w.rows % 8 == 0) && fits_buffers(c, c.m * c.w.rows * 2);
  return fits_buffers(c, c.m * c.w.cols * 2);
}

// y = [x | T][W~ | B]^T + bias.  t_cd: [m, r_pad] compute-dtype s x A^T.
int fused256_forward(const LayerCall& c, const void* t_cd, int64_t r_pad, void* y) {
  Big b = {};
  b.a1 = c.x;
  b.ld_a1 = c.w.cols;
  b.a2 = t_cd;
  b.r_pad = r_pad;
  b.b2 = c.lora_b;
  b.w = c.w;
  b.M = c.m;
  b.NB = c.w.rows;
  b.K1 = c.w.cols;
  b.r = c.r;
  b.tiles_m = (int32_t)ceil_div(c.m, TILE);
  b.tiles_n = (int32_t)ceil_div(c.w.rows, TILE);
  b.out = y;
  b.bias = c.bias;
  if (c.cd == CD_BF16) return run<CD_BF16, MODE_FWD>(b, c.stream, QLORA_K_FWD_GEMM);
  return run<CD_F16, MODE_FWD>(b, c.stream, QLORA_K_FWD_GEMM);
}

// dX = [dY | dT][W~ ; A].  dt_cd: [m, r_pad] compute-dtype s dY B.
int fused256_dx(const LayerCall& c, const void* dy, const void* dt_cd, int64_t r_pad, void* dx) {
  Big b = {};
  b.a1 = dy;
  b.ld_a1 = c.w.rows;
  b.a2 = dt_cd;
  b.r_pad = r_pad;
  b.b2 = c.lora_a;
  b.w = c.w;
  b.M = c.m;
  b.NB = c.w.cols;
  b.K1 = c.w.rows;
  b.r = c.r;
  b.tiles_m = (int32_t)ceil_div(c.m, TILE);
  b.tiles_n = (int32_t)ceil_div(c.w.cols, TILE);
  b.out = dx;
  b.bias = nullptr;
  if (c.cd == CD_BF16) return run<CD_BF16, MODE_DX>(b, c.stream, QLORA_K_BWD_DX);
  return run<CD_F16, MODE_DX>(b, c.stream, QLORA_K_BWD_DX);
}

}  // namespace qnf4
