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
// (XOR-swizzled 16-byte chunks), double buffered (4 x 32 KiB).
//
// Pipeline of stage k (one wave per SIMD, so all latency hiding is explicit and
// the side work is placed between the MFMAs in program order):
//   * one barrier per stage; before it each wave waits only for its own copy of
//     stage k's activations and its LDS writes, never for later prefetches;
//   * sub-step 0 issues the activation copy of stage k+1 (buffer_load ... lds,
//     global -> LDS with no register round trip; each row of a stage is one whole
//     128-byte line), spread over the MFMAs;
//   * sub-step 1 issues the loads of the NF4 codes (and block scales) of stage
//     k+2 into registers: they have more than a stage to arrive;
//   * all four sub-steps decode a quarter of the codes of stage k+1 into the
//     other W buffer and read the fragments of the next sub-step.
//
// NF4 decode (the method's dequantization, exact): code c -> fl32(L[c] * s_b) ->
// compute dtype; L sits in LDS (16 words in 16 banks: conflict-free lookups).
//   forward: lane t owns row t of the W tile: 64 codes (32 bytes) per stage;
//   dX:      the contraction runs over W's rows, so a lane decodes an 8 x 8 block
//            (8 rows x one 32-bit word of codes) and packs pairs from adjacent
//            rows, writing 16-byte runs of the transposed tile [k][n].
// The workgroup -> tile map gives each XCD (workgroups b, b + 8, ... share one) a
// compact block of tiles, so their common operand tiles stay in that XCD's L2.
//
// The dense kernel (dequantize-then-GEMM: W~ already in the compute dtype) copies
// both operands by DMA and runs 8 waves of 128 x 64 (two per SIMD, 185 registers
// each) with waves 0..3 issuing the copies; a forward whose rank is not a multiple
// of 8 takes the 4-wave form, whose low-rank tail is the fused kernel's code.  An
// incomplete last round of tiles is cut into contraction slices whose fp32 partial
// sums k_split_sum adds (both kernels).
#include <algorithm>

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
  // Dense kernel only: workgroups [0, full) take whole tiles; the next rem * split
  // take one contraction slice each of the tiles full .. full + rem - 1 (an
  // incomplete last round) and leave fp32 partial sums for k_split_sum.
  int32_t full, rem, split;
  float* part;        // [rem][split][kTileAcc] fp32, in accumulator order
  // Dense kernel only: the low-rank tail as pipelined stages when b2_rows is set:
  // the W-side tail operand as rows [NB][ld_b2] (fwd: lora_b, ld r; dX: A^T
  // [K][r_pad]); the r_b2 valid columns of a row (r fwd, r_pad dX; a multiple of 8).
  const void* b2_rows;
  int64_t ld_b2;
  int32_t r_b2;
};
constexpr int kTileAcc = TILE * TILE;  // accumulators of one tile

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, kRsrcWord3);
}
// Buffer loads: byte offset = voff (per lane) + soff (wave-uniform).  Every part
// that can fall outside a buffer stays in voff, which alone decides the range
// check; soff only carries offsets that are in bounds by construction.
__device__ __forceinline__ u32x4_t ld128(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t ld8(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
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

// Workgroup -> output tile.  Workgroups b, b + 8, ... run on the same XCD, so
// each XCD takes a contiguous chunk of T / 8 tiles of a grouped order: groups of
// kGroupM tile rows, column-major inside a group.  An XCD then holds a compact
// block (4 x 8 tiles for a 16 x 16 grid) and its L2 sees fewer distinct operand
// tiles per stage than with whole tile rows.
constexpr int kGroupM = 4;
// Position of workgroup b among n consecutive ones when each XCD takes a
// contiguous chunk of n / 8 positions.
__device__ __forceinline__ int xcd_chunk(int b, int n) { return (n & 7) == 0 ? (b & 7) * (n >> 3) + (b >> 3) : b; }
// Tile t of the grouped order.
__device__ __forceinline__ void grouped_tile(const Big& p, int t, int& tm, int& tn) {
  const int per = kGroupM * p.tiles_n, g = t / per, u = t % per;
  const int gm = min(kGroupM, p.tiles_m - g * kGroupM);
  tm = g * kGroupM + u % gm;
  tn = u / gm;
}
__device__ __forceinline__ void tile_of(const Big& p, int& tm, int& tn) {
  grouped_tile(p, xcd_chunk(blockIdx.x, p.tiles_m * p.tiles_n), tm, tn);
}
// Dense kernel: workgroup -> (tile, contraction slice, index among the cut tiles
// or -1).  The slices of the cut tiles follow the whole tiles; each XCD's chunk of
// them is one slice of a run of consecutive tiles of the grouped order.
__device__ __forceinline__ void item_of(const Big& p, int b, int& tm, int& tn, int& slice, int& rt) {
  slice = 0;
  rt = -1;
  if (b < p.full) {
    grouped_tile(p, xcd_chunk(b, p.full), tm, tn);
    return;
  }
  const int u = xcd_chunk(b - p.full, p.rem * p.split);
  slice = u / p.rem;
  rt = u - slice * p.rem;
  grouped_tile(p, p.full + rt, tm, tn);
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
// Out-of-range lanes have the top bit set (oob_unless) so that their loads
// return zeros; the per-stage parts are wave-uniform and go in soffset.
struct Lane {
  uint32_t a_off;        // activation: global byte offset of the first chunk this lane copies
  uint32_t a_step;       // bytes between its 8 chunks (32 rows apart)
  uint32_t c_off;        // codes: fwd, start of W row n0 + tid; dX, W row (tid % 8) * 8 of
                         //   the stage, column n0 + (tid / 8) * 8
  uint32_t b_idx;        // block index of the same place (fwd: row start; dX: its column block)
  bool ok;               // fwd: the W row exists; dX: the W columns exist
  uint32_t row_bytes;    // bytes of codes per W row (cols / 2)
  uint32_t row_blocks;   // blocks per W row (cols / block_size)
};

// Activation tile of stage kt straight from global memory into LDS buffer `dst`:
// instruction i of wave w fills rows 8 (4 i + w) .. +8; lane l lands in physical
// chunk l % 8 of row l / 8 and so fetches the logical chunk that maps there.
template <int MODE>
__device__ __forceinline__ void fetch_a1(const Big& p, const Lane& L, rsrc_t ra, char* dst, int wave, uint32_t kt,
                                         int i) {
  // The contraction is a whole number of stages (K for the forward: a multiple of
  // 64 by the layer's contract; N for dX: required by fused256_ok), so no column
  // check; rows past M read past the buffer and land as zeros.
  __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dst + (4 * i + wave) * 1024), 16,
                                           (int)(L.a_off + i * L.a_step), (int)(kt * (BK * 2)), 0, 0);
}
template <int MODE>
__device__ __forceinline__ void fetch_a(const Big& p, const Lane& L, rsrc_t ra, char* dst, int wave, uint32_t kt) {
#pragma unroll
  for (int i = 0; i < 8; ++i) fetch_a1<MODE>(p, L, ra, dst, wave, kt, i);
}

// Codes of stage kt.  Stages past the last (the prefetch runs two ahead) load
// the last stage again: the stage offsets travel in soffset and must stay inside
// the buffers.
template <int MODE, int DQ>
__device__ __forceinline__ void fetch_w(CodeRegs& R, const Big& p, const Lane& L, rsrc_t rc, rsrc_t rq,
                                        rsrc_t rs, uint32_t kt, uint32_t KT) {
  if (kt >= KT) kt = KT - 1;
  const Nf4W& w = p.w;
  const uint32_t bsh = (uint32_t)w.bs_shift, gsh = (uint32_t)w.g_shift;
  const uint32_t cv = oob_unless(L.ok, L.c_off);
  if constexpr (MODE == MODE_FWD) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t col = kt * BK + 32 * j;  // both 32-code halves lie in one block (bs >= 32)
      R.c[j] = ld128(rc, cv, col / 2);
      const uint32_t bu = col >> bsh;
      if constexpr (DQ) {
        R.sq[j] = ld8(rq, oob_unless(L.ok, L.b_idx), bu);
        R.sf[j] = __uint_as_float(ld32(rs, oob_unless(L.ok, ((L.b_idx + bu) >> gsh) * 4)));
      } else {
        R.sf[j] = __uint_as_float(ld32(rq, oob_unless(L.ok, L.b_idx * 4), bu * 4));
      }
    }
  } else {
    // W rows kt * 64 + (tid % 8) * 8 + i exist: the fused dX path takes W only
    // when its row count is a multiple of 64.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t nu = kt * BK + i;  // uniform part of the row index
      R.cw[i] = ld32(rc, cv, nu * L.row_bytes);
      if constexpr (DQ) {
        R.sq[i] = ld8(rq, oob_unless(L.ok, L.b_idx), nu * L.row_blocks);
        R.sf[i] = __uint_as_float(ld32(rs, oob_unless(L.ok, ((L.b_idx + nu * L.row_blocks) >> gsh) * 4)));
      } else {
        R.sf[i] = __uint_as_float(ld32(rq, oob_unless(L.ok, L.b_idx * 4), nu * L.row_blocks * 4));
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
        lv[8 * d + 2 * e] = lv_at(lds, byte_of(hi4, e));
        lv[8 * d + 2 * e + 1] = lv_at(lds, byte_of(lo4, e));
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

// The block scales of the lane's codes for one stage: fwd 2 (one per 32-code
// half), dX 8 (one per W row).
template <int MODE, int DQ>
__device__ __forceinline__ void stage_scales(const CodeRegs& R, float (&sc)[8]) {
#pragma unroll
  for (int i = 0; i < (MODE == MODE_FWD ? 2 : 8); ++i) {
    sc[i] = scale_of<DQ>(R, i);
    asm volatile("" : "+v"(sc[i]));  // a register of its own: the loaded set dies here
  }
}

template <int CD, int MODE>
__device__ __forceinline__ void finish_quarter(const float (&sc)[8], const float (&lv)[16], char* Bs, int tid,
                                               int qtr) {
  if constexpr (MODE == MODE_FWD) {
    const float s = sc[qtr >> 1];
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
        o[p2] = pack2<CD>(fl32_mul(lv[8 * u + 2 * p2], sc[2 * p2]), fl32_mul(lv[8 * u + 2 * p2 + 1], sc[2 * p2 + 1]));
      *(u32x4_t*)(Bs + chunk_addr(kg * 8 + j, ng)) = o;
    }
  }
}

template <int CD, int MODE, int DQ>
__device__ __forceinline__ void decode_quarter(const CodeRegs& R, const char* lds, char* Bs, int tid, int qtr) {
  float lv[16], sc[8];
  stage_scales<MODE, DQ>(R, sc);
  lookup_quarter<MODE>(R, lds, qtr, lv);
  finish_quarter<CD, MODE>(sc, lv, Bs, tid, qtr);
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

// A fragments of the wave's four 32-row blocks, B fragments of its JB 32-column blocks.
template <int JB>
struct FragsT {
  u32x4_t a[4], b[JB];
};
using Frags = FragsT<4>;

// Fragments of 16-element step ks: lane (row l % 32, half l / 32) reads logical
// chunk 2 ks + half of rows wm + 32 i + l % 32 (A) and wn + 32 j + l % 32 (B).
template <int JB>
__device__ __forceinline__ void read_frags(FragsT<JB>& F, const char* As, const char* Bs, int a_row, int b_row,
                                           int xr, int h, int ks) {
  const int cphys = ((2 * ks + h) ^ xr) << 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) F.a[i] = *(const u32x4_t*)(As + (a_row + 32 * i) * ROWB + cphys);
#pragma unroll
  for (int j = 0; j < JB; ++j) F.b[j] = *(const u32x4_t*)(Bs + (b_row + 32 * j) * ROWB + cphys);
}

// SWAP: the W-side fragment goes in as the MFMA's row operand, so block (i, j) is
// accumulated transposed (lane % 32 indexes the activation row; the 16 values of a
// lane are W-side columns).  The dense kernel works this way round.
template <int CD, bool SWAP>
__device__ __forceinline__ void mfma16(f32x16_t (&acc)[4][4], const Frags& F) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = SWAP ? mfma<CD>(F.b[j], F.a[i], acc[i][j]) : mfma<CD>(F.a[i], F.b[j], acc[i][j]);
}

// s_waitcnt lgkmcnt(0) alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0x3f | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier with no implied waits: the callers wait for exactly what the
// other waves will read (their own copies and LDS writes of the stage).  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Byte address (4 * code) of element e (0..15) of decode quarter q of the lane's
// codes: fwd, element 16 q + e of its W row (high nibble first within a byte);
// dX, row e % 8 of its 8 x 8 block, column 2 q + e / 8.
template <int MODE>
__device__ __forceinline__ uint32_t code_addr(const CodeRegs& R, int q, int e) {
  if constexpr (MODE == MODE_FWD) {
    const uint32_t word = R.c[q >> 1][2 * (q & 1) + (e >> 3)];
    const int byte = (e & 7) >> 1;
    return (word >> (8 * byte + ((e & 1) ? 0 : 4)) << 2) & 0x3cu;
  } else {
    const int j = 2 * q + (e >> 3);
    const uint32_t sh = 8 * (j >> 1) + ((j & 1) ? 0 : 4);
    return ((R.cw[e & 7] >> sh) << 2) & 0x3cu;
  }
}

// Part t (0..7) of finishing quarter q: two weights fl32(level * scale) packed into
// one word of the 16-byte chunk being assembled; parts 3 and 7 write a chunk.
template <int CD, int MODE>
__device__ __forceinline__ void finish_part(const float (&sc)[8], const float (&lv)[16], u32x4_t& o, char* Bs,
                                            int tid, int q, int t) {
  const int d = t >> 2, e = t & 3;  // chunk d of the quarter, word e of it
  if constexpr (MODE == MODE_FWD) {
    const float s = sc[q >> 1];
    o[e] = pack2<CD>(fl32_mul(lv[8 * d + 2 * e], s), fl32_mul(lv[8 * d + 2 * e + 1], s));
    if (e == 3) *(u32x4_t*)(Bs + chunk_addr(tid, 2 * q + d)) = o;
  } else {
    o[e] = pack2<CD>(fl32_mul(lv[8 * d + 2 * e], sc[2 * e]), fl32_mul(lv[8 * d + 2 * e + 1], sc[2 * e + 1]));
    if (e == 3) *(u32x4_t*)(Bs + chunk_addr((tid >> 3) * 8 + 2 * q + d, tid & 7)) = o;
  }
}

// The r-th fragment read of a sub-step, in the order the next sub-step's MFMAs
// (block (i, j) at slot i JB + j) first use them: 0..3 the A fragments a[i], 4.. the
// B fragments b[j].  JB = 2: b0 a0 b1 a1 a2 a3; JB = 4: a0 b0 b1 b2 b3 a1 a2 a3.
template <int JB>
__device__ __forceinline__ constexpr int frag_by_first_use(int r) {
  if constexpr (JB == 2) {
    constexpr int o[6] = {4, 0, 5, 1, 2, 3};
    return o[r];
  } else {
    constexpr int o[8] = {0, 4, 5, 6, 7, 1, 2, 3};
    return o[r];
  }
}

// One stage: 64 MFMAs from LDS buffer `cur`, in 4 sub-steps of 16.  The side work
// sits at fixed MFMA slots (fences keep the compiler from regrouping it):
//   every other slot: one fragment read for the next sub-step (in order of first use);
//   every slot: one level lookup for the next decode quarter (in sub-step 3, for
//     quarter 0 of the next stage, from Rn);
//   slots 8..15: one pack of the current quarter (lookups issued a sub-step ago),
//     its two chunk writes into the other W buffer;
//   odd slots of sub-step 0: one instruction of the activation copy of stage kn.
// lv[0] holds the lookups of quarter 0 on entry (and of the next stage's
// quarter 0 on exit).
template <int CD, int MODE, int DQ>
__device__ __forceinline__ void stage(f32x16_t (&acc)[4][4], char* lds, int cur, const CodeRegs& R,
                                      const CodeRegs& Rn, float (&lv)[2][16], const Big& p, const Lane& L, rsrc_t ra,
                                      int wave, uint32_t kn, bool do_a, int a_row, int b_row, int xr, int h, int tid) {
  char* As = lds + cur * TILE_BYTES;
  char* Bs = lds + (2 + cur) * TILE_BYTES;
  char* An = lds + (cur ^ 1) * TILE_BYTES;
  char* Bn = lds + (2 + (cur ^ 1)) * TILE_BYTES;
  Frags F[2];
  float sc[8];
  stage_scales<MODE, DQ>(R, sc);
  read_frags(F[0], As, Bs, a_row, b_row, xr, h, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    Frags& C = F[ks & 1];
    Frags& N = F[(ks + 1) & 1];
    float (&lc)[16] = lv[ks & 1];
    float (&ln)[16] = lv[(ks + 1) & 1];
    const int cphys = ((2 * (ks + 1) + h) ^ xr) << 4;
    u32x4_t o;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int i = t >> 2, j = t & 3;
      acc[i][j] = mfma<CD>(C.b[j], C.a[i], acc[i][j]);  // block (i, j) transposed
      if (ks < 3 && (t & 1) == 0) {
        const int f = frag_by_first_use<4>(t >> 1);
        if (f < 4) N.a[f] = *(const u32x4_t*)(As + (a_row + 32 * f) * ROWB + cphys);
        else N.b[f - 4] = *(const u32x4_t*)(Bs + (b_row + 32 * (f - 4)) * ROWB + cphys);
      }
      if (ks < 3) ln[t] = lv_at(lds, code_addr<MODE>(R, ks + 1, t));
      else ln[t] = lv_at(lds, code_addr<MODE>(Rn, 0, t));
      if (t >= 8) finish_part<CD, MODE>(sc, lc, o, Bn, tid, ks, t - 8);
      if (ks == 0 && (t & 1) == 1 && do_a) fetch_a1<MODE>(p, L, ra, An, wave, kn, t >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// LoRA segment: r_pad more contraction steps with [T | B] (fwd) or [dT | A] (dX),
// appended to the main contraction in the same accumulators.  Entered with every
// copy drained and the LDS free.
template <int CD, int MODE, bool SWAP>
__device__ __forceinline__ void lora_segment(f32x16_t (&acc)[4][4], char* lds, const Big& p, int64_t m0, int64_t n0,
                                             int tid, int wave, int lane, int a_row, int b_row, int xr, int h) {
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
      mfma16<CD, SWAP>(acc, F);
    }
    __syncthreads();
  }

}


__device__ __forceinline__ f32x4_t acc4(const f32x16_t& a, int q) {
  f32x4_t v = {a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
  return v;
}

// Partial sums of a cut tile's slice, fp32 [256][256] row-major: the wave's
// (transposed) block (i, j) gives row wm + 32 i + lane % 32 the four columns
// wn + 32 j + 8 q + 4 (lane / 32) .. + 3 from elements 4 q .. 4 q + 3 (one 16-byte
// store; lanes l and l + 32 fill 32 contiguous bytes of a row).  Rows from
// `rows` on (past the last token) are not stored: the slice sum skips them.
template <int JB>
__device__ __forceinline__ void store_partial(const f32x16_t (&acc)[4][JB], float* dst, int wm, int wn, int lane,
                                              int64_t rows) {
  const rsrc_t r = make_rsrc(dst, kTileAcc * 4);
  const uint32_t base = (uint32_t)(((wm + (lane & 31)) * TILE + wn + 4 * (lane >> 5)) * 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t off = oob_unless(wm + 32 * i + (lane & 31) < rows, base);
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc4(acc[i][j], q)), r, (int)off,
                                               (32 * i * TILE + 32 * j + 8 * q) * 4, 0);
  }
}

// The cut tiles' outputs: thread (b, t) of cut tile rt sums the four columns
// 4 (256 b + t) % 256 .. + 3 of tile row (256 b + t) / 64 over the slices in slice
// order, adds the bias and writes the compute dtype (a wave covers one whole tile
// row: 512 contiguous bytes).
template <int CD, int S>
__global__ __launch_bounds__(kThreads) void k_split_sum(Big p) {
  const int rt = blockIdx.y;
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  int tm, tn;
  grouped_tile(p, p.full + rt, tm, tn);
  const int64_t row = (int64_t)tm * TILE + (4 * idx) / TILE;
  const int64_t col = (int64_t)tn * TILE + (4 * idx) % TILE;
  if (row >= p.M) return;  // a row past the last token (its partial sums were not stored)
  const float* src = p.part + (size_t)rt * S * kTileAcc + 4 * idx;
  f32x4_t v[S];  // the partial sums are dead after this read, the output is not read again: both non-temporal
#pragma unroll
  for (int s = 0; s < S; ++s) v[s] = __builtin_nontemporal_load((const f32x4_t*)(src + (size_t)s * kTileAcc));
  f32x4_t t = v[0];
#pragma unroll
  for (int s = 1; s < S; ++s) t = t + v[s];
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = t[e] + (p.bias ? load_cd<CD>(p.bias, col + e < p.NB ? col + e : 0) : 0.f);
  uint16_t* dst = (uint16_t*)p.out + row * p.NB + col;
  if ((p.NB & 3) == 0 && col + 4 <= p.NB) {
    const u32x2_t w2 = {pack2<CD>(o[0], o[1]), pack2<CD>(o[2], o[3])};
    __builtin_nontemporal_store(w2, (u32x2_t*)dst);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col + e < p.NB) store_cd<CD>(p.out, row * p.NB + col + e, o[e]);
  }
}

// Epilogue of the 256-tile kernels, whose blocks are accumulated transposed: lane
// (r = lane % 32, h = lane / 32) of block (i, j) holds output row 32 i + r, columns
// 32 j + 8 q + 4 h + e in element 4 q + e.  Each wave rounds its 128 x 32 JB block
// (+ bias) to the compute dtype in its own 8 JB KiB of LDS (rows of 64 JB bytes;
// 16-byte chunk c of row m at chunk c ^ (m % 4 JB), so neither the 8-byte writes nor
// the 16-byte row reads collide on banks), then writes whole rows: 4 JB lanes per
// row, 64 / (4 JB) rows of 64 JB contiguous bytes per store instruction.  Entered
// with the LDS free.
template <int CD, int JB, int I0, int NI>
__device__ __forceinline__ void epilogue_rows(const f32x16_t (&acc)[4][JB], const Big& p, char* W, int64_t m0,
                                              int64_t n0, int wm, int wn, int lane, int h) {
  // rows 32 I0 .. 32 (I0 + NI) of the wave's block, staged in W (row m - 32 I0); the
  // output rows go out with non-temporal stores (the layer's output is not read again
  // by these kernels, and leaving it out of the caches kept the next kernels' operands
  // there: training step 3.52-3.53 against 3.55-3.56 ms)
  constexpr int RB = 64 * JB;  // bytes per staged row
  constexpr int NC = 4 * JB;   // 16-byte chunks per row
  const int r = lane & 31;
  float bv[JB][4][4];  // bias of the lane's columns (j, q, e)
#pragma unroll
  for (int j = 0; j < JB; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[j][q][e] = 0.f;
  if (p.bias) {
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t col = n0 + wn + 32 * j + 8 * q + 4 * h + e;
          bv[j][q][e] = load_cd<CD>(p.bias, col < p.NB ? col : 0);
        }
  }
#pragma unroll
  for (int i = I0; i < I0 + NI; ++i) {
    const int m = 32 * (i - I0) + r;
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w2[2];
        w2[0] = pack2<CD>(acc[i][j][4 * q] + bv[j][q][0], acc[i][j][4 * q + 1] + bv[j][q][1]);
        w2[1] = pack2<CD>(acc[i][j][4 * q + 2] + bv[j][q][2], acc[i][j][4 * q + 3] + bv[j][q][3]);
        *(uint2*)(W + m * RB + (((4 * j + q) ^ (m & (NC - 1))) << 4) + 8 * h) = make_uint2(w2[0], w2[1]);
      }
  }
  wait_lgkm0();  // the wave reads back only what it wrote
  const int c = lane & (NC - 1);
  const int64_t col = n0 + wn + 8 * c;
  const bool vec = (p.NB & 7) == 0;
#pragma unroll 4
  for (int it = 0; it < NI * NC / 2; ++it) {
    const int m = (64 / NC) * it + lane / NC;
    const u32x4_t v = *(const u32x4_t*)(W + m * RB + ((c ^ (m & (NC - 1))) << 4));
    const int64_t row = m0 + wm + 32 * I0 + m;
    if (row >= p.M) continue;
    uint16_t* dst = (uint16_t*)p.out + row * p.NB + col;
    if (vec && col + 8 <= p.NB) {
      __builtin_nontemporal_store(v, (u32x4_t*)dst);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < p.NB) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  }
}

template <int CD, int JB>
__device__ __forceinline__ void epilogue_lds(const f32x16_t (&acc)[4][JB], const Big& p, char* lds, int64_t m0,
                                             int64_t n0, int wave, int wm, int wn, int lane, int h) {
  epilogue_rows<CD, JB, 0, 4>(acc, p, lds + wave * (128 * 64 * JB), m0, n0, wm, wn, lane, h);
}

// The same in two passes of 64 rows through 8 JB KiB per wave at W (the persistent
// dense kernel stages there while the next tile's first stage lands elsewhere).
template <int CD, int JB>
__device__ __forceinline__ void epilogue_halves(const f32x16_t (&acc)[4][JB], const Big& p, char* W, int64_t m0,
                                                int64_t n0, int wm, int wn, int lane, int h) {
  epilogue_rows<CD, JB, 0, 2>(acc, p, W, m0, n0, wm, wn, lane, h);
  wait_lgkm0();  // the first pass's reads are done before the second pass overwrites W
  epilogue_rows<CD, JB, 2, 2>(acc, p, W, m0, n0, wm, wn, lane, h);
}

template <int CD, int MODE, int DQ>
__global__ __launch_bounds__(kThreads, 1) void k_fused256(Big p, Nf4Tables tab) {
  // [A0 | A1 | B0 | B1 | levels]
  __shared__ __attribute__((aligned(1024))) char lds[4 * TILE_BYTES + 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the DMA bases scalar
  if (tid < 16) *(float*)(lds + LV_OFF + 4 * tid) = tab.lv[tid];
  int tm, tn, slice, rt;
  item_of(p, blockIdx.x, tm, tn, slice, rt);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  slice = __builtin_amdgcn_readfirstlane(slice);
  rt = __builtin_amdgcn_readfirstlane(rt);
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
                              DQ ? (((nb - 1) >> w.g_shift) + 1) * 4 : nb * 4);

  Lane L;
  {
    // rows 8 (4 i + wave) + lane / 8 for i = 0..7: their swizzle does not depend on i
    const int row = 8 * wave + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    L.a_off = (uint32_t)(((m0 + row) * p.ld_a1 + 8 * c) * 2);
    L.a_step = (uint32_t)(32 * p.ld_a1 * 2);
  }
  L.row_bytes = (uint32_t)(w.cols / 2);
  L.row_blocks = (uint32_t)(w.cols >> w.bs_shift);
  if constexpr (MODE == MODE_FWD) {
    const uint32_t row = (uint32_t)(n0 + tid);
    L.ok = row < (uint32_t)w.rows;
    L.c_off = row * L.row_bytes;
    L.b_idx = row * L.row_blocks;
  } else {
    const uint32_t row = (uint32_t)((tid & 7) * 8), col = (uint32_t)(n0 + (tid >> 3) * 8);
    L.ok = col < (uint32_t)w.cols;
    L.c_off = row * L.row_bytes + col / 2;
    L.b_idx = row * L.row_blocks + (col >> w.bs_shift);
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Stages [k0, k1) of the contraction: all of it for a whole tile, slice `slice`
  // of split for a cut one (the fetches take absolute stage indices; loads past
  // k1 - 1 repeat it).
  const uint32_t KT = (uint32_t)((p.K1 + BK - 1) / BK);
  uint32_t k0 = 0, k1 = KT;
  if (rt >= 0) {
    k0 = (uint32_t)slice * KT / (uint32_t)p.split;
    k1 = (uint32_t)(slice + 1) * KT / (uint32_t)p.split;
  }
  const uint32_t nst = k1 - k0;
  constexpr int NW = fetch_w_loads<MODE, DQ>();
  CodeRegs R0, R1;
  fetch_a<MODE>(p, L, ra, lds, wave, k0);
  fetch_w<MODE, DQ>(R0, p, L, rc, rq, rs, k0, k1);
  fetch_w<MODE, DQ>(R1, p, L, rc, rq, rs, k0 + 1, k1);
  __syncthreads();  // level table
#pragma unroll
  for (int q = 0; q < 4; ++q) decode_quarter<CD, MODE, DQ>(R0, lds, lds + 2 * TILE_BYTES, tid, q);
  fetch_w<MODE, DQ>(R0, p, L, rc, rq, rs, k0 + 2, k1);
  wait_vmcnt<NW>();  // the activation tile of stage 0 (and the codes of stage 1) have landed
  wait_lgkm0();
  barrier_only();

  // Stage kt computes from buffer kt % 2 while it copies the activations of
  // stage kt + 1 into the other buffer and decodes there the codes of stage kt + 1
  // (R1 for even kt, R0 for odd); the set it has decoded then loads the codes of
  // stage kt + 3.
  float lv[2][16];
#pragma unroll
  for (int t = 0; t < 16; ++t) lv[0][t] = lv_at(lds, code_addr<MODE>(R1, 0, t));
  uint32_t kt = 0;  // relative to k0
  for (; kt + 2 <= nst; kt += 2) {
    stage<CD, MODE, DQ>(acc, lds, 0, R1, R0, lv, p, L, ra, wave, k0 + kt + 1, true, a_row, b_row, xr, h, tid);
    fetch_w<MODE, DQ>(R1, p, L, rc, rq, rs, k0 + kt + 3, k1);
    wait_vmcnt<NW>();  // this wave's copy of stage kt + 1 has landed (the code loads may still fly)
    wait_lgkm0();      // and its decode writes are in LDS
    barrier_only();
    const bool more = kt + 2 < nst;
    stage<CD, MODE, DQ>(acc, lds, 1, R0, R1, lv, p, L, ra, wave, k0 + kt + 2, more, a_row, b_row, xr, h, tid);
    fetch_w<MODE, DQ>(R0, p, L, rc, rq, rs, k0 + kt + 4, k1);
    if (more) wait_vmcnt<NW>(); else __builtin_amdgcn_s_waitcnt(0);
    wait_lgkm0();
    barrier_only();
  }
  if (kt < nst) {
    stage<CD, MODE, DQ>(acc, lds, 0, R1, R0, lv, p, L, ra, wave, k0 + kt + 1, false, a_row, b_row, xr, h, tid);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // the low-rank tail joins the last slice (or the whole tile)
  if (rt < 0 || slice == p.split - 1)
    lora_segment<CD, MODE, true>(acc, lds, p, m0, n0, tid, wave, lane, a_row, b_row, xr, h);
  if (rt < 0) epilogue_lds<CD>(acc, p, lds, m0, n0, wave, wm, wn, lane, h);
  else store_partial(acc, p.part + ((size_t)rt * p.split + slice) * kTileAcc, wm, wn, lane, p.M - m0);
}


// ---------------------------------------------------------------------------
// Dense variant (dequantize-then-GEMM): the W operand is a compute-dtype matrix
// Bd [NB, K1] (W~ for the forward, W~^T for dX, written by the dequantize
// kernels), copied into LDS by the same DMA as the activations.  Stage k: one
// barrier (every copy in flight is stage k's), then 64 MFMAs with the copy of
// stage k + 1 spread over sub-steps 0 (activations) and 1 (W), one instruction
// per two MFMAs, and the fragment reads of the next sub-step between them.
// ---------------------------------------------------------------------------
// The copy of one stage into LDS: rows 8 (4 d + w) + lane / 8 of each tile (d =
// 0..7 by instruction, w the wave); byte offset voffset + d * step + soff.
struct Copy {
  rsrc_t ra, rb;
  uint32_t a_off, b_off, a_step, b_step, soff;
};

// Waves 0..3 copy (one per SIMD); with eight waves, waves 4..7 only compute.
__device__ __forceinline__ void copy_one(const Copy& cp, char* dst_a, char* dst_b, int wave, int d, bool b_side) {
  if (!b_side)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(cp.ra, (lds_void*)(dst_a + (4 * d + wave) * 1024), 16,
                                             (int)(cp.a_off + d * cp.a_step), (int)cp.soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(cp.rb, (lds_void*)(dst_b + (4 * d + wave) * 1024), 16,
                                             (int)(cp.b_off + d * cp.b_step), (int)cp.soff, 0, 0);
}

// One stage of a wave's 128 x 32 JB block (NW = 16 / JB waves): 4 sub-steps of 4 JB
// MFMAs; the 4 + JB fragment reads of the next sub-step are spread over the MFMAs
// of the first three, and (DO_COPY: the copying waves, 0..3; the caller picks the
// form per wave, so no wave branches around its copies) the wave's 8 copies of each
// operand for the next stage go between the MFMAs of sub-steps 0 (activations) and 1
// (W side).
template <int CD, int DO_COPY, int JB>
__device__ __forceinline__ void dense_stage(f32x16_t (&acc)[4][JB], char* lds, int cur, const Copy& cp, int wave,
                                            int a_row, int b_row, int xr, int h) {
  constexpr int NW = 16 / JB, NMF = 4 * JB, NRD = 4 + JB;
  char* As = lds + cur * TILE_BYTES;
  char* Bs = lds + (2 + cur) * TILE_BYTES;
  char* An = lds + (cur ^ 1) * TILE_BYTES;
  char* Bn = lds + (2 + (cur ^ 1)) * TILE_BYTES;
  FragsT<JB> F[2];
  read_frags(F[0], As, Bs, a_row, b_row, xr, h, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    FragsT<JB>& C = F[ks & 1];
    FragsT<JB>& N = F[(ks + 1) & 1];
    const int cphys = ((2 * (ks + 1) + h) ^ xr) << 4;
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      const int i = t / JB, j = t % JB;
      acc[i][j] = mfma<CD>(C.b[j], C.a[i], acc[i][j]);  // block (i, j) transposed
      if (ks < 3) {
#pragma unroll
        for (int r = 0; r < NRD; ++r)
          if (r * NMF / NRD == t) {
            const int f = frag_by_first_use<JB>(r);
            if (f < 4) N.a[f] = *(const u32x4_t*)(As + (a_row + 32 * f) * ROWB + cphys);
            else N.b[f - 4] = *(const u32x4_t*)(Bs + (b_row + 32 * (f - 4)) * ROWB + cphys);
          }
      }
      if constexpr (DO_COPY) {
        if (NW == 4 && ks < 2 && (t & 1) == 1) copy_one(cp, An, Bn, wave, t >> 1, ks == 1);
        if (NW == 8 && ks < 2) copy_one(cp, An, Bn, wave, t, ks == 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One item of the dense kernel: a whole tile, or slice `slice` of cut tile rt.
struct DenseItem {
  int tm, tn, slice, rt;
  int64_t m0, n0;
  uint32_t k0, nmain, n_st;
  bool has_tail, dma_tail;
};

__device__ __forceinline__ DenseItem dense_item(const Big& p, int b) {
  DenseItem it;
  item_of(p, b, it.tm, it.tn, it.slice, it.rt);
  // all four are uniform: keep them (and every address derived from them) scalar
  it.tm = __builtin_amdgcn_readfirstlane(it.tm);
  it.tn = __builtin_amdgcn_readfirstlane(it.tn);
  it.slice = __builtin_amdgcn_readfirstlane(it.slice);
  it.rt = __builtin_amdgcn_readfirstlane(it.rt);
  it.m0 = (int64_t)it.tm * TILE;
  it.n0 = (int64_t)it.tn * TILE;
  // Stages: [k0, k1) of the main contraction (K1 is a multiple of 64 here; all of
  // it for a whole tile, slice `slice` of split for a cut one), then, for a whole
  // tile or the last slice, the low-rank tail: ceil(r_pad / 64) stages of [T | B]
  // (fwd) or [dT | A] (dX), chunks past the valid columns read as zeros.
  const uint32_t KT = (uint32_t)(p.K1 / BK);
  uint32_t k0 = 0, k1 = KT;
  if (it.rt >= 0) {
    k0 = (uint32_t)it.slice * KT / (uint32_t)p.split;
    k1 = (uint32_t)(it.slice + 1) * KT / (uint32_t)p.split;
  }
  it.k0 = k0;
  it.nmain = k1 - k0;
  it.has_tail = it.rt < 0 || it.slice == p.split - 1;
  it.dma_tail = it.has_tail && p.b2_rows != nullptr;
  it.n_st = it.nmain + (it.dma_tail ? (uint32_t)((p.r_pad + BK - 1) / BK) : 0u);
  return it;
}

// The copies of stage u of item `it` (u >= nmain: the tail) for the lane that copies
// rows row + 32 d, logical chunk c.
__device__ __forceinline__ Copy dense_copy(const Big& p, const void* bd, const DenseItem& it, int row, int c,
                                           uint32_t u) {
  Copy cp;
  if (__builtin_expect(u < it.nmain, 1)) {
    cp.ra = make_rsrc(p.a1, p.M * p.ld_a1 * 2);
    cp.rb = make_rsrc(bd, p.NB * p.K1 * 2);
    cp.a_off = (uint32_t)(((it.m0 + row) * p.ld_a1 + 8 * c) * 2);
    cp.b_off = (uint32_t)(((it.n0 + row) * p.K1 + 8 * c) * 2);
    cp.a_step = (uint32_t)(32 * p.ld_a1 * 2);
    cp.b_step = (uint32_t)(32 * p.K1 * 2);
    cp.soff = (it.k0 + u) * (BK * 2);
    return cp;
  }
  const uint32_t t0 = (u - it.nmain) * BK + 8 * c;  // first tail column of this lane's chunk
  cp.ra = make_rsrc(p.a2, p.M * p.r_pad * 2);
  cp.rb = make_rsrc(p.b2_rows, p.NB * p.ld_b2 * 2);
  cp.a_off = oob_unless(t0 < (uint32_t)p.r_pad, (uint32_t)(((it.m0 + row) * p.r_pad + t0) * 2));
  cp.b_off = oob_unless(t0 < (uint32_t)p.r_b2, (uint32_t)(((it.n0 + row) * p.ld_b2 + t0) * 2));
  cp.a_step = (uint32_t)(32 * p.r_pad * 2);
  cp.b_step = (uint32_t)(32 * p.ld_b2 * 2);
  cp.soff = 0;
  return cp;
}

// PERSIST (eight waves, tail by DMA, more items than workgroups): workgroup b takes
// items b, b + G, b + 2 G, ... (G = gridDim.x), the assignment a launch of one
// workgroup per item would make round by round.  After an item's last stage the
// copying waves request the next item's first stage into buffer 0 before the
// epilogue, which then stages its rows in two passes through buffers A1 / B1, so the
// copies land while the stores go out.
template <int CD, int MODE, int NW, bool PERSIST>
__global__ __launch_bounds__(64 * NW, 1) void k_dense256(Big p, const void* bd) {
  // NW waves of 128 x 32 JB output blocks: 4 waves of 128 x 128 (one per SIMD) or 8 of
  // 128 x 64 (two per SIMD, so one wave's MFMAs can run while the other waits)
  constexpr int JB = 16 / NW, WNC = 8 / JB;  // WNC: waves along the tile's columns
  static_assert(!PERSIST || NW == 8, "the persistent form is the eight-wave one");
  // [A0 | A1 | B0 | B1]
  __shared__ __attribute__((aligned(1024))) char lds[4 * TILE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave / WNC) * 128, wn = (wave % WNC) * (32 * JB);
  const int h = lane >> 5;
  const int a_row = wm + (lane & 31), b_row = wn + (lane & 31);
  const int xr = swz(lane & 31);
  // copies by waves 0..3: rows 8 (4 d + wave) + lane / 8 (d = 0..7) of each tile;
  // rows past M or NB read past their buffer (the row is in the lane offset) and land
  // as zeros
  const int row = 8 * (wave & 3) + (lane >> 3);
  const int c = (lane & 7) ^ swz(row);  // the logical chunk this lane's copies fetch
  const int items = p.full + p.rem * p.split;

  int b = blockIdx.x;
  DenseItem it = dense_item(p, b);
  if (wave < 4) {
    const Copy cp = dense_copy(p, bd, it, row, c, 0);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      copy_one(cp, lds, lds + 2 * TILE_BYTES, wave, d, false);
      copy_one(cp, lds, lds + 2 * TILE_BYTES, wave, d, true);
    }
  }
  for (;;) {
    f32x16_t acc[4][JB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    uint32_t u = 0;
    const Copy main_cp = dense_copy(p, bd, it, row, c, 0);
    if (NW == 4 || wave < 4) {
      for (; u + 1 < it.n_st; ++u) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copy of stage u and its fragment reads
        barrier_only();
        dense_stage<CD, 1>(acc, lds, u & 1, dense_copy(p, bd, it, row, c, u + 1), wave, a_row, b_row, xr, h);
      }
    } else {
      for (; u + 1 < it.n_st; ++u) {
        __builtin_amdgcn_s_waitcnt(0);  // its fragment reads (the other waves copy)
        barrier_only();
        dense_stage<CD, 0>(acc, lds, u & 1, main_cp, wave, a_row, b_row, xr, h);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    barrier_only();
    dense_stage<CD, 0>(acc, lds, u & 1, main_cp, wave, a_row, b_row, xr, h);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every wave is past the last stage's reads: the LDS is free

    // a tail whose W-side operand cannot be copied row by row (fwd with r % 8 != 0):
    // the host takes the four-wave form for it
    if constexpr (NW == 4) {
      if (it.has_tail && !it.dma_tail)
        lora_segment<CD, MODE, true>(acc, lds, p, it.m0, it.n0, tid, wave, lane, a_row, b_row, xr, h);
    }
    const int nb = b + (int)gridDim.x;
    if (PERSIST && nb < items) {
      const DenseItem nx = dense_item(p, nb);
      if (wave < 4) {
        const Copy cp = dense_copy(p, bd, nx, row, c, 0);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          copy_one(cp, lds, lds + 2 * TILE_BYTES, wave, d, false);
          copy_one(cp, lds, lds + 2 * TILE_BYTES, wave, d, true);
        }
      }
      // A1 for waves 0..3, B1 for waves 4..7: 8 JB KiB each
      char* W = lds + (wave < 4 ? TILE_BYTES : 3 * TILE_BYTES) + (wave & 3) * (64 * 64 * JB);
      if (it.rt < 0) epilogue_halves<CD>(acc, p, W, it.m0, it.n0, wm, wn, lane, h);
      else store_partial(acc, p.part + ((size_t)it.rt * p.split + it.slice) * kTileAcc, wm, wn, lane, p.M - it.m0);
      b = nb;
      it = nx;
      continue;
    }
    if (it.rt < 0) epilogue_lds<CD>(acc, p, lds, it.m0, it.n0, wave, wm, wn, lane, h);
    else store_partial(acc, p.part + ((size_t)it.rt * p.split + it.slice) * kTileAcc, wm, wn, lane, p.M - it.m0);
    break;
  }
}


// ---------------------------------------------------------------------------
// Fused forward in eight waves, two per SIMD: the dense kernel's stage with the W
// tile decoded from NF4 codes instead of copied.  Waves 0..3 decode (lane t owns W
// row t of the tile and decodes its 64 codes of the next stage between its MFMAs,
// as k_fused256 does); waves 4..7 copy the activation tile by DMA and otherwise only
// multiply, so on every SIMD the copying wave's MFMAs keep the matrix core busy
// while the decoding wave works through its decode.  (Splitting the decode evenly
// over both waves of a SIMD was slower: their decode phases then coincide.)  The
// low-rank tail is copied by DMA (rank a multiple of 8): its activation half by
// waves 4..7, its lora_b half by waves 0..3.
// ---------------------------------------------------------------------------
enum { NEXT_NONE = 0, NEXT_DECODE = 1, NEXT_COPY = 2 };

// One stage of a decoding wave: the 32 MFMAs of its 128 x 64 block from buffer cur
// with the next sub-step's fragment reads between them, and the preparation of the
// next stage's W tile in the other buffer: NEXT_DECODE decodes the codes R (per MFMA
// slot two level lookups of the next quarter and one pack of two weights of the
// current quarter, whose lookups were issued a sub-step earlier; the last sub-step
// looks up quarter 0 of Rn); NEXT_COPY copies the tail's lora_b rows (cp).
template <int CD, int DQ, int NEXT>
__device__ __forceinline__ void fused8_dec_stage(f32x16_t (&acc)[4][2], char* lds, int cur, const CodeRegs& R,
                                                 const CodeRegs& Rn, float (&lv)[2][16], const Copy& cp, int wave,
                                                 int a_row, int b_row, int xr, int h, int tid) {
  char* As = lds + cur * TILE_BYTES;
  char* Bs = lds + (2 + cur) * TILE_BYTES;
  char* An = lds + (cur ^ 1) * TILE_BYTES;
  char* Bn = lds + (2 + (cur ^ 1)) * TILE_BYTES;
  FragsT<2> F[2];
  float sc[8];
  if constexpr (NEXT == NEXT_DECODE) stage_scales<MODE_FWD, DQ>(R, sc);
  read_frags(F[0], As, Bs, a_row, b_row, xr, h, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    FragsT<2>& C = F[ks & 1];
    FragsT<2>& N = F[(ks + 1) & 1];
    float (&lc)[16] = lv[ks & 1];
    float (&ln)[16] = lv[(ks + 1) & 1];
    const int cphys = ((2 * (ks + 1) + h) ^ xr) << 4;
    u32x4_t o;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = t >> 1, j = t & 1;
      acc[i][j] = mfma<CD>(C.b[j], C.a[i], acc[i][j]);  // block (i, j) transposed
      if (ks < 3) {
#pragma unroll
        for (int r = 0; r < 6; ++r)
          if (r * 8 / 6 == t) {
            const int f = frag_by_first_use<2>(r);
            if (f < 4) N.a[f] = *(const u32x4_t*)(As + (a_row + 32 * f) * ROWB + cphys);
            else N.b[f - 4] = *(const u32x4_t*)(Bs + (b_row + 32 * (f - 4)) * ROWB + cphys);
          }
      }
      if constexpr (NEXT == NEXT_DECODE) {
#pragma unroll
        for (int e = 2 * t; e < 2 * t + 2; ++e)
          ln[e] = lv_at(lds, ks < 3 ? code_addr<MODE_FWD>(R, ks + 1, e) : code_addr<MODE_FWD>(Rn, 0, e));
        finish_part<CD, MODE_FWD>(sc, lc, o, Bn, tid, ks, t);
      } else if constexpr (NEXT == NEXT_COPY) {
        if (ks == 1) copy_one(cp, An, Bn, wave, t, true);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One stage of a copying wave: dense_stage with only the activation copies of the
// next stage (one per MFMA slot of sub-step 0).
template <int CD, bool COPY>
__device__ __forceinline__ void fused8_copy_stage(f32x16_t (&acc)[4][2], char* lds, int cur, const Copy& cp, int cw,
                                                  int a_row, int b_row, int xr, int h) {
  char* As = lds + cur * TILE_BYTES;
  char* Bs = lds + (2 + cur) * TILE_BYTES;
  char* An = lds + (cur ^ 1) * TILE_BYTES;
  FragsT<2> F[2];
  read_frags(F[0], As, Bs, a_row, b_row, xr, h, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    FragsT<2>& C = F[ks & 1];
    FragsT<2>& N = F[(ks + 1) & 1];
    const int cphys = ((2 * (ks + 1) + h) ^ xr) << 4;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = t >> 1, j = t & 1;
      acc[i][j] = mfma<CD>(C.b[j], C.a[i], acc[i][j]);
      if (ks < 3) {
#pragma unroll
        for (int r = 0; r < 6; ++r)
          if (r * 8 / 6 == t) {
            const int f = frag_by_first_use<2>(r);
            if (f < 4) N.a[f] = *(const u32x4_t*)(As + (a_row + 32 * f) * ROWB + cphys);
            else N.b[f - 4] = *(const u32x4_t*)(Bs + (b_row + 32 * (f - 4)) * ROWB + cphys);
          }
      }
      if (COPY && ks == 0) copy_one(cp, An, An, cw, t, false);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int CD, int DQ>
__global__ __launch_bounds__(8 * 64, 1) void k_fused8(Big p, Nf4Tables tab) {
  // [A0 | A1 | B0 | B1 | levels]
  __shared__ __attribute__((aligned(1024))) char lds[4 * TILE_BYTES + 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < 16) *(float*)(lds + LV_OFF + 4 * tid) = tab.lv[tid];
  int tm, tn, slice, rt;
  item_of(p, blockIdx.x, tm, tn, slice, rt);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  slice = __builtin_amdgcn_readfirstlane(slice);
  rt = __builtin_amdgcn_readfirstlane(rt);
  const int64_t m0 = (int64_t)tm * TILE, n0 = (int64_t)tn * TILE;
  const int wm = (wave >> 2) * 128, wn = (wave & 3) * 64;
  const int h = lane >> 5;
  const int a_row = wm + (lane & 31), b_row = wn + (lane & 31);
  const int xr = swz(lane & 31);
  const bool decoder = wave < 4;

  // DMA copies (activation tile by waves 4..7; the tail's lora_b rows by waves 0..3):
  // rows 8 (4 d + wave % 4) + lane / 8 of each tile, as in the dense kernel
  const int row = 8 * (wave & 3) + (lane >> 3);
  const int c = (lane & 7) ^ swz(row);
  Copy main_cp;
  main_cp.ra = make_rsrc(p.a1, p.M * p.ld_a1 * 2);
  main_cp.rb = main_cp.ra;
  main_cp.a_off = (uint32_t)(((m0 + row) * p.ld_a1 + 8 * c) * 2);
  main_cp.b_off = 0;
  main_cp.a_step = (uint32_t)(32 * p.ld_a1 * 2);
  main_cp.b_step = 0;

  // the codes of W row n0 + tid (decoding waves)
  const Nf4W& w = p.w;
  const rsrc_t rc = make_rsrc(w.codes, w.rows * w.cols / 2);
  const int64_t nb = w.rows * w.cols / w.bs;
  const rsrc_t rq = DQ ? make_rsrc(w.absmax_q, nb) : make_rsrc(w.absmax, nb * 4);
  const rsrc_t rs = make_rsrc(DQ ? (const void*)w.scale2 : (const void*)w.absmax,
                              DQ ? (((nb - 1) >> w.g_shift) + 1) * 4 : nb * 4);
  Lane L;
  L.row_bytes = (uint32_t)(w.cols / 2);
  L.row_blocks = (uint32_t)(w.cols >> w.bs_shift);
  {
    const uint32_t wrow = (uint32_t)(n0 + (tid & 255));
    L.ok = wrow < (uint32_t)w.rows;
    L.c_off = wrow * L.row_bytes;
    L.b_idx = wrow * L.row_blocks;
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const uint32_t KT = (uint32_t)(p.K1 / BK);
  uint32_t k0 = 0, k1 = KT;
  if (rt >= 0) {
    k0 = (uint32_t)slice * KT / (uint32_t)p.split;
    k1 = (uint32_t)(slice + 1) * KT / (uint32_t)p.split;
  }
  const bool has_tail = rt < 0 || slice == p.split - 1;
  const uint32_t nmain = k1 - k0;
  const uint32_t n_st = nmain + (has_tail ? (uint32_t)((p.r_pad + BK - 1) / BK) : 0u);
  const rsrc_t ra2 = make_rsrc(p.a2, p.M * p.r_pad * 2);
  const rsrc_t rb2 = make_rsrc(p.b2_rows, p.NB * p.ld_b2 * 2);
  auto copy_of = [&](uint32_t u) {  // stage u's copies (u >= nmain: the tail)
    if (u < nmain) {
      Copy cp = main_cp;
      cp.soff = (k0 + u) * (BK * 2);
      return cp;
    }
    const uint32_t t0 = (u - nmain) * BK + 8 * c;
    Copy cp;
    cp.ra = ra2;
    cp.rb = rb2;
    cp.a_off = oob_unless(t0 < (uint32_t)p.r_pad, (uint32_t)(((m0 + row) * p.r_pad + t0) * 2));
    cp.b_off = oob_unless(t0 < (uint32_t)p.r_b2, (uint32_t)(((n0 + row) * p.ld_b2 + t0) * 2));
    cp.a_step = (uint32_t)(32 * p.r_pad * 2);
    cp.b_step = (uint32_t)(32 * p.ld_b2 * 2);
    cp.soff = 0;
    return cp;
  };

  constexpr int NWL = fetch_w_loads<MODE_FWD, DQ>();
  CodeRegs R0, R1;
  float lv[2][16];
  if (decoder) {
    fetch_w<MODE_FWD, DQ>(R0, p, L, rc, rq, rs, k0, k1);
    fetch_w<MODE_FWD, DQ>(R1, p, L, rc, rq, rs, k0 + 1, k1);
  } else {
    const Copy cp = copy_of(0);
#pragma unroll
    for (int d = 0; d < 8; ++d) copy_one(cp, lds, lds, wave & 3, d, false);
  }
  __syncthreads();  // the level table
  if (decoder) {
    // stage 0's W tile (the codes of R0 landed first: R1's loads may still fly)
    wait_vmcnt<NWL>();
#pragma unroll
    for (int q = 0; q < 4; ++q) decode_quarter<CD, MODE_FWD, DQ>(R0, lds, lds + 2 * TILE_BYTES, tid, q);
    fetch_w<MODE_FWD, DQ>(R0, p, L, rc, rq, rs, k0 + 2, k1);
    wait_vmcnt<NWL>();
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  wait_lgkm0();
  barrier_only();

  uint32_t u = 0;
  if (decoder) {
    // stage u decodes stage u + 1's codes: R1 for even u, R0 for odd u; the set it
    // decoded then loads the codes of stage u + 3
#pragma unroll
    for (int t = 0; t < 16; ++t) lv[0][t] = lv_at(lds, code_addr<MODE_FWD>(R1, 0, t));
    for (; u + 2 < nmain; u += 2) {
      fused8_dec_stage<CD, DQ, NEXT_DECODE>(acc, lds, 0, R1, R0, lv, main_cp, wave, a_row, b_row, xr, h, tid);
      fetch_w<MODE_FWD, DQ>(R1, p, L, rc, rq, rs, k0 + u + 3, k1);
      wait_vmcnt<NWL>();  // the code loads may still fly
      wait_lgkm0();       // the W tile writes
      barrier_only();
      fused8_dec_stage<CD, DQ, NEXT_DECODE>(acc, lds, 1, R0, R1, lv, main_cp, wave, a_row, b_row, xr, h, tid);
      fetch_w<MODE_FWD, DQ>(R0, p, L, rc, rq, rs, k0 + u + 4, k1);
      wait_vmcnt<NWL>();
      wait_lgkm0();
      barrier_only();
    }
    if (u + 1 < nmain) {  // u is even here
      fused8_dec_stage<CD, DQ, NEXT_DECODE>(acc, lds, 0, R1, R0, lv, main_cp, wave, a_row, b_row, xr, h, tid);
      __builtin_amdgcn_s_waitcnt(0);
      barrier_only();
      ++u;
    }
    // the tail stages (their lora_b rows copied by DMA), then the last stage
    for (; u + 1 < n_st; ++u) {
      fused8_dec_stage<CD, DQ, NEXT_COPY>(acc, lds, u & 1, R0, R1, lv, copy_of(u + 1), wave & 3, a_row, b_row, xr,
                                          h, tid);
      __builtin_amdgcn_s_waitcnt(0);
      barrier_only();
    }
    fused8_dec_stage<CD, DQ, NEXT_NONE>(acc, lds, u & 1, R0, R1, lv, main_cp, wave, a_row, b_row, xr, h, tid);
  } else {
    for (; u + 1 < n_st; ++u) {
      fused8_copy_stage<CD, true>(acc, lds, u & 1, copy_of(u + 1), wave & 3, a_row, b_row, xr, h);
      __builtin_amdgcn_s_waitcnt(0);
      barrier_only();
    }
    fused8_copy_stage<CD, false>(acc, lds, u & 1, main_cp, wave & 3, a_row, b_row, xr, h);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  if (rt < 0) epilogue_lds<CD>(acc, p, lds, m0, n0, wave, wm, wn, lane, h);
  else store_partial(acc, p.part + ((size_t)rt * p.split + slice) * kTileAcc, wm, wn, lane, p.M - m0);
}

template <int CD, int S>
int launch_split_sum(const Big& b, hipStream_t s);
template <int CD>
int sum_slices(const Big& b, hipStream_t s);

// The fused GEMM, and for a cut last round the sum of its slices (one profiling
// scope: together they are the GEMM).
template <int CD, int MODE>
int run(const Big& b, hipStream_t s, int kind) {
  const int64_t items = (int64_t)b.full + (int64_t)b.rem * b.split;
  ProfScope prof(kind, s);
  if (MODE == MODE_FWD && b.b2_rows) {
    if (b.w.dq)
      k_fused8<CD, 1><<<dim3((unsigned)items), dim3(8 * 64), 0, s>>>(b, host_tables());
    else
      k_fused8<CD, 0><<<dim3((unsigned)items), dim3(8 * 64), 0, s>>>(b, host_tables());
  } else if (b.w.dq) {
    k_fused256<CD, MODE, 1><<<dim3((unsigned)items), dim3(kThreads), 0, s>>>(b, host_tables());
  } else {
    k_fused256<CD, MODE, 0><<<dim3((unsigned)items), dim3(kThreads), 0, s>>>(b, host_tables());
  }
  int rc = check_launch(MODE == MODE_FWD ? "k_fused256<fwd>" : "k_fused256<dx>");
  if (rc || !b.rem) return rc;
  return sum_slices<CD>(b, s);
}

// The dense GEMM, and for a cut last round the sum of its slices (both inside one
// profiling scope: together they are the GEMM).
template <int CD, int MODE>
int run_dense(const Big& b, const void* bd, hipStream_t s, int kind) {
  const int64_t items = (int64_t)b.full + (int64_t)b.rem * b.split;
  ProfScope prof(kind, s);
  // eight waves (two per SIMD) unless the low-rank tail cannot be copied row by row;
  // more items than CUs: one persistent workgroup per CU
  const int64_t cus = cu_count();
  if (b.b2_rows && items > cus)
    k_dense256<CD, MODE, 8, true><<<dim3((unsigned)cus), dim3(8 * 64), 0, s>>>(b, bd);
  else if (b.b2_rows)
    k_dense256<CD, MODE, 8, false><<<dim3((unsigned)items), dim3(8 * 64), 0, s>>>(b, bd);
  else
    k_dense256<CD, MODE, 4, false><<<dim3((unsigned)items), dim3(4 * 64), 0, s>>>(b, bd);
  int rc = check_launch(MODE == MODE_FWD ? "k_dense256<fwd>" : "k_dense256<dx>");
  if (rc || !b.rem) return rc;
  return sum_slices<CD>(b, s);
}

template <int CD, int S>
int launch_split_sum(const Big& b, hipStream_t s) {
  const dim3 g(kTileAcc / (4 * kThreads), (unsigned)b.rem);
  k_split_sum<CD, S><<<g, dim3(kThreads), 0, s>>>(b);
  return check_launch("k_split_sum");
}

template <int CD>
int sum_slices(const Big& b, hipStream_t s) {
  switch (b.split) {
    case 2: return launch_split_sum<CD, 2>(b, s);
    case 4: return launch_split_sum<CD, 4>(b, s);
    case 8: return launch_split_sum<CD, 8>(b, s);
  }
  return set_error(QLORA_ERR_UNSUPPORTED, "split sum: %d slices", b.split);
}

void set_split(Big& b, const DenseSplit& sp, void* split_ws) {
  b.full = sp.full;
  b.rem = sp.rem;
  b.split = sp.split;
  b.part = (float*)split_ws;
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
  if (c.w.rows <= 0 || c.w.cols <= 0 || c.m <= 0) return false;
  if (c.w.bs_shift < 0 || (c.w.dq && c.w.g_shift < 0)) return false;
  if (dx) return (c.w.rows % BK == 0) && fits_buffers(c, c.m * c.w.rows * 2);
  return fits_buffers(c, c.m * c.w.cols * 2);
}

// y = [x | T][W~ | B]^T + bias.  t_cd: [m, r_pad] compute-dtype s x A^T; sp and
// split_ws as for the dense kernel (dense_split(m, rows, cols)).
int fused256_forward(const LayerCall& c, const void* t_cd, int64_t r_pad, void* y, const DenseSplit& sp,
                     void* split_ws) {
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
  set_split(b, sp, split_ws);
  if (c.r % 8 == 0 && c.w.cols % BK == 0) {  // the eight-wave kernel (its tail copies lora_b rows)
    b.b2_rows = c.lora_b;
    b.ld_b2 = c.r;
    b.r_b2 = c.r;
  }
  if (c.cd == CD_BF16) return run<CD_BF16, MODE_FWD>(b, c.stream, QLORA_K_FWD_GEMM);
  return run<CD_F16, MODE_FWD>(b, c.stream, QLORA_K_FWD_GEMM);
}

// dX = [dY | dT][W~ ; A].  dt_cd: [m, r_pad] compute-dtype s dY B; sp and split_ws
// as for the dense kernel (dense_split(m, cols, rows)).
int fused256_dx(const LayerCall& c, const void* dy, const void* dt_cd, int64_t r_pad, void* dx, const DenseSplit& sp,
                void* split_ws) {
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
  set_split(b, sp, split_ws);
  if (c.cd == CD_BF16) return run<CD_BF16, MODE_DX>(b, c.stream, QLORA_K_BWD_DX);
  return run<CD_F16, MODE_DX>(b, c.stream, QLORA_K_BWD_DX);
}

// One round is a tile per compute unit (the kernel needs most of a CU's LDS).  When
// the last round is incomplete, its rem tiles are cut into split = 2 or 4
// contraction slices, 8 when all the tokens fit one tile row or, for the fused
// kernels, two (the largest that keeps rem * split within one round and at least 4
// stages per slice), so the round's workgroups run about 1 / split as long.
// (Measured on q + gate forwards: 8 slices took 128 and 256 tokens from 0.111 /
// 0.119 to 0.096 / 0.111 ms; at 512 tokens the doubled partial sums cost the
// dequantize-then-GEMM path 6%, while the decode-bound fused kernel gains: the
// block's training step at 300 / 512 tokens 1.07 / 1.15 -> 1.03 / 1.11 ms.)
DenseSplit dense_split(int64_t m, int64_t nb, int64_t k1, bool fused) {
  const int64_t C = cu_count();
  const int64_t tiles = ceil_div(m, TILE) * ceil_div(nb, TILE);
  DenseSplit d = {(int32_t)tiles, 0, 1};
  const int64_t F = tiles / C, R = tiles - F * C;
  if (R == 0) return d;
  const int64_t cap = std::min<int64_t>(C / R, (k1 / BK) / 4);
  const int32_t smax = (m <= TILE || (fused && m <= 2 * TILE)) ? 8 : 4;
  int32_t S = 1;
  while (S < smax && 2 * S <= cap) S *= 2;
  if (S == 1) return d;
  d.full = (int32_t)(F * C);
  d.rem = (int32_t)R;
  d.split = S;
  return d;
}

size_t dense_split_bytes(const DenseSplit& sp) { return (size_t)sp.rem * sp.split * kTileAcc * 4; }

// Whether the dense (dequantize-then-GEMM) kernels take this layer: the same
// shapes as the fused ones, and the dequantized copy must fit a buffer resource.
bool dense256_ok(const LayerCall& c, bool dx) {
  if (!fused256_ok(c, dx)) return false;
  return c.w.rows * c.w.cols * 2 < 0x7fff0000LL && (c.w.cols % BK == 0) && (c.w.rows % BK == 0 || !dx);
}

// y = [x | T][W~ | B]^T + bias with W~ [N, K] already in the compute dtype.  sp:
// dense_split(m, rows, cols); split_ws: dense_split_bytes(sp) bytes.
int dense256_forward(const LayerCall& c, const void* wd, const void* t_cd, int64_t r_pad, void* y,
                     const DenseSplit& sp, void* split_ws) {
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
  set_split(b, sp, split_ws);
  if (c.r % 8 == 0) {  // lora_b rows [N][r] copy whole 16-byte chunks: the tail is pipelined
    b.b2_rows = c.lora_b;
    b.ld_b2 = c.r;
    b.r_b2 = c.r;
  }
  if (c.cd == CD_BF16) return run_dense<CD_BF16, MODE_FWD>(b, wd, c.stream, QLORA_K_FWD_GEMM);
  return run_dense<CD_F16, MODE_FWD>(b, wd, c.stream, QLORA_K_FWD_GEMM);
}

// dX = [dY | dT][W~ ; A] with W~^T [K, N] already in the compute dtype.  sp:
// dense_split(m, cols, rows); split_ws as for the forward; a_t: A^T [K][r_pad] in the
// compute dtype, zero past r (the tail's W-side rows), or null.
int dense256_dx(const LayerCall& c, const void* dy, const void* wdt, const void* dt_cd, int64_t r_pad, void* dx,
                const DenseSplit& sp, void* split_ws, const void* a_t) {
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
  set_split(b, sp, split_ws);
  if (a_t) {
    b.b2_rows = a_t;
    b.ld_b2 = r_pad;
    b.r_b2 = (int32_t)r_pad;
  }
  if (c.cd == CD_BF16) return run_dense<CD_BF16, MODE_DX>(b, wdt, c.stream, QLORA_K_BWD_DX);
  return run_dense<CD_F16, MODE_DX>(b, wdt, c.stream, QLORA_K_BWD_DX);
}

}  // namespace qnf4
