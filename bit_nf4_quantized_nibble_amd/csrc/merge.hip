// merge.hip -- the trained adapter folded into a dense weight:
//
//   out [rows, cols] = RNE_cd(w_hat + s (B A)),  w_hat = fl32(L[code] * s_b)
//
// "LoRA and QLoRA, mathematically", section "The merge math, and when merging changes
// behavior", eq. (6.3.6): W_merged = W_0 + (alpha / r) B A, with the NF4 base
// dequantized first and the sum kept dense, since a 4-bit re-quantization would
// round the low-rank update away.  qlora-rs README "Honest capability matrix" (dense
// merge helper: NF4 unpacked at fp32, scale alpha / r or the rsLoRA one).
//
// The kernel is bound by HBM: per element it reads half a byte of codes (plus the
// block scale) and writes 2 bytes of bf16 / f16; the rank-r product B A is 2 r flops
// per element, which at r = 64 is more than the vector ALUs deliver at HBM speed,
// so it runs on MFMA.  A and B are small and stay in L2 across tiles.
#include <algorithm>
#include <atomic>

#include "common.h"

namespace qnf4 {
namespace {

// ---------------------------------------------------------------- MFMA tile kernel
constexpr int kMR = 64;                        // W rows (n) per tile
constexpr int kMC = 256;                       // W columns (k) per tile: 128 bytes of codes per row
constexpr int kRC = 64;                        // ranks staged per slice
constexpr int kMergeThreads = 512;             // 8 waves, each a 32 x 64 block of the tile
constexpr int kRuns = kMR * kMC / 8 / kMergeThreads;  // runs of 8 outputs per thread
constexpr int kBStage = kMR * kRC * 2;         // B slice [64 n][64 t] in LDS
constexpr int kDBytes = kMR * kMC * 4;         // D = B A of the tile, fp32 [64 n][256 k]

struct MergeP {
  Nf4W w;
  const void* a;    // [r, cols] cd
  const void* b;    // [rows, r] cd
  int32_t r;
  int32_t r16;      // r rounded up to 16 (the MFMA rank steps; ranks past r are zero)
  float s;
  void* out;        // [rows, cols] cd
  uint32_t tiles_x;  // tiles along the columns
  uint32_t ntiles;
};

template <int CD>
__device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (CD == CD_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* ptr, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)ptr, (short)0, (int)bytes, 0x00020000);
}
// A buffer offset with bit 31 set lies past every buffer here (all under 2 GiB): the
// load returns zeros.
__device__ __forceinline__ int oob_unless(bool ok, uint32_t off) { return (int)(off | ((uint32_t)(!ok) << 31)); }

// Buffer descriptors of one merge call: a load past the end of a buffer returns 0.
struct MergeRsrc {
  rsrc_t codes, scale, scale2, b, a;
};

template <int DQ>
__device__ __forceinline__ MergeRsrc make_merge_rsrc(const MergeP& p) {
  const Nf4W& w = p.w;
  const int64_t n = w.rows * w.cols, nb = n >> w.bs_shift;
  MergeRsrc r;
  r.codes = make_rsrc(w.codes, n / 2);
  r.scale = DQ ? make_rsrc(w.absmax_q, nb) : make_rsrc(w.absmax, nb * 4);
  r.scale2 = DQ ? make_rsrc(w.scale2, (((nb - 1) >> w.g_shift) + 1) * 4) : r.scale;
  r.b = make_rsrc(p.b, w.rows * p.r * 2);
  r.a = make_rsrc(p.a, p.r * w.cols * 2);
  return r;
}

// What a tile needs from memory, as raw loaded words (converted at use, so that
// nothing waits on them early): the codes and block scales of the thread's 4
// epilogue runs, and its share of the first rank slice of B (one 16-byte chunk) and
// of A (4 ranks x 8 columns, transposed on the way into LDS).
struct CodeRegs {
  uint32_t cw[kRuns];
  uint32_t qa[kRuns];  // q_b (a byte), or the bits of a_b without double quantization
  uint32_t s2[kRuns];  // bits of the group scale S (double quantization)
};
struct StageRegs {
  u32x4_t bq;
  u32x4_t aq[4];
};

// Slice [t0, t0 + 64) of B rows n0 .. n0 + 63: thread tid takes chunk tid & 7 of row
// tid >> 3 (rows past the weight read past the buffer; ranks past r are masked).
__device__ __forceinline__ u32x4_t fetch_b(const MergeP& p, const MergeRsrc& R, int64_t n0, int t0, int tid) {
  const int64_t n = n0 + (tid >> 3);
  const int t = t0 + 8 * (tid & 7);
  return __builtin_amdgcn_raw_buffer_load_b128(R.b, oob_unless(t < p.r, (uint32_t)((n * p.r + t) * 2)), 0, 0);
}
// Slice [t0, t0 + 64) of A, columns k0 .. k0 + 255: thread tid takes ranks
// t0 + 4 (tid & 15) + i (i = 0..3) of columns k0 + 8 (tid >> 4) .. + 7 (columns past
// cols read past the buffer: zeros; ranks past r are masked).
__device__ __forceinline__ void fetch_a(const MergeP& p, const MergeRsrc& R, int64_t k0, int t0, int tid,
                                        u32x4_t (&aq)[4]) {
  const int64_t k = k0 + 8 * (tid >> 4);
  const bool kin = k < p.w.cols;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * (tid & 15) + i;
    aq[i] = __builtin_amdgcn_raw_buffer_load_b128(R.a, oob_unless(t < p.r && kin, (uint32_t)((t * p.w.cols + k) * 2)),
                                                  0, 0);
  }
}

__device__ __forceinline__ void tile_origin(const MergeP& p, uint32_t tile, int64_t& n0, int64_t& k0) {
  const uint32_t ty = tile / p.tiles_x;
  n0 = (int64_t)ty * kMR;
  k0 = (int64_t)(tile - ty * p.tiles_x) * kMC;
}

// Epilogue runs of thread tid: rows (tid >> 5) + 16 j of the tile, columns
// 8 (tid & 31) .. + 7.  Runs below the last row read past the buffers (zeros); runs
// right of the last column read other elements, and are masked at the store.
template <int DQ>
__device__ __forceinline__ void fetch_codes(const MergeP& p, const MergeRsrc& R, uint32_t tile, int tid,
                                            CodeRegs& C) {
  const Nf4W& w = p.w;
  int64_t n0, k0;
  tile_origin(p, tile, n0, k0);
  const int64_t e0 = (n0 + (tid >> 5)) * w.cols + k0 + 8 * (tid & 31);
#pragma unroll
  for (int j = 0; j < kRuns; ++j) {
    const int64_t e = e0 + j * 16 * w.cols;
    const uint32_t blk = (uint32_t)(e >> w.bs_shift);
    C.cw[j] = __builtin_amdgcn_raw_buffer_load_b32(R.codes, (int)(uint32_t)(e >> 1), 0, 0);
    if constexpr (DQ) {
      C.qa[j] = __builtin_amdgcn_raw_buffer_load_b8(R.scale, (int)blk, 0, 0);
      C.s2[j] = __builtin_amdgcn_raw_buffer_load_b32(R.scale2, (int)((blk >> w.g_shift) * 4), 0, 0);
    } else {
      C.qa[j] = __builtin_amdgcn_raw_buffer_load_b32(R.scale, (int)(blk * 4), 0, 0);
      C.s2[j] = 0u;
    }
  }
}

__device__ __forceinline__ void fetch_stage(const MergeP& p, const MergeRsrc& R, uint32_t tile, int t0, int tid,
                                            StageRegs& S) {
  int64_t n0, k0;
  tile_origin(p, tile, n0, k0);
  S.bq = fetch_b(p, R, n0, t0, tid);
  fetch_a(p, R, k0, t0, tid, S.aq);
}

// LDS slice layout: 128-byte rows of 64 ranks; 16-byte chunk c of row x at c ^ (x & 7).
// B rows are copied as they are.  A arrives as 4 ranks x 8 columns per thread and
// leaves as 8 rows (columns) of 4 ranks: each 8-byte piece pairs the 16-bit halves
// of two input words (byte permutes), and the 16 lanes of a column group fill whole
// 128-byte rows.
__device__ __forceinline__ void stage(char* lds, int tid, const u32x4_t& bq, const u32x4_t (&aq)[4]) {
  {
    const int row = tid >> 3, c = tid & 7;
    *(u32x4_t*)(lds + row * 128 + ((c ^ (row & 7)) << 4)) = bq;
  }
  const int tq = tid & 15, kc = tid >> 4;
  const int chunk = tq >> 1, half = (tq & 1) * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
    u32x2_t v;
    v[0] = __builtin_amdgcn_perm(aq[1][e >> 1], aq[0][e >> 1], sel);
    v[1] = __builtin_amdgcn_perm(aq[3][e >> 1], aq[2][e >> 1], sel);
    const int row = 8 * kc + e;
    *(u32x2_t*)(lds + kBStage + row * 128 + ((chunk ^ (row & 7)) << 4) + half) = v;
  }
}

// Persistent: workgroup g takes tiles g, g + G, ... (G = grid size) of 64 x 256.
// Loads run one phase ahead of their use: the next tile's first rank slice is
// requested after this tile's rank product, its codes and scales after this tile's
// merge.  Per tile:
//   1. the first rank slice goes from registers to LDS (B rows; A transposed);
//   2. D = B A on MFMA (32x32x16): lane rows = W rows (B), columns = W columns (A^T);
//      ranks beyond the first 64 are staged slice by slice;
//   3. D goes through LDS as fp32 [n][k] (chunk ck of row nl at ck ^ 8 ((nl >> 2) & 1),
//      which puts the two half-waves on disjoint banks);
//   4. each thread merges 4 runs of 8 consecutive columns: w_hat = fl32(L[c] s_b),
//      out = RNE(fma(s, D, w_hat)); 32 lanes write 512 contiguous bytes of a row.
// Requires cd bf16 / f16, cols % 8 == 0, block_size a power of two >= 8 (with
// double quantization a power-of-two group, or one group), r % 8 == 0, and codes,
// A and B under 2 GiB.
template <int CD, int DQ>
__global__ __launch_bounds__(kMergeThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_merge_mfma(MergeP p,
                                                                                                     Nf4Tables tab) {
  __shared__ __attribute__((aligned(16))) char lds[kDBytes];
  __shared__ float s_lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  if (tid < 16) s_lv[tid] = tab.lv[tid];
  const Nf4W& w = p.w;
  const int wn = (wave & 1) * 32, wk = (wave >> 1) * 64;
  uint32_t tile = blockIdx.x;
  if (tile >= p.ntiles) return;
  const MergeRsrc R = make_merge_rsrc<DQ>(p);
  CodeRegs C;
  StageRegs S;
  fetch_codes<DQ>(p, R, tile, tid, C);
  fetch_stage(p, R, tile, 0, tid, S);
  float* dl = (float*)lds;
  while (true) {
    int64_t n0, k0;
    tile_origin(p, tile, n0, k0);
    const uint32_t next = tile + gridDim.x;
    __syncthreads();  // the previous tile's D is fully read
    stage(lds, tid, S.bq, S.aq);
    __syncthreads();

    f32x16_t acc[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[jt][v] = 0.f;
    for (int t0 = 0; t0 < p.r16; t0 += kRC) {
      if (t0) {  // later slices: staged here, not prefetched
        fetch_stage(p, R, tile, t0, tid, S);
        __syncthreads();
        stage(lds, tid, S.bq, S.aq);
        __syncthreads();
      }
      const int steps = min(kRC, p.r16 - t0) / 16;
      const int nl = wn + (lane & 31);
      for (int st = 0; st < steps; ++st) {
        const int tc = 2 * st + h;
        const u32x4_t av = *(const u32x4_t*)(lds + nl * 128 + ((tc ^ (nl & 7)) << 4));
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          const int kl = wk + 32 * jt + (lane & 31);
          const u32x4_t bv = *(const u32x4_t*)(lds + kBStage + kl * 128 + ((tc ^ (kl & 7)) << 4));
          acc[jt] = mfma<CD>(av, bv, acc[jt]);
        }
      }
    }
    if (next < p.ntiles) fetch_stage(p, R, next, 0, tid, S);

    __syncthreads();  // staged slices fully read: D overwrites them
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const int kl = wk + 32 * jt + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int nl = wn + 8 * (v >> 2) + 4 * h + (v & 3);
        dl[nl * kMC + (((kl >> 2) ^ (((nl >> 2) & 1) << 3)) << 2) + (kl & 3)] = acc[jt][v];
      }
    }
    __syncthreads();

    const int c8 = tid & 31;
    const int64_t k = k0 + 8 * c8;
    uint16_t* orow = (uint16_t*)p.out + (n0 + (tid >> 5)) * w.cols + k;
#pragma unroll
    for (int j = 0; j < kRuns; ++j) {
      const int nl = (tid >> 5) + 16 * j;
      if (n0 + nl >= w.rows || k >= w.cols) continue;
      const int sw = ((nl >> 2) & 1) << 3;
      const f32x4_t d0 = *(const f32x4_t*)(dl + nl * kMC + (((2 * c8) ^ sw) << 2));
      const f32x4_t d1 = *(const f32x4_t*)(dl + nl * kMC + (((2 * c8 + 1) ^ sw) << 2));
      const float sc = DQ ? fl32_mul((float)C.qa[j], __uint_as_float(C.s2[j])) : __uint_as_float(C.qa[j]);
      float f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {  // byte i / 2; element 2k in the high nibble
        const float what = fl32_mul(s_lv[(C.cw[j] >> ((i >> 1) * 8 + ((i & 1) ? 0 : 4))) & 15u], sc);
        f[i] = fmaf(p.s, i < 4 ? d0[i] : d1[i - 4], what);
      }
      u32x4_t o;
      o[0] = pack2<CD>(f[0], f[1]);
      o[1] = pack2<CD>(f[2], f[3]);
      o[2] = pack2<CD>(f[4], f[5]);
      o[3] = pack2<CD>(f[6], f[7]);
      __builtin_nontemporal_store(o, (u32x4_t*)(orow + j * 16 * w.cols));  // not read again here: keep A, B cached
    }
    if (next >= p.ntiles) break;
    fetch_codes<DQ>(p, R, next, tid, C);
    tile = next;
  }
}

// ---------------------------------------------------------------- generic kernel
// Any dtype (fp32 included), rank and shape: 64 x 64 tiles, each thread a 4 x 4
// block of outputs; B A summed in fp32 in rank order with fused multiply-adds.
constexpr int kGT = 64;
constexpr int kGR = 32;

struct GenP {
  Nf4W w;
  const void* a;  // [r, cols] cd
  const void* b;  // [rows, r] cd
  int32_t r;
  float s;
  void* out;      // [rows, cols] cd
};

template <int CD>
__global__ __launch_bounds__(256) void k_merge_generic(GenP p, Nf4Tables tab) {
  __shared__ float s_lv[16];
  __shared__ float bsh[kGT][kGR + 1];  // [n][t]
  __shared__ float ash[kGR][kGT];      // [t][k]
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  if (tid < 16) s_lv[tid] = tab.lv[tid];
  const Nf4W& w = p.w;
  const int64_t n0 = (int64_t)blockIdx.y * kGT, k0 = (int64_t)blockIdx.x * kGT;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = 0.f;
  for (int t0 = 0; t0 < p.r; t0 += kGR) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kGT * kGR / 256; ++q) {
      const int idx = tid + 256 * q;
      {
        const int nl = idx / kGR, tl = idx % kGR;
        const int64_t n = n0 + nl;
        const int t = t0 + tl;
        bsh[nl][tl] = (n < w.rows && t < p.r) ? load_cd<CD>(p.b, n * p.r + t) : 0.f;
      }
      {
        const int tl = idx / kGT, kl = idx % kGT;
        const int t = t0 + tl;
        const int64_t k = k0 + kl;
        ash[tl][kl] = (t < p.r && k < w.cols) ? load_cd<CD>(p.a, (int64_t)t * w.cols + k) : 0.f;
      }
    }
    __syncthreads();
    const int tcount = min(kGR, p.r - t0);
    for (int t = 0; t < tcount; ++t) {
      float bv[4], av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[i] = bsh[ty * 4 + i][t];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) av[jj] = ash[t][tx * 4 + jj];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fmaf(bv[i], av[jj], acc[i][jj]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = n0 + ty * 4 + i;
    if (n >= w.rows) continue;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int64_t k = k0 + tx * 4 + jj;
      if (k >= w.cols) continue;
      const int64_t e = n * w.cols + k;
      const uint32_t byte = w.codes[e >> 1];
      const uint32_t code = (e & 1) ? (byte & 15u) : (byte >> 4);
      const float what = fl32_mul(s_lv[code], block_scale(w, block_of(w, e)));
      store_cd<CD>(p.out, e, fmaf(p.s, acc[i][jj], what));
    }
  }
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }


}  // namespace

// out = RNE_cd(w_hat + s B A).  bf16 / f16 with r, cols and the block size multiples
// of 8 and 16-byte aligned arrays run on the persistent MFMA kernel with two
// workgroups per compute unit.  Everything else runs on the generic kernel, which
// gives the same w_hat and differs only in the order of the fp32 rank sum.
int launch_merge(const Nf4W& w, const void* a, const void* b, int32_t r, float s, int cd, void* out,
                 hipStream_t st) {
  const Nf4Tables& t = host_tables();
  ProfScope prof(QLORA_K_MERGE, st);
  const int64_t lim = 1LL << 31;
  const bool fast = (cd == CD_BF16 || cd == CD_F16) && r % 8 == 0 && w.cols % 8 == 0 && w.bs_shift >= 3 &&
                    (!w.dq || w.g_shift >= 0) && aligned16(a) && aligned16(b) && aligned16(out) &&
                    w.rows * w.cols / 2 < lim && w.rows * r * 2 < lim && r * w.cols * 2 < lim;
  if (fast) {
    MergeP p;
    p.w = w;
    p.a = a;
    p.b = b;
    p.r = r;
    p.r16 = (int32_t)round_up(r, 16);
    p.s = s;
    p.out = out;
    const int64_t tx = ceil_div(w.cols, kMC), nt = ceil_div(w.rows, kMR) * tx;
    p.tiles_x = (uint32_t)tx;
    p.ntiles = (uint32_t)nt;
    const int64_t grid = std::min<int64_t>(nt, 2 * (int64_t)cu_count());
    const dim3 g((unsigned)grid), blk(kMergeThreads);
    if (cd == CD_BF16) {
      if (w.dq) k_merge_mfma<CD_BF16, 1><<<g, blk, 0, st>>>(p, t);
      else k_merge_mfma<CD_BF16, 0><<<g, blk, 0, st>>>(p, t);
    } else {
      if (w.dq) k_merge_mfma<CD_F16, 1><<<g, blk, 0, st>>>(p, t);
      else k_merge_mfma<CD_F16, 0><<<g, blk, 0, st>>>(p, t);
    }
    return check_launch("k_merge_mfma");
  }
  GenP p;
  p.w = w;
  p.a = a;
  p.b = b;
  p.r = r;
  p.s = s;
  p.out = out;
  const int64_t gy = ceil_div(w.rows, kGT), gx = ceil_div(w.cols, kGT);
  if (gy > 65535 || gx > 0x7fffffff) return set_error(QLORA_ERR_UNSUPPORTED, "merge: weight too large");
  const dim3 grid((unsigned)gx, (unsigned)gy);
  if (cd == CD_BF16) k_merge_generic<CD_BF16><<<grid, dim3(256), 0, st>>>(p, t);
  else if (cd == CD_F16) k_merge_generic<CD_F16><<<grid, dim3(256), 0, st>>>(p, t);
  else k_merge_generic<CD_F32><<<grid, dim3(256), 0, st>>>(p, t);
  return check_launch("k_merge_generic");
}

}  // namespace qnf4
