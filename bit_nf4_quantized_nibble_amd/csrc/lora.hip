// lora.hip -- the rank-r products of the QLoRA layer (bf16 / f16 compute, r <= 64)
// on gfx950:
//
//   forward   T0 = x A^T                 [M, r]   contraction over K
//   backward  dT = s dY B                [M, r]   contraction over N
//             dA = dT^T x                [r, K]   contraction over the M tokens
//             dB = s dY^T T0             [N, r]   contraction over the M tokens
//
// ("LoRA and QLoRA, mathematically": only the low-rank factors train; qlora-rs
// README "Honest capability matrix": the adapters update, the base stays frozen.)
//
// All four are C[p, t] = sum_k Aop[p, k] Bop[t, k] with t < r <= 64: one skinny
// kernel, output tile 128 (p) x 64 (t), 4 waves of 32 x 64 (two MFMA 32x32x16
// tiles each), 64-element contraction stages in three LDS buffers (the copies run
// two stages ahead), and a split of the contraction into S slices whose fp32
// partial sums a second kernel adds in slice order.  Bop is a small [t][k] matrix
// with k contiguous (A, or a transposed copy of dT or T0), or, for dT, lora_b as
// it is stored, [k][t] with t contiguous (BT: 128-byte rows of t, chunk c of row k
// at chunk c ^ 4 ((k / 8) % 2); a fragment is gathered with 16-bit reads like a TN
// one).  Every tile is copied global -> LDS by DMA.  Aop is either
//   NT: a matrix [p][k] with k contiguous (x, dY): 128-byte rows of k, 16-byte
//       chunk c of row r at chunk c ^ swz(r), or
//   TN: a matrix X [k][p] with p contiguous (x or dY read along the tokens):
//       256-byte rows of p, chunk c of row k at chunk c ^ (k % 16); a fragment
//       (8 consecutive k of one p) is gathered with 16-bit reads, and the swizzle
//       puts the two row groups a read instruction touches on distinct banks.
#include <algorithm>

#include "common.h"
#include "reduce_dev.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int BP = 128;          // output rows (p) per workgroup
constexpr int BR = 64;           // rank columns (t) per workgroup
constexpr int BK = 64;           // contraction elements per stage
constexpr int ROWB = 128;        // swizzled NT / Bop LDS row: 64 elements
constexpr int XROW = 2 * BP;     // swizzled TN LDS row: 128 elements (256 bytes)
constexpr int A_BYTES = 16384;   // NT: 128 rows x 128 B; TN: 64 rows x 256 B
constexpr int B_BYTES = BR * ROWB;   // 8 KiB
constexpr int DEPTH = 2;          // stages whose copies fly ahead of the one in use (two
                                 // workgroups per CU fit; deeper prefetch measured no faster)
constexpr int NBUF = DEPTH + 1;
constexpr int STAGE = A_BYTES + B_BYTES;
constexpr int kCopies = 6;       // DMA instructions per lane per stage (4 Aop + 2 Bop)
static_assert(BR == kRedBR && kThreads == kRedThreads, "the partial-sum layout the reduction reads");

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t oob_unless(bool ok, uint32_t off) { return off | ((uint32_t)(!ok) << 31); }
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int CD>
__device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (CD == CD_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

struct SkP {
  const void* a;    // NT: [P][lda], k contiguous; TN: [arows][lda], p contiguous
  int64_t lda;
  int64_t arows;    // rows of a (TN: the true token count; rows up to Kc past it read as zeros)
  const void* b;    // [R][ldb], k contiguous (rows >= R read as zeros); BT: [brows][ldb],
                    // t contiguous (rows >= brows and columns >= R read as zeros)
  int64_t ldb, brows;
  int64_t P, R, Kc;
  int64_t kslice;   // contraction per slice (multiple of 64)
  float* part;      // [S][P][64] fp32
};

// Copy of one stage's Bop tile (64 rows of 64 elements): DMA instruction d of wave
// w fills rows 8 (4 d + w) .. +8; lane l lands in physical chunk l % 8 of row l / 8.
__device__ __forceinline__ void copy_b(const SkP& p, rsrc_t rb, char* dst, int wave, int lane, int64_t k) {
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int row = 8 * (4 * d + wave) + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(dst + (4 * d + wave) * 1024), 16,
                                             (int)oob_unless(row < p.R, (uint32_t)((row * p.ldb + k + 8 * c) * 2)),
                                             0, 0, 0);
  }
}

// BT Bop tile (rows k .. k+63 of lora_b as stored, R <= 64 columns of t): rows as in
// copy_b, logical chunk c of row `row` at physical chunk c ^ 4 ((row / 8) % 2), so the
// two row groups of a gather instruction (rows e and 8 + e) sit on distinct banks.
__device__ __forceinline__ void copy_b_t(const SkP& p, rsrc_t rb, char* dst, int wave, int lane, int64_t k) {
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int row = 8 * (4 * d + wave) + (lane >> 3);
    const int c = (lane & 7) ^ (4 * ((row >> 3) & 1));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rb, (lds_void*)(dst + (4 * d + wave) * 1024), 16,
        (int)oob_unless(8 * c < p.R, (uint32_t)(((k + row) * p.ldb + 8 * c) * 2)), 0, 0, 0);
  }
}

// NT Aop tile (128 rows of 64 elements) by DMA, like copy_b.
__device__ __forceinline__ void copy_a_nt(const SkP& p, rsrc_t ra, char* dst, int64_t p0, int wave, int lane,
                                          int64_t k) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int row = 8 * (4 * d + wave) + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    const int64_t gr = p0 + row;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dst + (4 * d + wave) * 1024), 16,
                                             (int)oob_unless(gr < p.P, (uint32_t)((gr * p.lda + k + 8 * c) * 2)),
                                             0, 0, 0);
  }
}

// TN Aop tile (X rows k .. k+63, columns p0 .. p0+127) by DMA: instruction d of
// wave w fills rows 4 (4 d + w) .. +4; lane l lands in physical chunk l % 16 of row
// l / 16.  Rows past the true token count and columns past P read as zeros.
__device__ __forceinline__ void copy_a_tn(const SkP& p, rsrc_t ra, char* dst, int64_t p0, int wave, int lane,
                                          int64_t k) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int row = 4 * (4 * d + wave) + (lane >> 4);
    const int c = (lane & 15) ^ (row & 15);
    const bool ok = p0 + 8 * c < p.P;  // P is a multiple of 8: a chunk is all in or all out
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ra, (lds_void*)(dst + (4 * d + wave) * 1024), 16,
        (int)oob_unless(ok, (uint32_t)(((k + row) * p.lda + p0 + 8 * c) * 2)), 0, 0, 0);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// dst [cols][ld_dst] (cd) = cd(scale * src[rows][ld_src]^T), src in cd or fp32;
// each dst row gets wd columns (ld_dst unless a narrower slice of a wider matrix is
// written), columns rows .. wd-1 zeros.  Tiles of 64 x 64 through LDS; one
// launch can carry two such jobs (workgroups [0, tiles of job 0) take job 0), and
// a job can ride on a rank-product launch (k_skinny).
struct TrJob {
  const void* src;
  int64_t ld_src, rows, cols;
  float scale;
  void* dst;
  int64_t ld_dst;  // row stride of dst
  int64_t wd;      // columns of dst written per row (zeros from rows on)
  int32_t tiles_x, tiles;
};
struct TrJobs {
  TrJob j[2];
};

// Tile b of job j through the LDS tile t (256 threads).
template <int CD, int SRC32>
__device__ __forceinline__ void transpose_tile(const TrJob& j, int b, float (*t)[65]) {
  const int64_t r0 = (int64_t)(b % j.tiles_x) * 64, c0 = (int64_t)(b / j.tiles_x) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  // all 16 loads of a thread leave before the first is used: out-of-range elements
  // read element 0 and are replaced by zero afterwards
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + ty + 4 * i, c = c0 + tx;
    const int64_t at = (r < j.rows && c < j.cols) ? r * j.ld_src + c : 0;
    v[i] = SRC32 ? ((const float*)j.src)[at] : load_cd<CD>(j.src, at);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + ty + 4 * i, c = c0 + tx;
    t[ty + 4 * i][tx] = (r < j.rows && c < j.cols) ? v[i] * j.scale : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int y = ty + 4 * i;
    const int64_t c = c0 + y, r = r0 + tx;
    if (c < j.cols && r < j.wd) store_cd<CD>(j.dst, c * j.ld_dst + r, r < j.rows ? t[tx][y] : 0.f);
  }
}

template <int CD, int SRC32>
__global__ __launch_bounds__(kThreads) void k_transpose(TrJobs js) {
  __shared__ float t[64][65];
  const int w = (int)blockIdx.x >= js.j[0].tiles ? 1 : 0;
  transpose_tile<CD, SRC32>(js.j[w], blockIdx.x - (w ? js.j[0].tiles : 0), t);
}

// One launch carries up to kSkJobs products (blockIdx.z picks the job; workgroups
// outside a job's own grid leave at once) and optionally a transpose (plane z = nj
// of the grid, its workgroups taking the tiles in turn).
constexpr int kSkJobs = 4;
struct SkP2 {
  SkP j[kSkJobs];
  uint32_t nx[kSkJobs], ny[kSkJobs];
  uint32_t nj;  // products
  TrJob tr;     // tr.tiles == 0: none
};

// MODE: 0 NT, 1 TN (Aop forms), 2 NT with the BT Bop.
template <int CD, int MODE>
__global__ __launch_bounds__(kThreads) void k_skinny(SkP2 ps) {
  constexpr bool TN = MODE == 1, BT = MODE == 2;
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * STAGE];  // stage b: [A | B]
  const int jb = blockIdx.z;
  if (jb == (int)ps.nj) {
    const int nb = (int)(gridDim.x * gridDim.y);
    for (int b = (int)(blockIdx.y * gridDim.x + blockIdx.x); b < ps.tr.tiles; b += nb) {
      if (b != (int)(blockIdx.y * gridDim.x + blockIdx.x)) __syncthreads();  // the tile before is stored
      transpose_tile<CD, 0>(ps.tr, b, (float (*)[65])lds);
    }
    return;
  }
  if (blockIdx.x >= ps.nx[jb] || blockIdx.y >= ps.ny[jb]) return;
  const SkP& p = ps.j[jb];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  const int64_t p0 = (int64_t)blockIdx.x * BP;
  const int64_t k0 = (int64_t)blockIdx.y * p.kslice;
  const int64_t k1 = k0 + p.kslice < p.Kc ? k0 + p.kslice : p.Kc;
  const int nst = (int)((k1 - k0) / BK);
  const rsrc_t ra = make_rsrc(p.a, p.arows * p.lda * 2);
  const rsrc_t rb = make_rsrc(p.b, (BT ? p.brows : p.R) * p.ldb * 2);
  const int xr = swz(i);  // swizzle of the 128-byte rows this lane reads (they differ by 32)
  // TN: column 32 wave + i is chunk pc, element pe of it; rows 8 h + j (j < 8) of
  // a 16-row step sit at chunk pc ^ ((8 h + j) % 16)
  const int pc = (32 * wave + i) >> 3, pe = (i & 7) * 2;
  int tn_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) tn_off[j] = (8 * h + j) * XROW + 16 * (pc ^ ((8 * h + j) & 15)) + pe;
  // BT: rank column 32 j + i of rows 8 h + e (e < 8) of a 16-row step: logical chunk
  // 4 j + i / 8, physical chunk (4 j + i / 8) ^ 4 h; block j = 1 sits 64 bytes after
  // block 0 for h = 0 and 64 before it for h = 1
  int bt_off[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bt_off[e] = (8 * h + e) * ROWB + 16 * ((i >> 3) ^ (4 * h)) + 2 * (i & 7);
  const int bt_j1 = h ? -64 : 64;

  f32x16_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;

  auto copy = [&](int st) {
    char* dst = lds + (st % NBUF) * STAGE;
    const int64_t k = k0 + (int64_t)st * BK;
    if (TN) copy_a_tn(p, ra, dst, p0, wave, lane, k);
    else copy_a_nt(p, ra, dst, p0, wave, lane, k);
    if (BT) copy_b_t(p, rb, dst + A_BYTES, wave, lane, k);
    else copy_b(p, rb, dst + A_BYTES, wave, lane, k);
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (d < nst) copy(d);
  for (int s = 0; s < nst; ++s) {
    // stage s landed in every wave (the up to DEPTH - 1 later stages may still fly;
    // a wave sees its copies complete in issue order); stage s - 1's reads done
    const int ahead = min(DEPTH - 1, nst - 1 - s);
    if (ahead >= 3) wait_vm<3 * kCopies>();
    else if (ahead == 2) wait_vm<2 * kCopies>();
    else if (ahead == 1) wait_vm<kCopies>();
    else wait_vm<0>();
    __builtin_amdgcn_s_waitcnt(0x3f | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    barrier_only();
    if (s + DEPTH < nst) copy(s + DEPTH);  // into the buffer stage s - 1 used
    const char* As = lds + (s % NBUF) * STAGE;
    const char* Bs = As + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cphys = ((2 * ks + h) ^ xr) << 4;
      u32x4_t a;
      if (TN) {
        // 8 consecutive k (rows 16 ks + 8 h ..) of column 32 wave + i
        const char* src = As + 16 * ks * XROW;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a[e] = (uint32_t)*(const uint16_t*)(src + tn_off[2 * e]) |
                 ((uint32_t)*(const uint16_t*)(src + tn_off[2 * e + 1]) << 16);
      } else {
        a = *(const u32x4_t*)(As + (32 * wave + i) * ROWB + cphys);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4_t b;
        if (BT) {
          // 8 consecutive k (rows 16 ks + 8 h ..) of rank column 32 j + i
          const char* src = Bs + 16 * ks * ROWB + j * bt_j1;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            b[e] = (uint32_t)*(const uint16_t*)(src + bt_off[2 * e]) |
                   ((uint32_t)*(const uint16_t*)(src + bt_off[2 * e + 1]) << 16);
        } else {
          b = *(const u32x4_t*)(Bs + (32 * j + i) * ROWB + cphys);
        }
        acc[j] = mfma<CD>(a, b, acc[j]);
      }
    }
  }

  // partial sums: lane (i, h) holds rows 32 wave + 8 (v / 4) + 4 h + v % 4, column 32 j + i
  float* out = p.part + (int64_t)blockIdx.y * p.P * BR;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = p0 + 32 * wave + 8 * (v >> 2) + 4 * h + (v & 3);
      if (row < p.P) out[row * BR + 32 * j + i] = acc[j][v];
    }
}

template <int CD>
__global__ __launch_bounds__(kThreads) void k_skreduce(RedJobs js) {
  skreduce_block<CD>(js, blockIdx.x);
}

}  // namespace

// The skinny path takes bf16 / f16 layers with r <= 64 whose contractions are whole
// stages and whose P dimensions are multiples of 8 (16-byte chunks).
bool skinny_ok(int cd, int64_t r) { return (cd == CD_BF16 || cd == CD_F16) && r >= 1 && r <= BR; }

// Slices of the contraction: about 256 workgroups, at most 8 slices (the partial
// sums are written and read back once more).
void skinny_split(int64_t P, int64_t Kc, int* S, int64_t* kslice) {
  const int64_t tiles = ceil_div(P, BP);
  int64_t s = ceil_div(256, tiles);
  const int64_t steps = Kc / BK;
  if (s > steps) s = steps;
  if (s > kRedMaxS) s = kRedMaxS;
  if (s < 1) s = 1;
  const int64_t ks = round_up(ceil_div(Kc, s), BK);
  *kslice = ks;
  *S = (int)ceil_div(Kc, ks);
}

size_t skinny_part_bytes(int64_t P, int64_t Kc) {
  int S;
  int64_t ks;
  skinny_split(P, Kc, &S, &ks);
  return (size_t)S * P * BR * 4;
}

// part = per-slice sums of Aop . Bop^T over the contraction 0 .. Kc (a multiple of
// 64); Aop NT [P][lda] or TN [arows][lda]; Bop [R][ldb] with ldb >= Kc, zero
// between its true width and Kc.
namespace {
int skinny_params(bool tn, const SkSpec& sp, float* part, SkP& p, int* S_out) {
  const bool bad_b = sp.bt ? (tn || sp.R % 8 || sp.ldb < sp.R || sp.brows * sp.ldb * 2 >= (1LL << 31))
                           : sp.ldb < sp.Kc;
  if (sp.Kc % BK || sp.lda % 8 || sp.ldb % 8 || bad_b || (tn && sp.P % 8))
    return set_error(QLORA_ERR_UNSUPPORTED, "rank product: shape not supported by the skinny kernel");
  p = SkP{};
  p.a = sp.a;
  p.lda = sp.lda;
  p.arows = sp.arows;
  p.b = sp.b;
  p.ldb = sp.ldb;
  p.brows = sp.brows;
  p.P = sp.P;
  p.R = sp.R;
  p.Kc = sp.Kc;
  p.part = part;
  skinny_split(sp.P, sp.Kc, S_out, &p.kslice);
  return QLORA_OK;
}

// The device form of a transpose job; false when it has nothing to write.
bool tr_job(const TransposeSpec& t, TrJob& j) {
  if (t.ld_dst == 0 || t.cols == 0) return false;
  j.src = t.src;
  j.ld_src = t.ld_src;
  j.rows = t.rows;
  j.cols = t.cols;
  j.scale = t.scale;
  j.dst = t.dst;
  j.ld_dst = t.ld_dst;
  j.wd = t.w_dst ? t.w_dst : t.ld_dst;
  j.tiles_x = (int32_t)ceil_div(j.wd, 64);
  j.tiles = (int32_t)(j.tiles_x * ceil_div(t.cols, 64));
  return j.tiles > 0;
}
}  // namespace

// part = per-slice sums of Aop . Bop^T over the contraction 0 .. Kc (a multiple of
// 64); Aop NT [P][lda] or TN [arows][lda]; Bop [R][ldb] with ldb >= Kc, zero
// between its true width and Kc, or (a.bt, NT only) [brows][ldb] as stored, rows
// from brows on read as zeros.  With b2 a second product of the same kind shares
// the launch (its slice count in *S2); with ride a transpose (compute-dtype source)
// takes one more plane of the grid.
int skinny_jobs(int cd, bool tn, const SkSpec& a, float* part, int* S_out, const SkSpec* b2, float* part2,
                int* S2, hipStream_t s, int kind, const TransposeSpec* ride) {
  SkP2 ps = {};
  int rc = skinny_params(tn, a, part, ps.j[0], S_out);
  if (rc) return rc;
  ps.nx[0] = (uint32_t)ceil_div(a.P, BP);
  ps.ny[0] = (uint32_t)*S_out;
  ps.nj = 1;
  if (b2) {
    if (b2->bt != a.bt) return set_error(QLORA_ERR_UNSUPPORTED, "rank product: jobs of one launch differ in form");
    if ((rc = skinny_params(tn, *b2, part2, ps.j[1], S2))) return rc;
    ps.nx[1] = (uint32_t)ceil_div(b2->P, BP);
    ps.ny[1] = (uint32_t)*S2;
    ps.nj = 2;
  }
  if (ride && ride->src_f32) return set_error(QLORA_ERR_UNSUPPORTED, "rank product: a riding transpose reads cd");
  const bool has_tr = ride && tr_job(*ride, ps.tr);
  const dim3 grid(std::max(ps.nx[0], ps.nx[1]), std::max(ps.ny[0], ps.ny[1]), ps.nj + (has_tr ? 1 : 0));
  ProfScope prof(kind, s);
  const int mode = tn ? 1 : a.bt ? 2 : 0;
  if (cd == CD_BF16) {
    if (mode == 1) k_skinny<CD_BF16, 1><<<grid, dim3(kThreads), 0, s>>>(ps);
    else if (mode == 2) k_skinny<CD_BF16, 2><<<grid, dim3(kThreads), 0, s>>>(ps);
    else k_skinny<CD_BF16, 0><<<grid, dim3(kThreads), 0, s>>>(ps);
  } else {
    if (mode == 1) k_skinny<CD_F16, 1><<<grid, dim3(kThreads), 0, s>>>(ps);
    else if (mode == 2) k_skinny<CD_F16, 2><<<grid, dim3(kThreads), 0, s>>>(ps);
    else k_skinny<CD_F16, 0><<<grid, dim3(kThreads), 0, s>>>(ps);
  }
  return check_launch("k_skinny");
}

// n NT products with the plain Bop form in as few launches as the job table allows
// (projections of a group that read the same x: the products share their Aop tiles
// in the caches and pay the launch once).
int skinny_many(int cd, const SkSpec* specs, float* const* parts, int* S_out, int n, hipStream_t s, int kind) {
  for (int first = 0; first < n; first += kSkJobs) {
    SkP2 ps = {};
    ps.nj = (uint32_t)std::min(kSkJobs, n - first);
    uint32_t gx = 0, gy = 0;
    for (uint32_t i = 0; i < ps.nj; ++i) {
      const SkSpec& sp = specs[first + i];
      if (sp.bt) return set_error(QLORA_ERR_UNSUPPORTED, "rank product: grouped jobs take the plain Bop form");
      int rc = skinny_params(false, sp, parts[first + i], ps.j[i], &S_out[first + i]);
      if (rc) return rc;
      ps.nx[i] = (uint32_t)ceil_div(sp.P, BP);
      ps.ny[i] = (uint32_t)S_out[first + i];
      gx = std::max(gx, ps.nx[i]);
      gy = std::max(gy, ps.ny[i]);
    }
    ProfScope prof(kind, s);
    const dim3 grid(gx, gy, ps.nj);
    if (cd == CD_BF16) k_skinny<CD_BF16, 0><<<grid, dim3(kThreads), 0, s>>>(ps);
    else k_skinny<CD_F16, 0><<<grid, dim3(kThreads), 0, s>>>(ps);
    int rc = check_launch("k_skinny");
    if (rc) return rc;
  }
  return QLORA_OK;
}

int skinny(int cd, bool tn, const void* a, int64_t lda, int64_t arows, const void* b, int64_t ldb, int64_t P,
           int64_t R, int64_t Kc, float* part, int* S_out, hipStream_t s, int kind) {
  SkSpec sp;
  sp.a = a;
  sp.lda = lda;
  sp.arows = arows;
  sp.b = b;
  sp.ldb = ldb;
  sp.P = P;
  sp.R = R;
  sp.Kc = Kc;
  return skinny_jobs(cd, tn, sp, part, S_out, nullptr, nullptr, nullptr, s, kind);
}

namespace {
// The device form of a reduction; false if it does not fit 32-bit indexing.
bool red_job(const SkRed& r, RedJob& j) {
  const int64_t wc = r.wcd ? r.wcd : r.ldcd;  // columns of the cd output written per row
  const int64_t width = (r.outcd && wc > r.R) ? wc : r.R;
  const int64_t rows = ((r.outt || r.side_t) && r.ldt > r.P) ? r.ldt : r.P;
  const int64_t lim = 1LL << 31;
  if (rows * width >= lim || (int64_t)r.S * r.P * BR >= 2 * lim || r.R * r.ldt >= lim || r.P * r.ldcd >= lim ||
      r.S > kRedMaxS)
    return false;
  j.part = r.part;
  j.side = r.side;
  j.out32 = r.out32;
  j.outcd = r.outcd;
  j.outt = r.outt;
  j.side_t = r.side_t;
  j.S = (uint32_t)r.S;
  j.P = (uint32_t)r.P;
  j.R = (uint32_t)r.R;
  j.ldcd = (uint32_t)r.ldcd;
  j.ldt = (uint32_t)r.ldt;
  j.width = (uint32_t)width;
  j.rows = (uint32_t)rows;
  j.nblk = (uint32_t)ceil_div(rows * width, kRedThreads);
  j.sc32 = r.sc32;
  j.sccd = r.sccd;
  j.trans = r.trans ? 1 : 0;
  return true;
}
}  // namespace

// The device form of up to kRedJobs reductions and the workgroups they take.
int make_red_jobs_n(const SkRed* reds, int n, RedJobs& js, int64_t& blocks) {
  js = RedJobs{};
  blocks = 0;
  if (n > kRedJobs) return set_error(QLORA_ERR_UNSUPPORTED, "rank product: %d reductions in one launch", n);
  for (int i = 0; i < n; ++i) {
    if (!red_job(reds[i], js.j[i]))
      return set_error(QLORA_ERR_UNSUPPORTED, "rank product: %lld x %lld too large", (long long)reds[i].P,
                       (long long)reds[i].R);
    blocks += js.j[i].nblk;
  }
  return QLORA_OK;
}

// The device form of one or two reductions and the workgroups they take.
int make_red_jobs(const SkRed& a, const SkRed* b, RedJobs& js, int64_t& blocks) {
  js = RedJobs{};
  if (!red_job(a, js.j[0]) || (b && !red_job(*b, js.j[1])))
    return set_error(QLORA_ERR_UNSUPPORTED, "rank product: %lld x %lld too large", (long long)a.P, (long long)a.R);
  blocks = (int64_t)js.j[0].nblk + (b ? js.j[1].nblk : 0);
  return QLORA_OK;
}

int skinny_reduce_jobs(int cd, const SkRed& a, const SkRed* b, hipStream_t s) {
  RedJobs js;
  int64_t blocks;
  int rc = make_red_jobs(a, b, js, blocks);
  if (rc) return rc;
  if (blocks == 0) return QLORA_OK;
  ProfScope prof(QLORA_K_REDUCE, s);
  if (cd == CD_BF16) k_skreduce<CD_BF16><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(js);
  else k_skreduce<CD_F16><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(js);
  return check_launch("k_skreduce");
}

int skinny_reduce(int cd, const float* part, int S, int64_t P, int64_t R, float sc32, float* out32, bool trans,
                  float sccd, void* outcd, int64_t ldcd, hipStream_t s) {
  SkRed r;
  r.part = part;
  r.S = S;
  r.P = P;
  r.R = R;
  r.sc32 = sc32;
  r.out32 = out32;
  r.trans = trans;
  r.sccd = sccd;
  r.outcd = outcd;
  r.ldcd = ldcd;
  return skinny_reduce_jobs(cd, r, nullptr, s);
}

// dst [cols][ld_dst] = cd(scale * src^T) for small matrices src [rows][ld_src]: one
// launch for the first job and, if given, a second one with the same source type.
int transpose_jobs(int cd, const TransposeSpec& a, const TransposeSpec* b, hipStream_t s) {
  if (b && b->src_f32 != a.src_f32) {
    const int rc = transpose_jobs(cd, a, nullptr, s);
    return rc ? rc : transpose_jobs(cd, *b, nullptr, s);
  }
  TrJobs js = {};
  const TransposeSpec* specs[2] = {&a, b};
  int64_t total = 0;
  for (int k = 0; k < 2; ++k)
    if (specs[k] && tr_job(*specs[k], js.j[k])) total += js.j[k].tiles;
  if (total == 0) return QLORA_OK;
  ProfScope prof(QLORA_K_REDUCE, s);
  const dim3 g((unsigned)total), blk(kThreads);
  if (cd == CD_BF16) {
    if (a.src_f32) k_transpose<CD_BF16, 1><<<g, blk, 0, s>>>(js);
    else k_transpose<CD_BF16, 0><<<g, blk, 0, s>>>(js);
  } else {
    if (a.src_f32) k_transpose<CD_F16, 1><<<g, blk, 0, s>>>(js);
    else k_transpose<CD_F16, 0><<<g, blk, 0, s>>>(js);
  }
  return check_launch("k_transpose");
}

int transpose_small(int cd, const void* src, bool src_f32, int64_t ld_src, int64_t rows, int64_t cols, float scale,
                    void* dst, int64_t ld_dst, hipStream_t s) {
  TransposeSpec t;
  t.src = src;
  t.src_f32 = src_f32;
  t.ld_src = ld_src;
  t.rows = rows;
  t.cols = cols;
  t.scale = scale;
  t.dst = dst;
  t.ld_dst = ld_dst;
  return transpose_jobs(cd, t, nullptr, s);
}

}  // namespace qnf4
