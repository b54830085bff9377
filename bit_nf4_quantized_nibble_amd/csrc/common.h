// common.h -- types and device helpers shared by the gfx950 kernels of
// libqlora_nf4.so.  Internal: not part of the C ABI (include/qlora_nf4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qlora_nf4.h"

namespace qnf4 {

// ----------------------------------------------------------------------------
// Vector types for MFMA operands and 16-byte memory traffic.
// ----------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef _Float16 f16x8_t __attribute__((__vector_size__(16)));
typedef float f32x16_t __attribute__((__vector_size__(64)));
typedef float f32x4_t __attribute__((__vector_size__(16)));
typedef unsigned int u32x4_t __attribute__((__vector_size__(16)));
typedef unsigned int u32x2_t __attribute__((__vector_size__(8)));

enum Cd : int { CD_F32 = QLORA_F32, CD_BF16 = QLORA_BF16, CD_F16 = QLORA_F16 };

// Level table and quantization lookups, computed once on the host (api.hip) and
// passed to kernels by value (kernel arguments land in scalar registers).
struct Nf4Tables {
  float lv[16];      // the 16 NF4 levels, ascending, binary32
  float thr[15];     // thr[j] = smallest binary32 above the midpoint of lv[j], lv[j+1]
  int bucket_base[32];   // code of the lowest value in bucket b of [-1, 1] (width 1/16)
  float bucket_thr[32];  // the one threshold inside bucket b, or +inf
};

// An NF4 weight as the kernels see it.
struct Nf4W {
  const uint8_t* codes;      // [rows * cols / 2]
  const float* absmax;       // [nb] (no double quant)
  const uint8_t* absmax_q;   // [nb] (double quant)
  const float* scale2;       // [ng] (double quant)
  int64_t rows, cols;
  int32_t bs;                // block size (elements)
  int32_t dq;                // double quantization on/off
  int32_t g;                 // blocks per second-level scale
  int32_t bs_shift;          // log2(bs) when bs is a power of two, else -1
  int32_t g_shift;           // log2(g) when g is a power of two, 31 when one group holds
                             // every block (fewer than 2^31), else -1
};

// Byte e of x in one instruction (left to itself the compiler shifts and masks:
// two instructions for bytes 1 and 2).
__device__ __forceinline__ uint32_t byte_of(uint32_t x, int e) {
  if (e == 0) return x & 0xffu;
  if (e == 3) return x >> 24;
  uint32_t r;
  if (e == 1) asm("v_bfe_u32 %0, %1, 8, 8" : "=v"(r) : "v"(x));
  else asm("v_bfe_u32 %0, %1, 16, 8" : "=v"(r) : "v"(x));
  return r;
}

// 8 * byte b of x (b a compile-time constant): one SDWA shift that reads the byte
__device__ __forceinline__ uint32_t byte_x8(uint32_t x, int b) {
  uint32_t r;
  switch (b) {
    case 0: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(x)); break;
    case 1: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(x)); break;
    case 2: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(x)); break;
    default: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(x)); break;
  }
  return r;
}

// Level pair of code byte e in [0, 256): (L[e >> 4], L[e & 15]), the element in the
// high nibble first.  Lanes 0..15 of the wave take the 16 levels from the kernel
// arguments and every lane fetches its two by lane permute (the whole wave must be
// active).
__device__ __forceinline__ float2 level_pair(const Nf4Tables& tab, int e) {
  int lvl = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) asm("v_writelane_b32 %0, %1, %2" : "+v"(lvl) : "s"(tab.lv[i]), "n"(i));
  return make_float2(__int_as_float(__builtin_amdgcn_ds_bpermute((e >> 4) << 2, lvl)),
                     __int_as_float(__builtin_amdgcn_ds_bpermute((e & 15) << 2, lvl)));
}

// Block of flat element e, and second-level group of block b.  Shifts when the
// sizes are powers of two (a 64-bit division costs dozens of instructions).
__device__ __forceinline__ int64_t block_of(const Nf4W& w, int64_t e) {
  return w.bs_shift >= 0 ? (e >> w.bs_shift) : e / w.bs;
}
__device__ __forceinline__ int64_t group_of(const Nf4W& w, int64_t b) {
  return w.g_shift >= 0 ? (b >> w.g_shift) : b / w.g;
}

// fl32(a * b), kept as a binary32 value.  Without the register barrier the
// compiler may fuse the product with a following f16 conversion into one
// mixed-precision FMA that rounds once to f16, skipping the binary32 rounding the
// dequantization defines (w_hat = fl32(L[c] * s_b), then rounded to the dtype).
__device__ __forceinline__ float fl32_mul(float a, float b) {
  float p = a * b;
  asm volatile("" : "+v"(p));
  return p;
}

// Scale of block b: the fp32 absmax, or fl32(q_b * S_group) with double quant.
__device__ __forceinline__ float block_scale(const Nf4W& w, int64_t b) {
  if (w.dq) return (float)w.absmax_q[b] * w.scale2[group_of(w, b)];
  return w.absmax[b];
}

// ----------------------------------------------------------------------------
// Compute-dtype conversions (round to nearest even, as the hardware converts).
// ----------------------------------------------------------------------------
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 values -> one word of two 16-bit values (lo in bits 0..15), each
// rounded to nearest even by a single packed conversion.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack2_f16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
template <int CD>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (CD == CD_BF16) return pack2_bf16(lo, hi);
  else return pack2_f16(lo, hi);
}
template <int CD>
__device__ __forceinline__ uint16_t to_cd16(float v) {
  if constexpr (CD == CD_BF16) return __builtin_bit_cast(uint16_t, (__bf16)v);
  else return __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <int CD>
__device__ __forceinline__ float from_cd16(uint16_t h) {
  if constexpr (CD == CD_BF16) return __uint_as_float((uint32_t)h << 16);
  else return (float)__builtin_bit_cast(_Float16, h);
}
// Load one element of a compute-dtype array as fp32.
template <int CD>
__device__ __forceinline__ float load_cd(const void* p, int64_t i) {
  if constexpr (CD == CD_F32) return ((const float*)p)[i];
  else return from_cd16<CD>(((const uint16_t*)p)[i]);
}
// Store an fp32 value into a compute-dtype array.
template <int CD>
__device__ __forceinline__ void store_cd(void* p, int64_t i, float v) {
  if constexpr (CD == CD_F32) ((float*)p)[i] = v;
  else ((uint16_t*)p)[i] = to_cd16<CD>(v);
}

constexpr int cd_bytes(int cd) { return cd == CD_F32 ? 4 : 2; }

// ----------------------------------------------------------------------------
// Host-side launch plumbing (defined in api.hip).
// ----------------------------------------------------------------------------
const Nf4Tables& host_tables();
int set_error(int status, const char* fmt, ...);
int check_launch(const char* what);

// Opt-in kernel timing (qlora_profile_enable): brackets one launch with a pair of
// events on its stream when recording is on; a no-op otherwise.
void prof_begin(int kind, hipStream_t s, void** token);
void prof_end(void* token, hipStream_t s);
struct ProfScope {
  void* token = nullptr;
  hipStream_t s;
  ProfScope(int kind, hipStream_t st) : s(st) { prof_begin(kind, st, &token); }
  ~ProfScope() { prof_end(token, s); }
};

inline int32_t log2_exact(int64_t v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int32_t s = 0;
  while ((1LL << s) < v) ++s;
  return s;
}

inline Nf4W make_w(const qlora_nf4_t* q) {
  Nf4W w;
  w.codes = q->codes;
  w.absmax = q->absmax;
  w.absmax_q = q->absmax_q;
  w.scale2 = q->absmax_scale2;
  w.rows = q->rows;
  w.cols = q->cols;
  w.bs = q->block_size;
  w.dq = q->double_quant;
  w.g = q->double_quant ? q->dq_group : 1;
  w.bs_shift = log2_exact(w.bs);
  w.g_shift = log2_exact(w.g);
  // One group holds every block: b >> 31 is 0 for every block index b < 2^31.
  const int64_t nb = w.bs > 0 ? q->rows * q->cols / w.bs : 0;
  if (w.g_shift < 0 && nb <= w.g && nb < (1LL << 31)) w.g_shift = 31;
  return w;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Compute units of the current device (cached per device).
int cu_count();

// How the dense 256 x 256 GEMM spreads its tiles over the compute units: the
// first `full` workgroups take whole tiles (whole rounds of one tile per CU); the
// `rem` tiles of an incomplete last round are each cut into `split` contraction
// slices (split 1, rem 0: no cut).
struct DenseSplit {
  int32_t full, rem, split;
};

// Launchers (quant.hip, gemm.hip, gemv.hip, merge.hip, train.hip).  Each returns a qlora_status_t.
int launch_quantize(const float* w, const qlora_nf4_t* q, hipStream_t s);
int launch_dequantize(const qlora_nf4_t* q, int out_dtype, void* out, hipStream_t s);

struct LayerCall {
  Nf4W w;
  int cd;
  int64_t m;          // tokens
  int32_t r;
  float scale;        // alpha / r (or alpha / sqrt(r))
  int32_t flags;      // QLORA_FLAG_* of the call
  const void* x;      // [m, cols]
  const uint8_t* drop_mask;  // [m, cols] keep mask of LoRA dropout, or null (no dropout);
                             // with dropout, scale already holds s / (1 - p)
  const void* lora_a; // [r, cols]
  const void* lora_b; // [rows, r]
  const void* bias;   // [rows] or null
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  int64_t ldy = 0;    // row stride of y in elements (0: rows); the decode GEMV honours it
};

// One reduction of the skinny kernel's per-slice partial sums part [S][P][64] (fp32,
// summed in slice order): out32 = sc32 * sum as [P][R] (or [R][P] with trans);
// outcd [P][ldcd] = cd(sccd * sum) with zero columns R .. ldcd-1; outt [R][ldt] =
// the transpose of that cd value with zero columns P .. ldt-1; side_t [R][ldt] =
// cd(side [P][R])^T with zero columns P .. ldt-1 (a transpose that shares the
// launch).  Null outputs are skipped.
struct SkRed {
  const float* part = nullptr;
  int S = 1;
  int64_t P = 0, R = 0;
  float sc32 = 1.f;
  float* out32 = nullptr;
  bool trans = false;
  float sccd = 1.f;
  void* outcd = nullptr;
  int64_t ldcd = 0;
  int64_t wcd = 0;  // columns of outcd written per row (zeros from R on); 0: ldcd
  void* outt = nullptr;
  int64_t ldt = 0;
  const float* side = nullptr;
  void* side_t = nullptr;
};
// One launch for one or two reductions (b may be null).
int skinny_reduce_jobs(int cd, const SkRed& a, const SkRed* b, hipStream_t s);

// One rank product of the skinny kernel (see skinny() in lora.hip).
struct SkSpec {
  const void* a = nullptr;
  int64_t lda = 0, arows = 0;
  const void* b = nullptr;
  int64_t ldb = 0, P = 0, R = 0, Kc = 0;
  bool bt = false;     // b as stored [brows][ldb] with the R columns contiguous (NT, R % 8 == 0)
  int64_t brows = 0;
};
struct TransposeSpec;
int skinny_jobs(int cd, bool tn, const SkSpec& a, float* part, int* S_out, const SkSpec* b2, float* part2,
                int* S2, hipStream_t s, int kind, const TransposeSpec* ride = nullptr);
// n NT products (plain Bop form), up to four per launch; product i writes parts[i].
int skinny_many(int cd, const SkSpec* specs, float* const* parts, int* S_out, int n, hipStream_t s, int kind);
// The device form of one or two reductions (workgroups of kRedThreads threads, one
// thread per element; job 1 takes the workgroups after job 0's nblk).
constexpr int kRedThreads = 256;
constexpr int kRedBR = 64;  // rank columns of the skinny kernel's partial sums
constexpr int kRedMaxS = 32;  // contraction slices of one rank product (and its reduction)
struct RedJob {
  const float* part;
  const float* side;
  float* out32;
  void* outcd;
  void* outt;
  void* side_t;
  uint32_t S, P, R, ldcd, ldt, width, rows, nblk;
  float sc32, sccd;
  int trans;
};
constexpr int kRedJobs = 4;  // reductions one launch can carry
struct RedJobs {
  RedJob j[kRedJobs];  // job w takes the workgroups after jobs 0 .. w-1 (unused jobs: nblk 0)
};
int make_red_jobs(const SkRed& a, const SkRed* b, RedJobs& js, int64_t& blocks);
// Up to kRedJobs reductions (reds[0 .. n)) for one launch.
int make_red_jobs_n(const SkRed* reds, int n, RedJobs& js, int64_t& blocks);

// dst [cols][ld_dst] = cd(scale * src[rows][ld_src]^T) (src in the compute dtype or
// fp32), columns rows .. ld_dst-1 of dst zero; one launch carries one or two.
struct TransposeSpec {
  const void* src = nullptr;
  bool src_f32 = false;
  int64_t ld_src = 0, rows = 0, cols = 0;
  float scale = 1.f;
  void* dst = nullptr;
  int64_t ld_dst = 0;
  int64_t w_dst = 0;  // columns of dst written per row (zeros from rows on); 0: ld_dst
};
int transpose_jobs(int cd, const TransposeSpec& a, const TransposeSpec* b, hipStream_t s);

int apply_mask(int cd, const void* x, const uint8_t* mask, int64_t n, void* out, hipStream_t s);
int zero_fill(void* p, int64_t bytes, hipStream_t s);
int rank_add_masked(int cd, void* dx, const uint8_t* mask, const void* dt, int64_t ld_dt, const void* a, int32_t r,
                    int64_t M, int64_t K, hipStream_t s);
size_t fwd_workspace_bytes(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd, int32_t flags);
size_t bwd_workspace_bytes(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd, int32_t flags);
// red: a reduction that rides on the same launch (its workgroups come ahead of the
// dequantize ones), or null.
// W~ into out: [rows, cols], or transposed [cols][ldo] (ldo = 0: rows) for the dX GEMM.
int dequant_into(const Nf4W& w, int cd, void* out, bool transposed, hipStream_t s, const SkRed* red = nullptr,
                 int64_t ldo = 0);
// The group forward's weights in one launch: W~_i into outs[i], reds[i] riding on it.
int dequant_group_into(const Nf4W* ws, int g, int cd, void* const* outs, const SkRed* reds, hipStream_t s);
int launch_forward(const LayerCall& c, void* y, float* t_save);
// Whether launch_forward takes the decode GEMV for this call (which writes y with
// row stride c.ldy; the other forwards write [m, rows]).
bool gemv_route(const LayerCall& c);
size_t cached_fwd_workspace_bytes(int64_t m, int64_t rows, int64_t cols, int32_t r, int cd);
int launch_forward_cached(const LayerCall& c, const void* wd, void* y, float* t_save);
int launch_backward(const LayerCall& c, const void* dy, const float* t_saved, void* dx,
                    float* d_a, float* d_b);

// The tiled kernels' entry points shared across files (gemm256.hip, lora.hip) and
// the layouts they take (gemm.hip, group.hip).
int fused256_forward(const LayerCall& c, const void* t_cd, int64_t r_pad, void* y, const DenseSplit& sp,
                     void* split_ws);
int fused256_dx(const LayerCall& c, const void* dy, const void* dt_cd, int64_t r_pad, void* dx, const DenseSplit& sp,
                void* split_ws);
bool fused256_ok(const LayerCall& c, bool dx);
bool dense256_ok(const LayerCall& c, bool dx);
int dense256_forward(const LayerCall& c, const void* wd, const void* t_cd, int64_t r_pad, void* y,
                     const DenseSplit& sp, void* split_ws);
int dense256_dx(const LayerCall& c, const void* dy, const void* wdt, const void* dt_cd, int64_t r_pad, void* dx,
                const DenseSplit& sp, void* split_ws, const void* a_t);
DenseSplit dense_split(int64_t m, int64_t nb, int64_t k1, bool fused = false);
size_t dense_split_bytes(const DenseSplit& sp);
// the rank-r products on the skinny MFMA kernel (lora.hip)
bool skinny_ok(int cd, int64_t r);
size_t skinny_part_bytes(int64_t P, int64_t Kc);
int skinny(int cd, bool tn, const void* a, int64_t lda, int64_t arows, const void* b, int64_t ldb, int64_t P,
           int64_t R, int64_t Kc, float* part, int* S_out, hipStream_t s, int kind);
int skinny_reduce(int cd, const float* part, int S, int64_t P, int64_t R, float sc32, float* out32, bool trans,
                  float sccd, void* outcd, int64_t ldcd, hipStream_t s);
int transpose_small(int cd, const void* src, bool src_f32, int64_t ld_src, int64_t rows, int64_t cols, float scale,
                    void* dst, int64_t ld_dst, hipStream_t s);
// Layouts the tiled kernels take: block a multiple of 32 that divides cols, cols a
// multiple of 64 (everything else runs on the generic tile engine).
inline bool fast_layout(const Nf4W& w) { return w.bs % 32 == 0 && w.cols % 64 == 0 && w.cols % w.bs == 0; }

// Projections that read the same input, called as one group (group.hip).
constexpr int kGroupMax = QLORA_GROUP_MAX;
struct GroupCall {
  int g = 0;
  LayerCall c[kGroupMax];       // projection i as a single-layer call (its workspace set per use)
  int64_t off[kGroupMax + 1];   // first column of projection i in the concatenated output; off[g] = N
  int64_t toff[kGroupMax + 1];  // first column of its slice of the concatenated rank operand
  int64_t N = 0, R8 = 0, RP = 0;  // sum of the rows; of the ranks each rounded up to 8; R8 rounded up to 64
};
size_t group_workspace_bytes(int op, const GroupCall& gc);
int launch_forward_group(const GroupCall& gc, const void* bias, void* y, float* const* t_save, void* ws,
                         hipStream_t s);
int launch_backward_group(const GroupCall& gc, const void* dy, const float* const* t_saved, void* dx,
                          float* const* d_a, float* const* d_b, void* ws, hipStream_t s);
int launch_merge(const Nf4W& w, const void* a, const void* b, int32_t r, float s, int cd, void* out,
                 hipStream_t st);
int launch_mse(const void* y, const void* t, int64_t n, int cd, float* loss, void* dy, float* partial,
               hipStream_t s);
int launch_adamw(float* theta, const float* g, float* m, float* v, int64_t n, const qlora_adamw_t& o, int32_t step,
                 void* theta_cd, int cd, hipStream_t s);
size_t stack_workspace_bytes(const qlora_stack_layer_t* layers, int32_t L, int64_t m, int32_t r, int cd,
                             int32_t flags);
int launch_stack_step(const qlora_stack_layer_t* layers, int32_t L, const void* x, int64_t m, const void* target,
                      int32_t r, float scale, int32_t flags, int cd, const qlora_adamw_t& opt, int32_t step,
                      float* loss, void* ws, hipStream_t s);

}  // namespace qnf4
