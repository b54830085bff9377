// quant.hip -- NF4 quantize (+ double quantization of the scales) and dequantize
// for gfx950.  Both are HBM streams; the arithmetic is arranged so that every
// code, scale and dequantized value is bit-identical to the definition:
//
//   qlora-rs README, "Honest capability matrix": per-block absmax scales, NF4
//   pack/unpack, double quant to u8 with a scale-of-scales that replaces the
//   resident fp32 scales; "NF4 Quantization": the 16 levels.
//   "LoRA and QLoRA, mathematically", "NF4: quantizing the frozen base": levels at
//   normal quantiles; each weight takes the nearest level of w / absmax.
//
// Quantize layout: each lane owns 8 consecutive fp32 weights (two 16-byte loads)
// and produces one 32-bit word of packed codes.  A block of BS weights spans
// BS/8 adjacent lanes, whose absmax is combined with lane shuffles.  One
// workgroup walks one double-quant group (or a 16384-element span without DQ),
// so the group max and the u8 encoding need no second pass over HBM.
#include "common.h"
#include "reduce_dev.h"

namespace qnf4 {

namespace {

constexpr int kThreads = 256;

// Nearest-level code of a normalised value x in [-1, 1]: a 32-bucket table over
// [-1, 1] holds, per bucket, the code of its lowest value and the single
// threshold inside it (the host checks that no bucket holds two thresholds and
// that no threshold sits within rounding distance of a bucket edge).
__device__ __forceinline__ uint32_t nearest_code(float x, const int* __restrict__ base,
                                                 const float* __restrict__ thr) {
  float u = fmaf(x, 16.0f, 16.0f);
  int b = (int)fminf(fmaxf(u, 0.0f), 31.0f);
  return (uint32_t)(base[b] + (x >= thr[b] ? 1 : 0));
}

// x = fl32(w / a) by Markstein's correction: r = RN(1/a) once per block, then
// y = RN(w r) is within an ulp of w / a and RN(y + RN(w - a y) r) = RN(w / a).
// Blocks of very small or very large magnitude are rescaled by an exact power of
// two first so that 1/a stays a normal number.  The caller passes the block's
// sc, as = a sc and rcp = RN(1 / as) (see block_recip); a == 0 gives x = 0.
struct BlockRecip {
  float sc, as, rcp;
};
__device__ __forceinline__ BlockRecip block_recip(float a) {
  BlockRecip r;
  r.sc = (a < 0x1p-64f) ? 0x1p64f : ((a > 0x1p64f) ? 0x1p-64f : 1.0f);
  r.as = a * r.sc;
  r.rcp = 1.0f / r.as;
  return r;
}
__device__ __forceinline__ float normalize(float w, float a, const BlockRecip& r) {
  const float ws = w * r.sc;
  const float y = ws * r.rcp;
  const float rem = fmaf(-r.as, y, ws);
  const float x = fmaf(rem, r.rcp, y);
  return a == 0.0f ? 0.0f : x;
}

template <int BS>
__global__ __launch_bounds__(kThreads) void k_quantize(const float* __restrict__ w, int64_t n,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ absmax,
                                                       uint8_t* __restrict__ absmax_q,
                                                       float* __restrict__ scale2,
                                                       int blocks_per_wg, int dq, int64_t dq_group,
                                                       Nf4Tables tab) {
  constexpr int LPB = BS / 8;  // lanes per block
  __shared__ int s_base[32];
  __shared__ float s_thr[32];
  __shared__ float s_amax[4096];  // block scales of this group (double quant only)
  __shared__ float s_red[kThreads / 64];
  __shared__ uint32_t s_gmax[2];  // dq == 2: bits of the maxima of the (at most two) groups met here

  const int tid = threadIdx.x;
  if (tid < 32) {
    s_base[tid] = tab.bucket_base[tid];
    s_thr[tid] = tab.bucket_thr[tid];
  }
  if (tid < 2) s_gmax[tid] = 0u;
  __syncthreads();

  const int64_t nb = n / BS;
  const int64_t blk0 = (int64_t)blockIdx.x * blocks_per_wg;
  const int64_t nblk = (blk0 + blocks_per_wg <= nb) ? blocks_per_wg : nb - blk0;
  const int64_t e_begin = blk0 * BS;
  const int64_t e_count = nblk * BS;
  // dq == 2 (groups larger than a workgroup's span): the span meets group g_first and
  // possibly the next one, starting at local block `split`.
  const int64_t g_first = dq == 2 ? blk0 / dq_group : 0;
  const int64_t split = dq == 2 ? (g_first + 1) * dq_group - blk0 : 0;

  for (int64_t e = (int64_t)tid * 8; e < e_count; e += (int64_t)kThreads * 8) {
    const f32x4_t* src = (const f32x4_t*)(w + e_begin + e);
    f32x4_t v0 = __builtin_nontemporal_load(src);
    f32x4_t v1 = __builtin_nontemporal_load(src + 1);
    float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
    for (int off = 1; off < LPB; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));

    const int64_t blk_local = e / BS;
    if ((tid % LPB) == 0) {
      if (dq == 2)
        atomicMax(&s_gmax[blk_local >= split ? 1 : 0], __float_as_uint(a));  // a >= 0: bits order as values
      else if (dq)
        s_amax[blk_local] = a;
      else
        absmax[blk0 + blk_local] = a;
    }

    const BlockRecip br = block_recip(a);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = nearest_code(normalize(v[i], a, br), s_base, s_thr);
      // element 2k -> high nibble of byte k
      word |= c << ((i >> 1) * 8 + ((i & 1) ? 0 : 4));
    }
    *(uint32_t*)(codes + (e_begin + e) / 2) = word;
  }

  if (!dq) return;
  __syncthreads();
  if (dq == 2) {  // fold this span's group maxima into the global ones (k_dq_large_finish divides)
    if (tid == 0) atomicMax((uint32_t*)scale2 + g_first, s_gmax[0]);
    if (tid == 1 && split < nblk) atomicMax((uint32_t*)scale2 + g_first + 1, s_gmax[1]);
    return;
  }
  // Group max of the block scales, then S = fl32(max / 255) and
  // q_b = round-half-even(a_b / S) (exact: the fp64 quotient of two binary32
  // values never rounds onto a half-integer it is not equal to).
  float c = 0.0f;
  for (int64_t b = tid; b < nblk; b += kThreads) c = fmaxf(c, s_amax[b]);
  for (int off = 32; off >= 1; off >>= 1) c = fmaxf(c, __shfl_xor(c, off, 64));
  if ((tid & 63) == 0) s_red[tid >> 6] = c;
  __syncthreads();
  c = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float S = c / 255.0f;
  if (tid == 0) scale2[blockIdx.x] = S;
  for (int64_t b = tid; b < nblk; b += kThreads) {
    double q = 0.0;
    if (S > 0.0f) {
      q = __builtin_rint((double)s_amax[b] / (double)S);
      q = q < 0.0 ? 0.0 : (q > 255.0 ? 255.0 : q);
    }
    absmax_q[blk0 + b] = (uint8_t)q;
  }
}

// Double quantization with groups larger than 4096 blocks (up to one group for the
// whole tensor): the group maxima need a pass over every block first.  k_quantize
// (dq == 2) writes the codes and folds the block absmaxes into scale2[g] as a
// maximum (atomic max on the bits of non-negative floats, from zero); this pass
// re-reads W, recomputes each block's absmax and encodes q_b = round-half-even(a_b / S)
// with S = fl32(max / 255); k_dq_large_finish then stores S itself.  Same values as
// the one-pass kernel.
__global__ __launch_bounds__(kThreads) void k_fill_zero(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

template <int BS>
__global__ __launch_bounds__(kThreads) void k_dq_large_q(const float* __restrict__ w, int64_t n,
                                                         uint8_t* __restrict__ absmax_q,
                                                         const float* __restrict__ gmax, int blocks_per_wg,
                                                         int64_t dq_group) {
  constexpr int LPB = BS / 8;
  const int tid = threadIdx.x;
  const int64_t nb = n / BS;
  const int64_t blk0 = (int64_t)blockIdx.x * blocks_per_wg;
  const int64_t nblk = (blk0 + blocks_per_wg <= nb) ? blocks_per_wg : nb - blk0;
  const int64_t g_first = blk0 / dq_group, split = (g_first + 1) * dq_group - blk0;
  const float S0 = gmax[g_first] / 255.0f;
  const float S1 = split < nblk ? gmax[g_first + 1] / 255.0f : 0.0f;
  for (int64_t e = (int64_t)tid * 8; e < nblk * BS; e += (int64_t)kThreads * 8) {
    const f32x4_t* src = (const f32x4_t*)(w + blk0 * BS + e);
    const f32x4_t v0 = __builtin_nontemporal_load(src);
    const f32x4_t v1 = __builtin_nontemporal_load(src + 1);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) a = fmaxf(a, fmaxf(fabsf(v0[i]), fabsf(v1[i])));
#pragma unroll
    for (int off = 1; off < LPB; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    const int64_t b = e / BS;
    if ((tid % LPB) == 0) {
      const float S = b >= split ? S1 : S0;
      double q = 0.0;
      if (S > 0.0f) {
        q = __builtin_rint((double)a / (double)S);
        q = q < 0.0 ? 0.0 : (q > 255.0 ? 255.0 : q);
      }
      absmax_q[blk0 + b] = (uint8_t)q;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_dq_large_finish(float* __restrict__ scale2, int64_t ng) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < ng) scale2[i] = scale2[i] / 255.0f;
}

// Dequantize: each lane decodes 32 consecutive weights (16 bytes of codes).
template <int OUT>
__global__ __launch_bounds__(kThreads) void k_dequantize(Nf4W q, int64_t n, void* __restrict__ out,
                                                         Nf4Tables tab) {
  __shared__ float s_lv[16];
  if (threadIdx.x < 16) s_lv[threadIdx.x] = tab.lv[threadIdx.x];
  __syncthreads();
  const int64_t e0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 32;
  if (e0 >= n) return;
  const bool full = (e0 + 32 <= n);
  uint32_t words[4];
  if (full) {
    u32x4_t v = *(const u32x4_t*)(q.codes + e0 / 2);
    words[0] = v[0]; words[1] = v[1]; words[2] = v[2]; words[3] = v[3];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      words[i] = (e0 + 8 * i < n) ? *(const uint32_t*)(q.codes + e0 / 2 + 4 * i) : 0u;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t e = e0 + 8 * i;
    if (e >= n) break;
    const float s = block_scale(q, block_of(q, e));
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // byte j/2 of the word; element 2k sits in the high nibble
      uint32_t c = (words[i] >> ((j >> 1) * 8 + ((j & 1) ? 0 : 4))) & 15u;
      f[j] = fl32_mul(s_lv[c], s);
    }
    if constexpr (OUT == CD_F32) {
      float4* o = (float4*)((float*)out + e);
      o[0] = make_float4(f[0], f[1], f[2], f[3]);
      o[1] = make_float4(f[4], f[5], f[6], f[7]);
    } else {
      u32x4_t o;
      o[0] = pack2<OUT>(f[0], f[1]);
      o[1] = pack2<OUT>(f[2], f[3]);
      o[2] = pack2<OUT>(f[4], f[5]);
      o[3] = pack2<OUT>(f[6], f[7]);
      *(u32x4_t*)((uint16_t*)out + e) = o;
    }
  }
}

// Any even block size (the kernels above take powers of two from 8 to 512): one
// wavefront per block.  Lane l reads the weight pairs (2j, 2j + 1) with j = l + 64 i
// of its block, the block absmax is combined across the wavefront, and lane l
// writes the code bytes j it read.  Without double quantization lane 0 stores the
// absmax; with it, lane 0 folds the block absmax into scale2[group] as a maximum
// (atomic max on the bits of non-negative floats, from zero) and k_dq_any_q
// encodes the u8 scales in a second pass.  Same values as the one-pass kernels.
constexpr int kAnyBlocksPerWg = kThreads / 64;

__device__ __forceinline__ float block_absmax_wave(const float* __restrict__ wb, int64_t bs, int lane) {
  float a = 0.0f;
  for (int64_t j = lane; 2 * j < bs; j += 64) {
    const float2 v = *(const float2*)(wb + 2 * j);
    a = fmaxf(a, fmaxf(fabsf(v.x), fabsf(v.y)));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  return a;
}

__global__ __launch_bounds__(kThreads) void k_quantize_any(const float* __restrict__ w, int64_t nb, int64_t bs,
                                                           uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                           float* __restrict__ gmax, int64_t dq_group,
                                                           Nf4Tables tab) {
  __shared__ int s_base[32];
  __shared__ float s_thr[32];
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 32) {
    s_base[tid] = tab.bucket_base[tid];
    s_thr[tid] = tab.bucket_thr[tid];
  }
  __syncthreads();
  const int64_t b = (int64_t)blockIdx.x * kAnyBlocksPerWg + (tid >> 6);
  if (b >= nb) return;
  const float* wb = w + b * bs;
  const float a = block_absmax_wave(wb, bs, lane);
  if (lane == 0) {
    if (gmax) atomicMax((uint32_t*)gmax + b / dq_group, __float_as_uint(a));
    else absmax[b] = a;
  }
  const BlockRecip br = block_recip(a);
  uint8_t* cb = codes + b * (bs / 2);
  for (int64_t j = lane; 2 * j < bs; j += 64) {
    const float2 v = *(const float2*)(wb + 2 * j);
    const uint32_t hi = nearest_code(normalize(v.x, a, br), s_base, s_thr);
    const uint32_t lo = nearest_code(normalize(v.y, a, br), s_base, s_thr);
    cb[j] = (uint8_t)((hi << 4) | lo);  // element 2j in the high nibble
  }
}

// Second pass of double quantization for any block size: q_b = round-half-even(a_b / S)
// with S = fl32(max / 255) of the block's group (gmax still holds the maximum).
__global__ __launch_bounds__(kThreads) void k_dq_any_q(const float* __restrict__ w, int64_t nb, int64_t bs,
                                                       uint8_t* __restrict__ absmax_q,
                                                       const float* __restrict__ gmax, int64_t dq_group) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t b = (int64_t)blockIdx.x * kAnyBlocksPerWg + (tid >> 6);
  if (b >= nb) return;
  const float a = block_absmax_wave(w + b * bs, bs, lane);
  if (lane == 0) {
    const float S = gmax[b / dq_group] / 255.0f;
    double q = 0.0;
    if (S > 0.0f) {
      q = __builtin_rint((double)a / (double)S);
      q = q < 0.0 ? 0.0 : (q > 255.0 ? 255.0 : q);
    }
    absmax_q[b] = (uint8_t)q;
  }
}

// Dequantize for any even block size and any n: thread i decodes code byte i
// (elements 2i and 2i + 1, which share a block because blocks start at even
// offsets) and stores the pair.
template <int OUT>
__global__ __launch_bounds__(kThreads) void k_dequantize_any(Nf4W q, int64_t n, void* __restrict__ out,
                                                             Nf4Tables tab) {
  __shared__ float s_lv[16];
  if (threadIdx.x < 16) s_lv[threadIdx.x] = tab.lv[threadIdx.x];
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (2 * i >= n) return;
  const uint32_t byte = q.codes[i];
  const float s = block_scale(q, block_of(q, 2 * i));
  const float f0 = fl32_mul(s_lv[byte >> 4], s), f1 = fl32_mul(s_lv[byte & 15u], s);
  if constexpr (OUT == CD_F32) *(float2*)((float*)out + 2 * i) = make_float2(f0, f1);
  else *(uint32_t*)((uint16_t*)out + 2 * i) = pack2<OUT>(f0, f1);
}

}  // namespace

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* ptr, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)ptr, (short)0, (int)bytes, 0x00020000);
}
// Out-of-range offset: the top bit puts it past every buffer (all are < 2 GiB).
__device__ __forceinline__ uint32_t oob_unless(bool ok, uint32_t off) { return off | ((uint32_t)(!ok) << 31); }

// Raw words of the block scale of element e (converted at use, so that every load of
// a thread leaves before any is waited on; a read past a buffer returns 0).
struct ScaleRsrc {
  rsrc_t q, s2;
};
// With double quantization the group size is a power of two (g_shift) or one group
// holds every block (g_shift 31): ceil(nb / g) = ((nb - 1) >> g_shift) + 1.
template <int DQ>
__device__ __forceinline__ ScaleRsrc make_scale_rsrc(const Nf4W& w, int64_t nb) {
  ScaleRsrc r;
  r.q = DQ ? make_rsrc(w.absmax_q, nb) : make_rsrc(w.absmax, nb * 4);
  r.s2 = DQ ? make_rsrc(w.scale2, (((nb - 1) >> w.g_shift) + 1) * 4) : r.q;
  return r;
}
template <int DQ>
__device__ __forceinline__ void load_scale(const ScaleRsrc& r, const Nf4W& w, uint32_t blk, uint32_t& qa,
                                           uint32_t& s2) {
  if constexpr (DQ) {
    qa = __builtin_amdgcn_raw_buffer_load_b8(r.q, (int)blk, 0, 0);
    s2 = __builtin_amdgcn_raw_buffer_load_b32(r.s2, (int)((blk >> w.g_shift) * 4), 0, 0);
  } else {
    qa = __builtin_amdgcn_raw_buffer_load_b32(r.q, (int)(blk * 4), 0, 0);
    s2 = 0u;
  }
}
// s_b: a_b, or fl32(q_b * S) with double quantization.
template <int DQ>
__device__ __forceinline__ float scale_of(uint32_t qa, uint32_t s2) {
  if constexpr (DQ) return fl32_mul((float)qa, __uint_as_float(s2));
  else return __uint_as_float(qa);
}

// Dequantize (block size a power of two >= 8, n a multiple of 8, codes under 2 GiB;
// with double quantization a power-of-two group or a single group): lane l of a
// workgroup handles the 8-element chunks l + 256 j (j < 8) of the workgroup's
// 16384 elements, so each load (4 bytes of codes per lane) and each 16-byte store
// instruction covers contiguous memory across the wave.  All 8 chunks' codes and
// scales are requested before the first is used; chunks past the end read past the
// buffers (zeros) and store nothing.  Same values as k_dequantize.
// The first gridDim.x - nmain workgroups run the reductions `red` instead (see
// reduce_dev.h): placed ahead of the dequantize, their load latency overlaps it
// instead of trailing the launch.  One launch can dequantize up to kDqParts
// weights (the projections of a group, each into its own output): the workgroups
// after the reductions take part 0's chunks, then part 1's, and so on.
constexpr int kDqParts = 4;
struct DqParts {
  Nf4W w[kDqParts];
  void* out[kDqParts];
  int64_t n[kDqParts];      // elements of part i
  uint32_t end[kDqParts];   // workgroups of parts 0 .. i
  int32_t np;
};
template <int OUT, int DQ>
__global__ __launch_bounds__(kThreads) void k_dequant_chunks(DqParts ps, Nf4Tables tab, RedJobs red, uint32_t nmain) {
  const uint32_t nred = gridDim.x - nmain;
  if (blockIdx.x < nred) {
    skreduce_block<OUT == CD_F16 ? CD_F16 : CD_BF16>(red, blockIdx.x);
    return;
  }
  uint32_t bx = blockIdx.x - nred;
  int pi = 0;  // the part (uniform across the workgroup)
#pragma unroll
  for (int k = 0; k < kDqParts - 1; ++k)
    if (pi == k && k + 1 < ps.np && bx >= ps.end[k]) pi = k + 1;
  if (pi > 0) bx -= ps.end[pi - 1];
  const Nf4W& q = ps.w[pi];
  const int64_t n = ps.n[pi];
  void* __restrict__ out = ps.out[pi];
  __shared__ float s_lv[16];
  if (threadIdx.x < 16) s_lv[threadIdx.x] = tab.lv[threadIdx.x];
  const rsrc_t rc = make_rsrc(q.codes, n / 2);
  const ScaleRsrc rs = make_scale_rsrc<DQ>(q, n >> q.bs_shift);
  const int64_t ch0 = (int64_t)bx * (kThreads * 8) + threadIdx.x;
  const int64_t nch = n / 8;
  uint32_t cw[8], qa[8], s2[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t ch = ch0 + kThreads * j;
    cw[j] = __builtin_amdgcn_raw_buffer_load_b32(rc, (int)(uint32_t)(ch * 4), 0, 0);
    load_scale<DQ>(rs, q, (uint32_t)((ch * 8) >> q.bs_shift), qa[j], s2[j]);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t ch = ch0 + kThreads * j;
    if (ch >= nch) break;
    const float sc = scale_of<DQ>(qa[j], s2[j]);
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)  // byte i / 2; element 2k in the high nibble
      f[i] = fl32_mul(s_lv[(cw[j] >> ((i >> 1) * 8 + ((i & 1) ? 0 : 4))) & 15u], sc);
    if constexpr (OUT == CD_F32) {
      float4* o = (float4*)((float*)out + ch * 8);
      o[0] = make_float4(f[0], f[1], f[2], f[3]);
      o[1] = make_float4(f[4], f[5], f[6], f[7]);
    } else {
      u32x4_t o;
      o[0] = pack2<OUT>(f[0], f[1]);
      o[1] = pack2<OUT>(f[2], f[3]);
      o[2] = pack2<OUT>(f[4], f[5]);
      o[3] = pack2<OUT>(f[6], f[7]);
      *(u32x4_t*)((uint16_t*)out + ch * 8) = o;
    }
  }
}

// Transposed dequantize for the dequantize-then-GEMM backward: out [cols, rows] =
// RNE_cd(fl32(L[c] * s_b))^T, the same values as k_dequantize.  One workgroup per
// 64 x 64 T slab of W (T tiles of 64 x 64 along its columns).  Each lane requests
// the codes (16 consecutive codes of one W row per tile) and block scales of all
// T tiles before it decodes the first, decodes them into LDS tiles [k][n], and
// after one barrier writes 16 elements of one output row per tile.
// Tile rows are 128 bytes; 16-byte chunk c of row k sits at c ^ 2 ((k >> 4) & 3),
// so the four column groups of a 2-byte write instruction land on distinct banks.
// rows and cols are multiples of 64, the block size a power of two >= 8 (with
// double quantization a power-of-two group or one group), codes under 2 GiB
// (checked by the caller).  Tiles past the last column load the first codes
// (unused) and write nothing.
// The first gridDim.x - nmain workgroups run the reduction `red` (see
// reduce_dev.h), ahead of the dequantize so that their latency overlaps it; the
// workgroup b = blockIdx.x - (gridDim.x - nmain) after them takes slab (b % gx, b / gx).
template <int OUT, int DQ, int T>
__global__ __launch_bounds__(kThreads) void k_dequantize_t(Nf4W q, void* __restrict__ out, int64_t ldo, Nf4Tables tab,
                                                           RedJobs red, uint32_t gx, uint32_t nmain) {
  const uint32_t nred = gridDim.x - nmain;
  if (blockIdx.x < nred) {
    skreduce_block<OUT>(red, blockIdx.x);
    return;
  }
  const uint32_t bx = blockIdx.x - nred;
  __shared__ float s_lv[16];
  __shared__ __attribute__((aligned(16))) uint16_t tile[T][64 * 64];  // [k][n] per tile
  const int tid = threadIdx.x;
  if (tid < 16) s_lv[tid] = tab.lv[tid];
  const int64_t n = q.rows * q.cols;
  const rsrc_t rc = make_rsrc(q.codes, n / 2);
  const ScaleRsrc rs = make_scale_rsrc<DQ>(q, n >> q.bs_shift);
  const int64_t n0 = (int64_t)(bx / gx) * 64, kb = (int64_t)(bx % gx) * (64 * T);
  const int nr = tid >> 2, kc = (tid & 3) * 16;
  uint32_t cw[T][2], qa[T][2], s2[T][2];
#pragma unroll
  for (int u = 0; u < T; ++u) {
    const bool ok = kb + 64 * u < q.cols;  // the same for the whole workgroup
    const int64_t e0 = (n0 + nr) * q.cols + kb + 64 * u + kc;
    const uint32_t co = ok ? (uint32_t)(e0 / 2) : 0u;
    cw[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rc, (int)co, 0, 0);
    cw[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rc, (int)(co + 4), 0, 0);
    const uint32_t b0 = ok ? (uint32_t)(e0 >> q.bs_shift) : 0u;
    const uint32_t b1 = ok ? (uint32_t)((e0 + 8) >> q.bs_shift) : 0u;
    load_scale<DQ>(rs, q, b0, qa[u][0], s2[u][0]);
    load_scale<DQ>(rs, q, b1, qa[u][1], s2[u][1]);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < T; ++u) {
    if (kb + 64 * u >= q.cols) break;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t word = cw[u][hf];
      const float s = scale_of<DQ>(qa[u][hf], s2[u][hf]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t c = (word >> ((j >> 1) * 8 + ((j & 1) ? 0 : 4))) & 15u;
        const int k = kc + 8 * hf + j;
        tile[u][k * 64 + ((((nr >> 3) ^ (2 * ((k >> 4) & 3)))) << 3) + (nr & 7)] = to_cd16<OUT>(fl32_mul(s_lv[c], s));
      }
    }
  }
  __syncthreads();
  // lanes 4 kr .. 4 kr + 3 write output row kr: chunks 0..3 (64 contiguous bytes)
  // with one instruction, chunks 4..7 with the next
  const int kr = tid >> 2, ca = tid & 3, sw = 2 * ((kr >> 4) & 3);
#pragma unroll
  for (int u = 0; u < T; ++u) {
    if (kb + 64 * u >= q.cols) break;
    const u32x4_t v0 = *(const u32x4_t*)&tile[u][kr * 64 + ((ca ^ sw) << 3)];
    const u32x4_t v1 = *(const u32x4_t*)&tile[u][kr * 64 + (((ca + 4) ^ sw) << 3)];
    uint16_t* o = (uint16_t*)out + (kb + 64 * u + kr) * ldo + n0 + 8 * ca;
    *(u32x4_t*)o = v0;
    *(u32x4_t*)(o + 32) = v1;
  }
}

// Four-tile form of the transposed dequantize (64 x 256 slab, block size a power of
// two >= 32): lane (nr = tid / 4, ca = tid % 4) loads the codes of row n0 + nr at
// contraction kb + 128 h + 32 ca .. + 32 (h = 0, 1) with one 16-byte load each, so
// one load instruction reads 64 contiguous bytes of 16 rows; each 32-code run lies
// in one block (one scale).  A code byte decodes to its two elements through the
// level-pair table (one LDS read, two fl32 products, one packed rounding) and the
// two 16-bit halves go to rows k and k + 1 of tile 2 h + ca / 2 ([k][n], the same
// swizzle as k_dequantize_t).  Tiles are TS4 bytes apart (8 KiB + 128), so the
// four column groups of a store instruction land on distinct banks.  Same values
// as k_dequantize.
constexpr int TS4 = 64 * 64 * 2 + 128;
template <int OUT, int DQ>
__global__ __launch_bounds__(kThreads) void k_dequantize_t4(Nf4W q, void* __restrict__ out, int64_t ldo,
                                                            Nf4Tables tab, RedJobs red, uint32_t gx, uint32_t nmain) {
  const uint32_t nred = gridDim.x - nmain;  // the reduction's workgroups come first
  if (blockIdx.x < nred) {
    skreduce_block<OUT>(red, blockIdx.x);
    return;
  }
  const uint32_t bx = blockIdx.x - nred;
  __shared__ __attribute__((aligned(16))) float2 s_pair[256];
  __shared__ __attribute__((aligned(16))) unsigned char tile[4 * TS4];
  const int tid = threadIdx.x;
  const int64_t n = q.rows * q.cols;
  const rsrc_t rc = make_rsrc(q.codes, n / 2);
  const ScaleRsrc rs = make_scale_rsrc<DQ>(q, n >> q.bs_shift);
  const int64_t n0 = (int64_t)(bx / gx) * 64, kb = (int64_t)(bx % gx) * 256;
  const int nr = tid >> 2, ca = tid & 3;
  u32x4_t cw[2];
  uint32_t qa[2], s2[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t k = kb + 128 * h + 32 * ca;
    const bool ok = k < q.cols;  // cols % 64 == 0: a 32-code run is all inside or all outside
    const int64_t e0 = (n0 + nr) * q.cols + k;
    cw[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                            rc, (int)oob_unless(ok, (uint32_t)(e0 / 2)), 0, 0));
    load_scale<DQ>(rs, q, ok ? (uint32_t)(e0 >> q.bs_shift) : 0u, qa[h], s2[h]);
  }
  s_pair[tid] = level_pair(tab, tid);
  __syncthreads();
  // byte address of element (k, n0 + nr) in a tile, less k * 128, for (k >> 4) & 3 = 2 (ca & 1) + v
  const int odd = ca & 1;
  int base[2];
#pragma unroll
  for (int v = 0; v < 2; ++v)
    base[v] = 4096 * odd + 16 * ((nr >> 3) ^ (2 * ((2 * odd + v) & 3))) + 2 * (nr & 7);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float sc = scale_of<DQ>(qa[h], s2[h]);
    unsigned char* tb = tile + (2 * h + (ca >> 1)) * TS4;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float2 lv[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) lv[b] = *(const float2*)((const char*)s_pair + byte_x8(cw[h][w], b));
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        // byte 4 w + b: elements k = 32 (ca & 1) + 8 w + 2 b (high nibble) and k + 1
        const uint32_t pk = pack2<OUT>(fl32_mul(lv[b].x, sc), fl32_mul(lv[b].y, sc));
        unsigned char* at = tb + base[w >> 1] + (8 * w + 2 * b) * 128;
        *(uint16_t*)at = (uint16_t)pk;
        *(uint16_t*)(at + 128) = (uint16_t)(pk >> 16);
      }
    }
  }
  __syncthreads();
  // lanes 4 kr .. 4 kr + 3 write output row kr of each tile: chunks 0..3 (64
  // contiguous bytes) with one instruction, chunks 4..7 with the next
  const int kr = tid >> 2, sw = 2 * ((kr >> 4) & 3);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (kb + 64 * u >= q.cols) break;
    const unsigned char* row = tile + u * TS4 + kr * 128;
    const u32x4_t v0 = *(const u32x4_t*)(row + 16 * (ca ^ sw));
    const u32x4_t v1 = *(const u32x4_t*)(row + 16 * ((ca + 4) ^ sw));
    uint16_t* o = (uint16_t*)out + (kb + 64 * u + kr) * ldo + n0 + 8 * ca;
    *(u32x4_t*)o = v0;
    *(u32x4_t*)(o + 32) = v1;
  }
}

// Any even block size outside the power-of-two kernels (see k_quantize_any).
int launch_quantize_any(const float* w, const qlora_nf4_t* q, hipStream_t s) {
  const int64_t n = q->rows * q->cols;
  const int64_t bs = q->block_size, nb = n / bs;
  const int64_t grid = ceil_div(nb, kAnyBlocksPerWg);
  if (grid > 0x7fffffff) return set_error(QLORA_ERR_UNSUPPORTED, "quantize: tensor too large");
  const Nf4Tables& t = host_tables();
  ProfScope prof(QLORA_K_QUANTIZE, s);
  if (q->double_quant) {
    const int64_t ng = ceil_div(nb, q->dq_group);
    k_fill_zero<<<dim3((unsigned)ceil_div(ng, kThreads)), dim3(kThreads), 0, s>>>(q->absmax_scale2, ng);
    k_quantize_any<<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, nb, bs, q->codes, nullptr, q->absmax_scale2,
                                                                   q->dq_group, t);
    k_dq_any_q<<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, nb, bs, q->absmax_q, q->absmax_scale2,
                                                               q->dq_group);
    k_dq_large_finish<<<dim3((unsigned)ceil_div(ng, kThreads)), dim3(kThreads), 0, s>>>(q->absmax_scale2, ng);
  } else {
    k_quantize_any<<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, nb, bs, q->codes, q->absmax, nullptr, 1, t);
  }
  return check_launch("k_quantize_any");
}

int launch_quantize(const float* w, const qlora_nf4_t* q, hipStream_t s) {
  const int64_t n = q->rows * q->cols;
  const int bs = q->block_size;
  if (bs < 8 || bs > 512 || (bs & (bs - 1))) return launch_quantize_any(w, q, s);
  const int64_t nb = n / bs;
  // dq: 0 none, 1 groups of up to 4096 blocks (one workgroup each, one pass),
  // 2 larger groups (spans of 16384 elements, a second pass for the u8 scales).
  const int dq = !q->double_quant ? 0 : (q->dq_group <= 4096 ? 1 : 2);
  const int64_t g = q->double_quant ? q->dq_group : 1;
  const int blocks_per_wg = dq == 1 ? q->dq_group : (bs >= 16384 ? 1 : 16384 / bs);
  const int64_t grid = ceil_div(nb, blocks_per_wg);
  const int64_t ng = ceil_div(nb, g);
  const Nf4Tables& t = host_tables();
  if (grid > 0x7fffffff) return set_error(QLORA_ERR_UNSUPPORTED, "quantize: tensor too large");
  ProfScope prof(QLORA_K_QUANTIZE, s);
  if (dq == 2) {
    k_fill_zero<<<dim3((unsigned)ceil_div(ng, kThreads)), dim3(kThreads), 0, s>>>(q->absmax_scale2, ng);
    int rc = check_launch("k_fill_zero");
    if (rc) return rc;
  }
#define QNF4_Q(BS)                                                                         \
  case BS:                                                                                 \
    k_quantize<BS><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(                        \
        w, n, q->codes, q->absmax, q->absmax_q, q->absmax_scale2, blocks_per_wg, dq, g, t); \
    if (dq == 2)                                                                           \
      k_dq_large_q<BS><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(                    \
          w, n, q->absmax_q, q->absmax_scale2, blocks_per_wg, g);                          \
    break;
  switch (bs) {
    QNF4_Q(8)
    QNF4_Q(16)
    QNF4_Q(32)
    QNF4_Q(64)
    QNF4_Q(128)
    QNF4_Q(256)
    QNF4_Q(512)
    default:
      return set_error(QLORA_ERR_UNSUPPORTED, "quantize: block_size %d not supported", bs);
  }
#undef QNF4_Q
  if (dq == 2) k_dq_large_finish<<<dim3((unsigned)ceil_div(ng, kThreads)), dim3(kThreads), 0, s>>>(q->absmax_scale2, ng);
  return check_launch("k_quantize");
}

int dequant_flat(const Nf4W& w, int cd, void* out, hipStream_t s, const SkRed* red);

int launch_dequantize(const qlora_nf4_t* q, int out_dtype, void* out, hipStream_t s) {
  const Nf4W w = make_w(q);
  return dequant_flat(w, out_dtype, out, s, nullptr);
}

// The device form of an optional reduction riding on a dequantize launch.
int ride_along(const SkRed* red, RedJobs& js, int64_t& blocks) {
  js = RedJobs{};
  blocks = 0;
  return red ? make_red_jobs(*red, nullptr, js, blocks) : QLORA_OK;
}

// Flat dequantize of all rows * cols elements into out (f32 / bf16 / f16); `red`
// (bf16 / f16 only) rides on the same launch.
// Whether k_dequant_chunks takes this weight (and, with a riding reduction, this dtype).
bool chunks_ok(const Nf4W& w, int cd, bool red) {
  const int64_t n = w.rows * w.cols;
  return w.bs_shift >= 3 && n % 8 == 0 && (!w.dq || w.g_shift >= 0) && n / 2 < (1LL << 31) &&
         !(red && cd == CD_F32);
}

// One k_dequant_chunks launch over np parts (all with or all without double
// quantization) and the reductions riding on it.
int launch_chunks(const DqParts& ps, int cd, bool dq, const RedJobs& js, int64_t nred, hipStream_t s) {
  const int64_t grid = ps.end[ps.np - 1];
  if (grid + nred > 0x7fffffff) return set_error(QLORA_ERR_UNSUPPORTED, "dequantize: tensor too large");
  const Nf4Tables& t = host_tables();
  const dim3 g((unsigned)(grid + nred)), blk(kThreads);
  const uint32_t nm = (uint32_t)grid;
  if (cd == CD_BF16) {
    if (dq) k_dequant_chunks<CD_BF16, 1><<<g, blk, 0, s>>>(ps, t, js, nm);
    else k_dequant_chunks<CD_BF16, 0><<<g, blk, 0, s>>>(ps, t, js, nm);
  } else if (cd == CD_F16) {
    if (dq) k_dequant_chunks<CD_F16, 1><<<g, blk, 0, s>>>(ps, t, js, nm);
    else k_dequant_chunks<CD_F16, 0><<<g, blk, 0, s>>>(ps, t, js, nm);
  } else if (cd == CD_F32) {
    if (dq) k_dequant_chunks<CD_F32, 1><<<g, blk, 0, s>>>(ps, t, js, nm);
    else k_dequant_chunks<CD_F32, 0><<<g, blk, 0, s>>>(ps, t, js, nm);
  } else {
    return set_error(QLORA_ERR_DTYPE, "dequantize: bad dtype %d", cd);
  }
  return check_launch("k_dequant_chunks");
}

// The workgroups of k_dequant_chunks for n elements.
int64_t chunk_wgs(int64_t n) { return ceil_div(n / 8, kThreads * 8); }

int dequant_flat(const Nf4W& w, int cd, void* out, hipStream_t s, const SkRed* red) {
  const int64_t n = w.rows * w.cols;
  const Nf4Tables& t = host_tables();
  RedJobs js;
  int64_t nred;
  int rc = ride_along(red, js, nred);
  if (rc) return rc;
  ProfScope prof(QLORA_K_DEQUANTIZE, s);
  if (chunks_ok(w, cd, red != nullptr)) {
    DqParts ps = {};
    ps.w[0] = w;
    ps.out[0] = out;
    ps.n[0] = n;
    ps.end[0] = (uint32_t)chunk_wgs(n);  // n / 2 < 2^31
    ps.np = 1;
    return launch_chunks(ps, cd, w.dq != 0, js, nred, s);
  }
  if (red && (rc = skinny_reduce_jobs(cd, *red, nullptr, s))) return rc;
  if (w.bs % 8 == 0 && n % 32 == 0) {
    const int64_t grid = ceil_div(n / 32, kThreads);
    if (grid > 0x7fffffff) return set_error(QLORA_ERR_UNSUPPORTED, "dequantize: tensor too large");
    if (cd == CD_BF16) k_dequantize<CD_BF16><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, n, out, t);
    else if (cd == CD_F16) k_dequantize<CD_F16><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, n, out, t);
    else if (cd == CD_F32) k_dequantize<CD_F32><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, n, out, t);
    else return set_error(QLORA_ERR_DTYPE, "dequantize: bad dtype %d", cd);
    return check_launch("k_dequantize");
  }
  const int64_t grid = ceil_div(n / 2, kThreads);
  if (grid > 0x7fffffff) return set_error(QLORA_ERR_UNSUPPORTED, "dequantize: tensor too large");
  if (cd == CD_BF16) k_dequantize_any<CD_BF16><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, n, out, t);
  else if (cd == CD_F16) k_dequantize_any<CD_F16><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, n, out, t);
  else if (cd == CD_F32) k_dequantize_any<CD_F32><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, n, out, t);
  else return set_error(QLORA_ERR_DTYPE, "dequantize: bad dtype %d", cd);
  return check_launch("k_dequantize_any");
}

template <int OUT, int DQ>
void run_dqt(bool four, uint32_t gx, uint32_t nmain, int64_t nred, const Nf4W& w, void* out, int64_t ldo,
             const Nf4Tables& t, const RedJobs& js, hipStream_t s) {
  const dim3 grid((unsigned)(nmain + nred));
  if (four && w.bs_shift >= 5) k_dequantize_t4<OUT, DQ><<<grid, dim3(kThreads), 0, s>>>(w, out, ldo, t, js, gx, nmain);
  else if (four) k_dequantize_t<OUT, DQ, 4><<<grid, dim3(kThreads), 0, s>>>(w, out, ldo, t, js, gx, nmain);
  else k_dequantize_t<OUT, DQ, 1><<<grid, dim3(kThreads), 0, s>>>(w, out, ldo, t, js, gx, nmain);
}

// Dequantize W into a compute-dtype buffer inside a layer call: [rows, cols]
// (forward) or its transpose [cols][ldo] (dX; ldo = 0 means rows, a larger ldo
// writes W~^T as the column slice of a wider matrix).  The transpose needs rows and
// cols to be multiples of 64.
// W~_i of g weights into outs[i] (flat, rows_i x cols_i each), reds[i] riding on the
// same launch: one launch when every weight takes k_dequant_chunks with the same
// double-quantization setting and g <= kDqParts, else one dequantize each.
int dequant_group_into(const Nf4W* ws, int g, int cd, void* const* outs, const SkRed* reds, hipStream_t s) {
  bool one = g >= 1 && g <= kDqParts && g <= kRedJobs;
  for (int i = 0; i < g && one; ++i) one = chunks_ok(ws[i], cd, true) && ws[i].dq == ws[0].dq;
  if (!one) {
    for (int i = 0; i < g; ++i) {
      const int rc = dequant_into(ws[i], cd, outs[i], false, s, &reds[i]);
      if (rc) return rc;
    }
    return QLORA_OK;
  }
  RedJobs js;
  int64_t nred;
  int rc = make_red_jobs_n(reds, g, js, nred);
  if (rc) return rc;
  ProfScope prof(QLORA_K_DEQUANTIZE, s);
  DqParts ps = {};
  int64_t e = 0;
  for (int i = 0; i < g; ++i) {
    ps.w[i] = ws[i];
    ps.out[i] = outs[i];
    ps.n[i] = ws[i].rows * ws[i].cols;
    e += chunk_wgs(ps.n[i]);
    if (e > 0x7fffffff) return set_error(QLORA_ERR_UNSUPPORTED, "dequantize: group too large");
    ps.end[i] = (uint32_t)e;
  }
  ps.np = g;
  return launch_chunks(ps, cd, ws[0].dq != 0, js, nred, s);
}

int dequant_into(const Nf4W& w, int cd, void* out, bool transposed, hipStream_t s, const SkRed* red, int64_t ldo) {
  if (transposed) {
    if (ldo == 0) ldo = w.rows;
    if (ldo < w.rows || ldo % 8 || w.cols * ldo >= (1LL << 31))
      return set_error(QLORA_ERR_UNSUPPORTED, "dequantize^T: output stride %lld not supported", (long long)ldo);
    const Nf4Tables& t = host_tables();
    RedJobs js;
    int64_t nred;
    int rc = ride_along(red, js, nred);
    if (rc) return rc;
    ProfScope prof(QLORA_K_DEQUANTIZE, s);
    if (w.rows % 64 || w.cols % 64) return set_error(QLORA_ERR_UNSUPPORTED, "dequantize^T: shape not a multiple of 64");
    if (w.bs_shift < 3 || (w.dq && w.g_shift < 0) || w.rows * w.cols / 2 >= (1LL << 31))
      return set_error(QLORA_ERR_UNSUPPORTED, "dequantize^T: block / group sizes or size not supported");
    // four tiles per workgroup while that still leaves >= 1024 workgroups, else one
    const int T4 = (w.rows / 64) * ceil_div(w.cols, 256) >= 1024;
    const int64_t gx = ceil_div(w.cols, T4 ? 256 : 64), nmain = gx * (w.rows / 64);
    if (nmain + nred > 0x7fffffff) return set_error(QLORA_ERR_UNSUPPORTED, "dequantize^T: tensor too large");
    if (cd == CD_BF16) {
      if (w.dq) run_dqt<CD_BF16, 1>(T4, (uint32_t)gx, (uint32_t)nmain, nred, w, out, ldo, t, js, s);
      else run_dqt<CD_BF16, 0>(T4, (uint32_t)gx, (uint32_t)nmain, nred, w, out, ldo, t, js, s);
    } else if (cd == CD_F16) {
      if (w.dq) run_dqt<CD_F16, 1>(T4, (uint32_t)gx, (uint32_t)nmain, nred, w, out, ldo, t, js, s);
      else run_dqt<CD_F16, 0>(T4, (uint32_t)gx, (uint32_t)nmain, nred, w, out, ldo, t, js, s);
    }
    else return set_error(QLORA_ERR_DTYPE, "dequantize^T: bad dtype %d", cd);
    return check_launch("k_dequantize_t");
  }
  return dequant_flat(w, cd, out, s, red);
}

}  // namespace qnf4
