// gemv.hip -- decode-shaped forward (m <= 16 tokens) of the QLoRA layer on gfx950.
//
// y[m, n] = sum_k x[m, k] W~[n, k] + sum_t T[m, t] B[n, t] (+ bias[n]),
// T = s x A^T, W~ = cd(fl32(L[c] s_b)) (qlora-rs README "Honest capability
// matrix": dequant honours the compute dtype; rust_ai_core QLoraConfig
// scale() = alpha / r).  At m <= 16 the layer moves the packed weight once and
// does at most 32 flops per weight, so it is bound by HBM: the kernel streams
// each row's codes with 16-byte loads, decodes in registers and accumulates all m
// tokens at once, one wavefront per output row.
#include "common.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxM = 16;

// T[m, t] = s * sum_k x[m, k] A[t, k]; t0[m, t] = the unscaled sum (optional).
template <int CD>
__global__ __launch_bounds__(kThreads) void k_lora_down_small(const void* __restrict__ x,
                                                              const void* __restrict__ A, int64_t M,
                                                              int64_t K, int32_t r, float scale,
                                                              float* __restrict__ T,
                                                              float* __restrict__ t0) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= r) return;
  float acc[kMaxM];
#pragma unroll
  for (int i = 0; i < kMaxM; ++i) acc[i] = 0.f;
  for (int64_t k = lane; k < K; k += 64) {
    const float a = load_cd<CD>(A, t * K + k);
#pragma unroll
    for (int i = 0; i < kMaxM; ++i)
      if (i < M) acc[i] = fmaf(load_cd<CD>(x, (int64_t)i * K + k), a, acc[i]);
  }
#pragma unroll
  for (int i = 0; i < kMaxM; ++i)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[i] += __shfl_xor(acc[i], off, 64);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < kMaxM; ++i)
      if (i < M) {
        T[(int64_t)i * r + t] = acc[i] * scale;
        if (t0) t0[(int64_t)i * r + t] = acc[i];
      }
  }
}

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

template <int CD>
int gemv_forward_t(const LayerCall& c, void* y, float* t_save) {
  float* T = (float*)c.ws;
  {
  ProfScope prof(QLORA_K_LORA_DOWN, c.stream);
  k_lora_down_small<CD><<<dim3((unsigned)ceil_div(c.r, kThreads / 64)), dim3(kThreads), 0, c.stream>>>(
      c.x, c.lora_a, c.m, c.w.cols, c.r, c.scale, T, t_save);
  int rc = check_launch("k_lora_down_small");
  if (rc) return rc;
  }
  ProfScope prof(QLORA_K_GEMV, c.stream);
  k_gemv<CD><<<dim3((unsigned)ceil_div(c.w.rows, kThreads / 64)), dim3(kThreads), 0, c.stream>>>(
      c.w, c.x, c.m, T, c.lora_b, c.r, c.bias, y, host_tables());
  return check_launch("k_gemv");
}

}  // namespace

size_t gemv_workspace_bytes(int64_t m, int32_t r) { return (size_t)round_up(m * r * 4, 256); }

int gemv_forward(const LayerCall& c, void* y, float* t_save) {
  switch (c.cd) {
    case CD_BF16: return gemv_forward_t<CD_BF16>(c, y, t_save);
    case CD_F16: return gemv_forward_t<CD_F16>(c, y, t_save);
    case CD_F32: return gemv_forward_t<CD_F32>(c, y, t_save);
  }
  return set_error(QLORA_ERR_DTYPE, "forward: bad compute dtype %d", c.cd);
}

}  // namespace qnf4
