// dropout.hip -- the pieces LoRA dropout adds to the layer.
//
// rust_ai_core QLoraConfig docs, "Fields" (the LoRA configuration holds rank, alpha
// and dropout); "LoRA and QLoRA, mathematically", "Tooling" (PEFT's LoraConfig and
// its dropout).  Dropout acts on the input of the low-rank branch only, as inverted
// dropout with a caller-drawn keep mask M (1 = kept) and rate p:
//   y  = x W~^T + s (x_d A^T) B^T,  x_d = x M / (1 - p);
//   dX = dY W~ + (dT A) M / (1 - p),  dA = dT^T x_d,  dB = s dY^T (x_d A^T),  dT = s dY B.
// The layer keeps x M (exact in the compute dtype) as the branch input and folds
// 1 / (1 - p) into the branch scale, so T, dT, dA and dB come from the usual
// kernels; dX takes the base product from the usual GEMM and the masked low-rank
// term from k_rank_add_masked.
#include <algorithm>

#include "common.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;

// out = x * mask (the kept elements exactly, the dropped ones zero).
template <int CD>
__global__ __launch_bounds__(kThreads) void k_apply_mask(const void* __restrict__ x, const uint8_t* __restrict__ mask,
                                                         int64_t n, void* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    store_cd<CD>(out, i, mask[i] ? load_cd<CD>(x, i) : 0.0f);
}

__global__ __launch_bounds__(kThreads) void k_zero_bytes(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < words; i += (int64_t)gridDim.x * kThreads)
    p[i] = 0u;
}

// dx[i][k] = RNE_cd(dx[i][k] + M[i][k] * sum_t dT[i][t] A[t][k]) over 64 x 64 tiles:
// dT (compute dtype, leading dimension ld_dt) and A staged in LDS as fp32 slices of
// 32 ranks, each thread a 4 x 4 block of outputs, the rank sum in fp32 in rank order.
constexpr int kT = 64;
constexpr int kR = 32;

template <int CD>
__global__ __launch_bounds__(kThreads) void k_rank_add_masked(void* __restrict__ dx, const uint8_t* __restrict__ mask,
                                                              const void* __restrict__ dt, int64_t ld_dt,
                                                              const void* __restrict__ a, int32_t r, int64_t M,
                                                              int64_t K) {
  __shared__ float dsh[kT][kR + 1];  // [i][t]
  __shared__ float ash[kR][kT];      // [t][k]
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t i0 = (int64_t)blockIdx.y * kT, k0 = (int64_t)blockIdx.x * kT;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int t0 = 0; t0 < r; t0 += kR) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kT * kR / kThreads; ++q) {
      const int idx = tid + kThreads * q;
      {
        const int il = idx / kR, tl = idx % kR;
        const int64_t i = i0 + il;
        const int t = t0 + tl;
        dsh[il][tl] = (i < M && t < r) ? load_cd<CD>(dt, i * ld_dt + t) : 0.f;
      }
      {
        const int tl = idx / kT, kl = idx % kT;
        const int t = t0 + tl;
        const int64_t k = k0 + kl;
        ash[tl][kl] = (t < r && k < K) ? load_cd<CD>(a, (int64_t)t * K + k) : 0.f;
      }
    }
    __syncthreads();
    const int tc = min(kR, r - t0);
    for (int t = 0; t < tc; ++t) {
      float dv[4], av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dv[i] = dsh[ty * 4 + i][t];
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = ash[t][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(dv[i], av[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = i0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k = k0 + tx * 4 + j;
      if (k >= K) continue;
      const int64_t e = row * K + k;
      if (mask[e]) store_cd<CD>(dx, e, load_cd<CD>(dx, e) + acc[i][j]);
    }
  }
}

int64_t grid_for(int64_t n) { return std::max<int64_t>(1, std::min<int64_t>(4096, ceil_div(n, kThreads))); }

}  // namespace

int apply_mask(int cd, const void* x, const uint8_t* mask, int64_t n, void* out, hipStream_t s) {
  if (n == 0) return QLORA_OK;
  const dim3 g((unsigned)grid_for(n)), b(kThreads);
  if (cd == CD_BF16) k_apply_mask<CD_BF16><<<g, b, 0, s>>>(x, mask, n, out);
  else if (cd == CD_F16) k_apply_mask<CD_F16><<<g, b, 0, s>>>(x, mask, n, out);
  else k_apply_mask<CD_F32><<<g, b, 0, s>>>(x, mask, n, out);
  return check_launch("k_apply_mask");
}

// Zero a 4-byte-aligned buffer with a kernel (also safe inside a captured graph).
int zero_fill(void* p, int64_t bytes, hipStream_t s) {
  const int64_t words = bytes / 4;
  if (words == 0) return QLORA_OK;
  k_zero_bytes<<<dim3((unsigned)grid_for(words)), dim3(kThreads), 0, s>>>((uint32_t*)p, words);
  return check_launch("k_zero_bytes");
}

int rank_add_masked(int cd, void* dx, const uint8_t* mask, const void* dt, int64_t ld_dt, const void* a, int32_t r,
                    int64_t M, int64_t K, hipStream_t s) {
  const int64_t gy = ceil_div(M, kT), gx = ceil_div(K, kT);
  if (gy > 65535) return set_error(QLORA_ERR_UNSUPPORTED, "dropout: too many tokens (%lld)", (long long)M);
  ProfScope prof(QLORA_K_BWD_DX, s);
  const dim3 g((unsigned)gx, (unsigned)gy), b(kThreads);
  if (cd == CD_BF16) k_rank_add_masked<CD_BF16><<<g, b, 0, s>>>(dx, mask, dt, ld_dt, a, r, M, K);
  else if (cd == CD_F16) k_rank_add_masked<CD_F16><<<g, b, 0, s>>>(dx, mask, dt, ld_dt, a, r, M, K);
  else k_rank_add_masked<CD_F32><<<g, b, 0, s>>>(dx, mask, dt, ld_dt, a, r, M, K);
  return check_launch("k_rank_add_masked");
}

}  // namespace qnf4
