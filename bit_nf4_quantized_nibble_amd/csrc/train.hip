// train.hip -- the training step of a stack of QLoRA linear layers: MSE loss and
// its gradient, AdamW on the adapters, and the host sequence that runs the stack
// forward, the loss, the stack backward and the updates on one stream.
//
// qlora-rs README, "Training (layer stack)": QuantizedLinear layers stacked, a
// training_step with an MSE loss, AdamW updating the LoRA adapters while the NF4
// bases stay frozen; "Honest capability matrix": multi-layer MSE training.
//
// Both kernels are elementwise HBM streams.  The loss is summed in a fixed order
// (per-thread strided sums, then fixed trees), so it is deterministic run to run.
#include <math.h>

#include <algorithm>
#include <vector>

#include "common.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kMsePartials = 1024;  // workgroups of the loss pass at most

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) s += red[w];
  return s;
}

// dy = RNE_cd(2 (y - t) / N) for every element; partial[blockIdx] = sum of (y - t)^2
// over the elements this workgroup visits (grid-stride, fixed assignment).
template <int CD>
__global__ __launch_bounds__(kThreads) void k_mse(const void* __restrict__ y, const void* __restrict__ t, int64_t n,
                                                  void* __restrict__ dy, float* __restrict__ partial) {
  __shared__ float red[kThreads / 64];
  const float nf = (float)n;
  float acc = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const float d = load_cd<CD>(y, i) - load_cd<CD>(t, i);
    acc = fmaf(d, d, acc);
    store_cd<CD>(dy, i, (2.0f * d) / nf);
  }
  const float s = block_sum(acc, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// loss = (sum of the partials in index order, by a fixed tree) / N.
__global__ __launch_bounds__(kThreads) void k_mse_final(const float* __restrict__ partial, int np, int64_t n,
                                                        float* __restrict__ loss) {
  __shared__ float red[kThreads / 64];
  float acc = 0.f;
  for (int i = threadIdx.x; i < np; i += kThreads) acc += partial[i];
  const float s = block_sum(acc, red);
  if (threadIdx.x == 0) loss[0] = s / (float)n;
}

struct AdamW {
  float lr, b1, b2, eps, wd, bc1, bc2;  // bc = 1 - beta^t
};

// m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
// theta = theta (1 - lr wd) - lr (m / bc1) / (sqrt(v / bc2) + eps);  theta_cd = RNE_cd(theta).
template <int CD>
__global__ __launch_bounds__(kThreads) void k_adamw(float* __restrict__ theta, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v, int64_t n, AdamW o,
                                                    void* __restrict__ theta_cd) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const float gi = g[i];
    const float mi = o.b1 * m[i] + (1.0f - o.b1) * gi;
    const float vi = o.b2 * v[i] + (1.0f - o.b2) * (gi * gi);
    const float mhat = mi / o.bc1, vhat = vi / o.bc2;
    const float th = theta[i] * (1.0f - o.lr * o.wd) - o.lr * (mhat / (sqrtf(vhat) + o.eps));
    m[i] = mi;
    v[i] = vi;
    theta[i] = th;
    if (theta_cd) store_cd<CD>(theta_cd, i, th);
  }
}

int64_t grid_for(int64_t n, int64_t cap) { return std::max<int64_t>(1, std::min<int64_t>(cap, ceil_div(n, kThreads))); }

}  // namespace

int launch_mse(const void* y, const void* t, int64_t n, int cd, float* loss, void* dy, float* partial,
               hipStream_t s) {
  ProfScope prof(QLORA_K_LOSS, s);
  const int64_t grid = grid_for(n, kMsePartials);
  const dim3 g((unsigned)grid), b(kThreads);
  if (cd == CD_BF16) k_mse<CD_BF16><<<g, b, 0, s>>>(y, t, n, dy, partial);
  else if (cd == CD_F16) k_mse<CD_F16><<<g, b, 0, s>>>(y, t, n, dy, partial);
  else k_mse<CD_F32><<<g, b, 0, s>>>(y, t, n, dy, partial);
  int rc = check_launch("k_mse");
  if (rc) return rc;
  k_mse_final<<<dim3(1), b, 0, s>>>(partial, (int)grid, n, loss);
  return check_launch("k_mse_final");
}

size_t mse_workspace_bytes() { return kMsePartials * sizeof(float); }

int launch_adamw(float* theta, const float* g, float* m, float* v, int64_t n, const qlora_adamw_t& o, int32_t step,
                 void* theta_cd, int cd, hipStream_t s) {
  ProfScope prof(QLORA_K_OPTIM, s);
  AdamW a;
  a.lr = o.lr;
  a.b1 = o.beta1;
  a.b2 = o.beta2;
  a.eps = o.eps;
  a.wd = o.weight_decay;
  a.bc1 = (float)(1.0 - pow((double)o.beta1, (double)step));
  a.bc2 = (float)(1.0 - pow((double)o.beta2, (double)step));
  const dim3 grid((unsigned)grid_for(n, 2048)), b(kThreads);
  if (cd == CD_BF16) k_adamw<CD_BF16><<<grid, b, 0, s>>>(theta, g, m, v, n, a, theta_cd);
  else if (cd == CD_F16) k_adamw<CD_F16><<<grid, b, 0, s>>>(theta, g, m, v, n, a, theta_cd);
  else k_adamw<CD_F32><<<grid, b, 0, s>>>(theta, g, m, v, n, a, theta_cd);
  return check_launch("k_adamw");
}

// ---------------------------------------------------------------- the stack step
namespace {
struct StackPlan {
  std::vector<size_t> off_h;   // h_1 .. h_L (h_L = y)
  std::vector<size_t> off_t0;  // T0 per layer
  size_t off_dy = 0, off_g0 = 0, off_g1 = 0, off_part = 0, off_layer = 0, layer_bytes = 0, total = 0;
};

size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

StackPlan plan_stack(const qlora_stack_layer_t* layers, int32_t L, int64_t m, int32_t r, int cd, int32_t flags) {
  StackPlan P;
  const size_t es = cd_bytes(cd);
  size_t off = 0;
  int64_t maxw = 1;
  for (int l = 0; l < L; ++l) {
    const int64_t rows = layers[l].w->rows, cols = layers[l].w->cols;
    P.off_h.push_back(off);
    off += al((size_t)(m * rows) * es);
    P.off_t0.push_back(off);
    off += al((size_t)(m * r) * 4);
    if (l > 0) maxw = std::max(maxw, cols);
    P.layer_bytes = std::max(P.layer_bytes, std::max(fwd_workspace_bytes(m, rows, cols, r, cd, flags),
                                                     bwd_workspace_bytes(m, rows, cols, r, cd, flags)));
  }
  P.off_dy = off;
  off += al((size_t)(m * layers[L - 1].w->rows) * es);
  P.off_g0 = off;
  off += al((size_t)(m * maxw) * es);
  P.off_g1 = off;
  off += al((size_t)(m * maxw) * es);
  P.off_part = off;
  off += al(mse_workspace_bytes());
  P.off_layer = off;
  off += al(P.layer_bytes);
  P.total = off;
  return P;
}
}  // namespace

size_t stack_workspace_bytes(const qlora_stack_layer_t* layers, int32_t L, int64_t m, int32_t r, int cd,
                             int32_t flags) {
  return plan_stack(layers, L, m, r, cd, flags).total;
}

int launch_stack_step(const qlora_stack_layer_t* layers, int32_t L, const void* x, int64_t m, const void* target,
                      int32_t r, float scale, int32_t flags, int cd, const qlora_adamw_t& opt, int32_t step,
                      float* loss, void* ws, hipStream_t s) {
  const StackPlan P = plan_stack(layers, L, m, r, cd, flags);
  char* base = (char*)ws;
  auto call = [&](int l, const void* in) {
    LayerCall c;
    c.w = make_w(layers[l].w);
    c.cd = cd;
    c.m = m;
    c.r = r;
    c.scale = scale;
    c.flags = flags;
    c.x = in;
    c.drop_mask = nullptr;
    c.lora_a = layers[l].lora_a;
    c.lora_b = layers[l].lora_b;
    c.bias = nullptr;
    c.ws = base + P.off_layer;
    c.ws_bytes = P.layer_bytes;
    c.stream = s;
    return c;
  };
  int rc;
  // forward: h_{l+1} = layer_l(h_l), T0_l kept for the backward
  const void* h = x;
  for (int l = 0; l < L; ++l) {
    void* out = base + P.off_h[l];
    if ((rc = launch_forward(call(l, h), out, (float*)(base + P.off_t0[l])))) return rc;
    h = out;
  }
  // loss and dL/dy
  void* dy = base + P.off_dy;
  if ((rc = launch_mse(h, target, m * layers[L - 1].w->rows, cd, loss, dy, (float*)(base + P.off_part), s)))
    return rc;
  // backward, last layer first; dX of layer 0 is not needed
  const void* g = dy;
  for (int l = L - 1; l >= 0; --l) {
    const void* in = l ? (const void*)(base + P.off_h[l - 1]) : x;
    void* dx = l ? (void*)(base + (((L - 1 - l) & 1) ? P.off_g1 : P.off_g0)) : nullptr;
    if ((rc = launch_backward(call(l, in), g, (const float*)(base + P.off_t0[l]), dx, layers[l].grad_a,
                              layers[l].grad_b)))
      return rc;
    g = dx;
  }
  // AdamW on every adapter; the compute-dtype copies follow the fp32 masters
  for (int l = 0; l < L; ++l) {
    const int64_t rows = layers[l].w->rows, cols = layers[l].w->cols;
    if ((rc = launch_adamw(layers[l].a32, layers[l].grad_a, layers[l].m_a, layers[l].v_a, (int64_t)r * cols, opt,
                           step, layers[l].lora_a, cd, s)))
      return rc;
    if ((rc = launch_adamw(layers[l].b32, layers[l].grad_b, layers[l].m_b, layers[l].v_b, rows * (int64_t)r, opt,
                           step, layers[l].lora_b, cd, s)))
      return rc;
  }
  return QLORA_OK;
}

}  // namespace qnf4
