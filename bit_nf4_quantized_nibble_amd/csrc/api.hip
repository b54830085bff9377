// api.hip -- host side of libqlora_nf4.so: the C ABI declared in
// include/qlora_nf4.h, argument validation, error reporting and the NF4 level
// table.  Validation happens before anything is launched, so a refused call
// writes nothing (qlora-rs export refuses invalid layers before writing; the
// rust_ai_core QLoraConfig validate_for_training returns an error for an
// invalid configuration).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "common.h"

namespace qnf4 {

namespace {
thread_local char g_err[512] = "";

// ---------------------------------------------------------------- NF4 levels
// "LoRA and QLoRA, mathematically", "NF4: quantizing the frozen base": 16 levels at
// the quantiles of a normal distribution (printed to 3 decimals on the qlora-rs
// README, "NF4 Quantization").  Construction: with the offset
// d = (1 - 1/30)/2 + (1 - 1/32)/2, 8 positive levels are the normal quantiles at
// d - j (d - 1/2) / 8 (j = 0..7), 7 negative levels are minus those at
// d - j (d - 1/2) / 7 (j = 0..6), plus an exact zero; all divide by the largest and
// round once to binary32.  The quantile is found by Newton's method on the CDF.
double normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }
double normal_pdf(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }
double normal_quantile_upper(double p) {  // p in (1/2, 1)
  double x = 0.0;
  for (int it = 0; it < 200; ++it) {
    const double dx = (normal_cdf(x) - p) / normal_pdf(x);
    x -= dx;
    if (fabs(dx) <= 1e-17 * (1.0 + fabs(x))) break;
  }
  return x;
}

Nf4Tables g_tables;
bool g_tables_ok = false;
std::once_flag g_tables_once;

void build_tables() {
  const double d = 0.5 * (1.0 - 1.0 / 30.0) + 0.5 * (1.0 - 1.0 / 32.0);
  const double top = normal_quantile_upper(d);
  double lv[16];
  int i = 0;
  for (int j = 0; j <= 6; ++j) lv[i++] = -normal_quantile_upper(d - j * (d - 0.5) / 7.0) / top;
  lv[i++] = 0.0;
  for (int j = 7; j >= 0; --j) lv[i++] = normal_quantile_upper(d - j * (d - 0.5) / 8.0) / top;
  Nf4Tables t;
  for (int k = 0; k < 16; ++k) t.lv[k] = (float)lv[k];
  // Nearest level with ties to the lower code: code = #{j : x > mid_j} with the
  // midpoints exact in fp64; for binary32 x that is #{j : x >= thr_j}, thr_j the
  // smallest binary32 strictly above mid_j.
  for (int j = 0; j < 15; ++j) {
    const double mid = ((double)t.lv[j] + (double)t.lv[j + 1]) / 2.0;
    float th = (float)mid;
    if ((double)th <= mid) th = nextafterf(th, INFINITY);
    t.thr[j] = th;
  }
  // Bucket table: bucket b holds x with b <= 16 (x + 1) < b + 1.
  bool ok = true;
  for (int b = 0; b < 32; ++b) {
    const double lo = b / 16.0 - 1.0, hi = (b + 1) / 16.0 - 1.0;
    int base = 0, inside = 0;
    float th = INFINITY;
    for (int j = 0; j < 15; ++j) {
      if ((double)t.thr[j] <= lo)
        ++base;
      else if ((double)t.thr[j] < hi || (b == 31 && (double)t.thr[j] <= 1.0)) {
        ++inside;
        th = t.thr[j];
      }
      // fl32(16 x + 16) may misplace x by a few 1e-7 near an edge: keep thresholds away.
      if (fabs((double)t.thr[j] - lo) < 1e-6 || fabs((double)t.thr[j] - hi) < 1e-6) ok = false;
    }
    if (inside > 1) ok = false;
    t.bucket_base[b] = base;
    t.bucket_thr[b] = th;
  }
  g_tables = t;
  g_tables_ok = ok;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_cd(int32_t cd) { return cd == QLORA_F32 || cd == QLORA_BF16 || cd == QLORA_F16; }

int validate_desc(const qlora_nf4_t* q, bool need_data, const char* who) {
  if (!q) return set_error(QLORA_ERR_INVALID_ARG, "%s: null descriptor", who);
  if (q->rows < 0 || q->cols < 0) return set_error(QLORA_ERR_SHAPE, "%s: negative shape", who);
  if (q->reserved != 0) return set_error(QLORA_ERR_INVALID_ARG, "%s: reserved field must be 0", who);
  const int64_t n = q->rows * q->cols;
  const int32_t bs = q->block_size;
  if (bs <= 0 || (bs & 1)) return set_error(QLORA_ERR_SHAPE, "%s: block_size %d must be positive and even", who, bs);
  if (n % bs != 0) return set_error(QLORA_ERR_SHAPE, "%s: %lld elements not a multiple of block_size %d", who, (long long)n, bs);
  if (q->double_quant != 0 && q->double_quant != 1)
    return set_error(QLORA_ERR_INVALID_ARG, "%s: double_quant must be 0 or 1", who);
  if (q->double_quant && q->dq_group <= 0)
    return set_error(QLORA_ERR_INVALID_ARG, "%s: dq_group must be positive", who);
  if (!need_data || n == 0) return QLORA_OK;
  if (!q->codes) return set_error(QLORA_ERR_INVALID_ARG, "%s: null codes", who);
  if (!aligned16(q->codes)) return set_error(QLORA_ERR_INVALID_ARG, "%s: codes must be 16-byte aligned", who);
  if (q->double_quant) {
    if (!q->absmax_q || !q->absmax_scale2)
      return set_error(QLORA_ERR_INVALID_ARG, "%s: double quant needs absmax_q and absmax_scale2", who);
  } else if (!q->absmax) {
    return set_error(QLORA_ERR_INVALID_ARG, "%s: null absmax", who);
  }
  return QLORA_OK;
}

int validate_layer(const qlora_nf4_t* w, const void* x, int64_t m, const void* lora_a,
                   const void* lora_b, int32_t r, float alpha, int32_t flags, int32_t cd,
                   const char* who) {
  int rc = validate_desc(w, true, who);
  if (rc) return rc;
  if (!valid_cd(cd)) return set_error(QLORA_ERR_DTYPE, "%s: bad compute dtype %d", who, cd);
  if (m < 0) return set_error(QLORA_ERR_SHAPE, "%s: negative m", who);
  if (r < 1) return set_error(QLORA_ERR_INVALID_ARG, "%s: rank r must be >= 1 (got %d)", who, r);
  if (!isfinite(alpha)) return set_error(QLORA_ERR_INVALID_ARG, "%s: alpha must be finite", who);
  if (flags & ~(QLORA_FLAG_RSLORA | QLORA_FLAG_FUSED | QLORA_FLAG_DEQUANT_GEMM | QLORA_FLAG_DROPOUT))
    return set_error(QLORA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", who, flags);
  if ((flags & QLORA_FLAG_FUSED) && (flags & QLORA_FLAG_DEQUANT_GEMM))
    return set_error(QLORA_ERR_INVALID_ARG, "%s: QLORA_FLAG_FUSED and QLORA_FLAG_DEQUANT_GEMM exclude each other", who);
  if (w->rows < 1 || w->cols < 1) return set_error(QLORA_ERR_SHAPE, "%s: empty weight", who);
  if (!x || !lora_a || !lora_b) return set_error(QLORA_ERR_INVALID_ARG, "%s: null x / lora_a / lora_b", who);
  if (!aligned16(x) || !aligned16(lora_a) || !aligned16(lora_b))
    return set_error(QLORA_ERR_INVALID_ARG, "%s: x, lora_a and lora_b must be 16-byte aligned", who);
  return QLORA_OK;
}

// Optional device arrays of a layer call: null, or 16-byte aligned.
int check_aligned(const char* who, const char* names, std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return set_error(QLORA_ERR_INVALID_ARG, "%s: %s must be 16-byte aligned", who, names);
  return QLORA_OK;
}

float lora_scale(float alpha, int32_t r, int32_t flags) {
  if (flags & QLORA_FLAG_RSLORA) return (float)((double)alpha / sqrt((double)r));
  return (float)((double)alpha / (double)r);
}

int check_tables(const char* who) {
  std::call_once(g_tables_once, build_tables);
  if (!g_tables_ok) return set_error(QLORA_ERR_UNSUPPORTED, "%s: NF4 lookup table failed its self-check", who);
  return QLORA_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need, const char* who) {
  if (ws_bytes < need)
    return set_error(QLORA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu required", who, ws_bytes, need);
  if (need > 0 && (!ws || ((uintptr_t)ws & 255u)))
    return set_error(QLORA_ERR_WORKSPACE, "%s: workspace must be non-null and 256-byte aligned", who);
  return QLORA_OK;
}

// ---------------------------------------------------------------- scratch memory
// The workspace of qlora_linear_fwd_noalloc: a device array in the library's own
// code object, so the call allocates nothing.  Every GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: the device address of each GPU's copy comes from
// hipGetSymbolAddress with that GPU current, once per device, and only that
// address is ever handed to kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on first use).
int scratch_address(void** out, const char* who) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(QLORA_ERR_HIP, "%s: no current device (or device index %d beyond %d)", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(QLORA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed: %s", who, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

}  // namespace

const Nf4Tables& host_tables() {
  std::call_once(g_tables_once, build_tables);
  return g_tables;
}

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(QLORA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return QLORA_OK;
}

// ---------------------------------------------------------------- kernel timing
namespace {
struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec*> g_prof_pending, g_prof_free;
double g_prof_ms[QLORA_K_COUNT];
int64_t g_prof_n[QLORA_K_COUNT];

const char* kKernelNames[QLORA_K_COUNT] = {
    "quantize", "dequantize", "lora_down", "reduce", "fwd_gemm", "gemv",
    "bwd_dt",   "bwd_dx",     "bwd_da",    "bwd_db", "merge", "loss", "optim"};

// Wait for every recorded pair and fold it into the totals (lock held).
int prof_drain() {
  int rc = QLORA_OK;
  for (ProfRec* p : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p->b) != hipSuccess || hipEventElapsedTime(&ms, p->a, p->b) != hipSuccess)
      rc = QLORA_ERR_HIP;
    g_prof_ms[p->kind] += ms;
    g_prof_n[p->kind] += 1;
    g_prof_free.push_back(p);
  }
  g_prof_pending.clear();
  return rc;
}
}  // namespace

int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

void prof_begin(int kind, hipStream_t s, void** token) {
  *token = nullptr;
  if (!g_prof_on) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  ProfRec* p;
  if (!g_prof_free.empty()) {
    p = g_prof_free.back();
    g_prof_free.pop_back();
  } else {
    p = new ProfRec;
    // timing-only events: no system-scope cache writeback and invalidation when they
    // are recorded, so the pair brackets the launch and not a flush around it
    if (hipEventCreateWithFlags(&p->a, hipEventDisableSystemFence) != hipSuccess) {
      delete p;
      return;
    }
    if (hipEventCreateWithFlags(&p->b, hipEventDisableSystemFence) != hipSuccess) {
      (void)hipEventDestroy(p->a);
      delete p;
      return;
    }
  }
  p->kind = kind;
  if (hipEventRecord(p->a, s) != hipSuccess) {
    g_prof_free.push_back(p);
    return;
  }
  *token = p;
}

void prof_end(void* token, hipStream_t s) {
  if (!token) return;
  ProfRec* p = (ProfRec*)token;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (hipEventRecord(p->b, s) != hipSuccess) {
    g_prof_free.push_back(p);
    return;
  }
  g_prof_pending.push_back(p);
}

}  // namespace qnf4

using namespace qnf4;

extern "C" {

int qlora_abi_version(void) { return QLORA_NF4_ABI_VERSION; }

int qlora_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int rc = prof_drain();
  if (on) {
    for (int k = 0; k < QLORA_K_COUNT; ++k) {
      g_prof_ms[k] = 0.0;
      g_prof_n[k] = 0;
    }
  }
  g_prof_on = on != 0;
  return rc == QLORA_OK ? QLORA_OK : set_error(rc, "profile: event wait failed");
}

int qlora_profile_read(int32_t kind, double* ms, int64_t* launches) {
  if (kind < 0 || kind >= QLORA_K_COUNT || !ms || !launches)
    return set_error(QLORA_ERR_INVALID_ARG, "profile_read: bad kind or null output");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int rc = prof_drain();
  *ms = g_prof_ms[kind];
  *launches = g_prof_n[kind];
  return rc == QLORA_OK ? QLORA_OK : set_error(rc, "profile_read: event wait failed");
}

const char* qlora_kernel_name(int32_t kind) {
  return (kind >= 0 && kind < QLORA_K_COUNT) ? kKernelNames[kind] : "";
}

const char* qlora_last_error(void) { return g_err; }

int qlora_nf4_levels(float out[16]) {
  if (!out) return set_error(QLORA_ERR_INVALID_ARG, "levels: null output");
  const Nf4Tables& t = host_tables();
  for (int i = 0; i < 16; ++i) out[i] = t.lv[i];
  return QLORA_OK;
}

int qlora_nf4_quantize(const float* w, qlora_nf4_t* q, void* stream) {
  g_err[0] = 0;
  int rc = validate_desc(q, true, "quantize");
  if (rc) return rc;
  const int64_t n = q->rows * q->cols;
  if (n == 0) return QLORA_OK;
  if (!w) return set_error(QLORA_ERR_INVALID_ARG, "quantize: null weight");
  if (!aligned16(w)) return set_error(QLORA_ERR_INVALID_ARG, "quantize: weight must be 16-byte aligned");
  if ((rc = check_tables("quantize"))) return rc;
  return launch_quantize(w, q, (hipStream_t)stream);
}

int qlora_nf4_dequantize(const qlora_nf4_t* q, int32_t out_dtype, void* out, void* stream) {
  g_err[0] = 0;
  int rc = validate_desc(q, true, "dequantize");
  if (rc) return rc;
  if (!valid_cd(out_dtype)) return set_error(QLORA_ERR_DTYPE, "dequantize: bad dtype %d", out_dtype);
  const int64_t n = q->rows * q->cols;
  if (n == 0) return QLORA_OK;
  if (!out) return set_error(QLORA_ERR_INVALID_ARG, "dequantize: null output");
  if (!aligned16(out)) return set_error(QLORA_ERR_INVALID_ARG, "dequantize: output must be 16-byte aligned");
  if ((rc = check_tables("dequantize"))) return rc;
  return launch_dequantize(q, out_dtype, out, (hipStream_t)stream);
}

size_t qlora_workspace_bytes(int32_t op, int64_t m, int64_t rows, int64_t cols, int32_t r, int32_t cd) {
  if (m < 0 || rows < 0 || cols < 0 || r < 1 || !valid_cd(cd)) return 0;
  const int32_t flags = op >> QLORA_OP_FLAGS_SHIFT;
  op &= (1 << QLORA_OP_FLAGS_SHIFT) - 1;
  if (flags & ~(QLORA_FLAG_RSLORA | QLORA_FLAG_FUSED | QLORA_FLAG_DEQUANT_GEMM | QLORA_FLAG_DROPOUT)) return 0;
  if (op == QLORA_OP_FWD) return fwd_workspace_bytes(m, rows, cols, r, cd, flags);
  if (op == QLORA_OP_FWD_CACHED) {
    if (flags & ~QLORA_FLAG_RSLORA || (cd != CD_BF16 && cd != CD_F16)) return 0;
    return cached_fwd_workspace_bytes(m, rows, cols, r, cd);
  }
  if (op == QLORA_OP_BWD) return bwd_workspace_bytes(m, rows, cols, r, cd, flags);
  return 0;
}

namespace {
int fwd_impl(const qlora_nf4_t* w, const void* x, int64_t m, const void* lora_a, const void* lora_b, int32_t r,
             float alpha, int32_t flags, const void* bias, int32_t cd, const uint8_t* mask, float p, void* y,
             float* t_save, void* ws, size_t ws_bytes, void* stream, const char* who) {
  int rc = validate_layer(w, x, m, lora_a, lora_b, r, alpha, flags, cd, who);
  if (rc) return rc;
  if (!y) return set_error(QLORA_ERR_INVALID_ARG, "%s: null y", who);
  if ((rc = check_aligned(who, "y, bias, t_save and the dropout mask", {y, bias, t_save, mask}))) return rc;
  if (m == 0) return QLORA_OK;
  if (mask) flags |= QLORA_FLAG_DROPOUT;
  if ((rc = check_ws(ws, ws_bytes, fwd_workspace_bytes(m, w->rows, w->cols, r, cd, flags), who))) return rc;
  if ((rc = check_tables(who))) return rc;
  LayerCall c;
  c.w = make_w(w);
  c.cd = cd;
  c.m = m;
  c.r = r;
  c.scale = mask ? (float)((double)lora_scale(alpha, r, flags) / (1.0 - (double)p)) : lora_scale(alpha, r, flags);
  c.flags = flags;
  c.x = x;
  c.drop_mask = mask;
  c.lora_a = lora_a;
  c.lora_b = lora_b;
  c.bias = bias;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return launch_forward(c, y, t_save);
}

int bwd_impl(const qlora_nf4_t* w, const void* x, const void* dy, int64_t m, const void* lora_a,
             const void* lora_b, int32_t r, float alpha, int32_t flags, int32_t cd, const uint8_t* mask, float p,
             const float* t_saved, void* dx, float* d_a, float* d_b, void* ws, size_t ws_bytes, void* stream,
             const char* who) {
  int rc = validate_layer(w, x, m, lora_a, lora_b, r, alpha, flags, cd, who);
  if (rc) return rc;
  if (!dy || !d_a || !d_b) return set_error(QLORA_ERR_INVALID_ARG, "%s: null dy / d_a / d_b", who);
  if ((rc = check_aligned(who, "dy, dx, d_a, d_b, t_saved and the dropout mask", {dy, dx, d_a, d_b, t_saved, mask})))
    return rc;
  if (m == 0) return set_error(QLORA_ERR_SHAPE, "%s: m must be >= 1 (dA, dB would be all zero)", who);
  if (mask) flags |= QLORA_FLAG_DROPOUT;
  if ((rc = check_ws(ws, ws_bytes, bwd_workspace_bytes(m, w->rows, w->cols, r, cd, flags), who))) return rc;
  if ((rc = check_tables(who))) return rc;
  LayerCall c;
  c.w = make_w(w);
  c.cd = cd;
  c.m = m;
  c.r = r;
  c.scale = mask ? (float)((double)lora_scale(alpha, r, flags) / (1.0 - (double)p)) : lora_scale(alpha, r, flags);
  c.flags = flags;
  c.x = x;
  c.drop_mask = mask;
  c.lora_a = lora_a;
  c.lora_b = lora_b;
  c.bias = nullptr;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return launch_backward(c, dy, t_saved, dx, d_a, d_b);
}

int check_dropout(const uint8_t* mask, float p, const char* who) {
  if (!mask) return set_error(QLORA_ERR_INVALID_ARG, "%s: null dropout mask", who);
  if (!(p >= 0.f && p < 1.f)) return set_error(QLORA_ERR_INVALID_ARG, "%s: dropout rate %g outside [0, 1)", who, p);
  return QLORA_OK;
}
}  // namespace

int qlora_linear_fwd(const qlora_nf4_t* w, const void* x, int64_t m, const void* lora_a,
                     const void* lora_b, int32_t r, float alpha, int32_t flags, const void* bias,
                     int32_t cd, void* y, float* t_save, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (flags & QLORA_FLAG_DROPOUT)
    return set_error(QLORA_ERR_INVALID_ARG, "linear_fwd: QLORA_FLAG_DROPOUT belongs to qlora_linear_fwd_dropout");
  return fwd_impl(w, x, m, lora_a, lora_b, r, alpha, flags, bias, cd, nullptr, 0.f, y, t_save, ws, ws_bytes, stream,
                  "linear_fwd");
}

int qlora_linear_fwd_noalloc(const qlora_nf4_t* w, const void* x, int64_t m, const void* lora_a,
                             const void* lora_b, int32_t r, float alpha, int32_t flags, const void* bias,
                             int32_t cd, void* y, float* t_save, void* stream) {
  g_err[0] = 0;
  const char* who = "linear_fwd_noalloc";
  if (flags & QLORA_FLAG_DROPOUT)
    return set_error(QLORA_ERR_INVALID_ARG, "%s: QLORA_FLAG_DROPOUT belongs to qlora_linear_fwd_dropout", who);
  // Above 16 tokens the fused kernels, unless the caller asks for the copy of W~.
  if (!(flags & QLORA_FLAG_DEQUANT_GEMM)) flags |= QLORA_FLAG_FUSED;
  int rc = validate_layer(w, x, m, lora_a, lora_b, r, alpha, flags, cd, who);
  if (rc) return rc;
  const size_t need = fwd_workspace_bytes(m, w->rows, w->cols, r, cd, flags);
  if (need > kScratchBytes)
    return set_error(QLORA_ERR_WORKSPACE, "%s: this call needs %zu bytes of scratch memory, the library holds %zu",
                     who, need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_address(&ws, who))) return rc;
  return fwd_impl(w, x, m, lora_a, lora_b, r, alpha, flags, bias, cd, nullptr, 0.f, y, t_save, ws, kScratchBytes,
                  stream, who);
}

size_t qlora_noalloc_scratch_bytes(void) { return kScratchBytes; }

int qlora_linear_fwd_cached(const void* w_cd, int64_t rows, int64_t cols, const void* x, int64_t m,
                            const void* lora_a, const void* lora_b, int32_t r, float alpha, int32_t flags,
                            const void* bias, int32_t cd, void* y, float* t_save, void* ws, size_t ws_bytes,
                            void* stream) {
  g_err[0] = 0;
  const char* who = "linear_fwd_cached";
  if (cd != CD_BF16 && cd != CD_F16) return set_error(QLORA_ERR_DTYPE, "%s: compute dtype must be bf16 or f16", who);
  if (m < 0 || rows < 1 || cols < 1) return set_error(QLORA_ERR_SHAPE, "%s: bad shape", who);
  if (r < 1) return set_error(QLORA_ERR_INVALID_ARG, "%s: rank r must be >= 1 (got %d)", who, r);
  if (!isfinite(alpha)) return set_error(QLORA_ERR_INVALID_ARG, "%s: alpha must be finite", who);
  if (flags & ~QLORA_FLAG_RSLORA) return set_error(QLORA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", who, flags);
  if (!w_cd || !x || !lora_a || !lora_b || !y)
    return set_error(QLORA_ERR_INVALID_ARG, "%s: null w_cd / x / lora_a / lora_b / y", who);
  int rc = check_aligned(who, "w_cd, x, lora_a, lora_b, y, bias and t_save", {w_cd, x, lora_a, lora_b, y, bias, t_save});
  if (rc) return rc;
  if (cols % 64 != 0)
    return set_error(QLORA_ERR_UNSUPPORTED, "%s: cols (%lld) must be a multiple of 64", who, (long long)cols);
  const int64_t lim = 0x7fff0000LL;
  if (rows * cols * 2 >= lim || m * cols * 2 >= lim)
    return set_error(QLORA_ERR_UNSUPPORTED, "%s: w_cd or x spans 2 GiB or more", who);
  if (m == 0) return QLORA_OK;
  if ((rc = check_ws(ws, ws_bytes, cached_fwd_workspace_bytes(m, rows, cols, r, cd), who))) return rc;
  LayerCall c;
  c.w = Nf4W{};
  c.w.rows = rows;
  c.w.cols = cols;
  c.cd = cd;
  c.m = m;
  c.r = r;
  c.scale = lora_scale(alpha, r, flags);
  c.flags = flags;
  c.x = x;
  c.drop_mask = nullptr;
  c.lora_a = lora_a;
  c.lora_b = lora_b;
  c.bias = bias;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return launch_forward_cached(c, w_cd, y, t_save);
}

int qlora_linear_fwd_dropout(const qlora_nf4_t* w, const void* x, int64_t m, const void* lora_a,
                             const void* lora_b, int32_t r, float alpha, int32_t flags, const void* bias,
                             int32_t cd, const uint8_t* mask, float p, void* y, float* t_save, void* ws,
                             size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int rc = check_dropout(mask, p, "linear_fwd_dropout");
  if (rc) return rc;
  return fwd_impl(w, x, m, lora_a, lora_b, r, alpha, flags, bias, cd, mask, p, y, t_save, ws, ws_bytes, stream,
                  "linear_fwd_dropout");
}

int qlora_linear_bwd(const qlora_nf4_t* w, const void* x, const void* dy, int64_t m,
                     const void* lora_a, const void* lora_b, int32_t r, float alpha, int32_t flags,
                     int32_t cd, const float* t_saved, void* dx, float* d_a, float* d_b, void* ws,
                     size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (flags & QLORA_FLAG_DROPOUT)
    return set_error(QLORA_ERR_INVALID_ARG, "linear_bwd: QLORA_FLAG_DROPOUT belongs to qlora_linear_bwd_dropout");
  return bwd_impl(w, x, dy, m, lora_a, lora_b, r, alpha, flags, cd, nullptr, 0.f, t_saved, dx, d_a, d_b, ws, ws_bytes,
                  stream, "linear_bwd");
}

namespace {
// The group's projections as single-layer calls.  query: a workspace query (shapes
// only, no pointers checked).
int build_group(int32_t g, const qlora_nf4_t* const* w, const void* x, int64_t m, const void* const* lora_a,
                const void* const* lora_b, const int32_t* r, const float* alpha, int32_t flags, int32_t cd,
                void* ws, size_t ws_bytes, void* stream, bool query, const char* who, GroupCall& gc) {
  if (g < 1 || g > QLORA_GROUP_MAX)
    return set_error(QLORA_ERR_INVALID_ARG, "%s: group size %d outside 1 .. %d", who, g, QLORA_GROUP_MAX);
  if (!w || !r || (!query && (!alpha || !lora_a || !lora_b)))
    return set_error(QLORA_ERR_INVALID_ARG, "%s: null array argument", who);
  if (flags & ~QLORA_FLAG_RSLORA)
    return set_error(QLORA_ERR_INVALID_ARG, "%s: flags 0x%x (the group takes QLORA_FLAG_RSLORA only)", who, flags);
  int64_t off = 0, toff = 0;
  gc.g = g;
  for (int i = 0; i < g; ++i) {
    int rc;
    if (query) {
      if (!w[i]) return set_error(QLORA_ERR_INVALID_ARG, "%s: null weight %d", who, i);
      if ((rc = validate_desc(w[i], false, who))) return rc;
      if (!valid_cd(cd)) return set_error(QLORA_ERR_DTYPE, "%s: bad compute dtype %d", who, cd);
      if (m < 0 || r[i] < 1 || w[i]->rows < 1) return set_error(QLORA_ERR_SHAPE, "%s: bad shape", who);
    } else if ((rc = validate_layer(w[i], x, m, lora_a[i], lora_b[i], r[i], alpha[i], flags, cd, who))) {
      return rc;
    }
    if (w[i]->cols != w[0]->cols)
      return set_error(QLORA_ERR_SHAPE, "%s: weight %d has %lld cols, weight 0 %lld", who, i, (long long)w[i]->cols,
                       (long long)w[0]->cols);
    LayerCall& c = gc.c[i];
    c.w = make_w(w[i]);
    c.cd = cd;
    c.m = m;
    c.r = r[i];
    c.scale = query ? 1.f : lora_scale(alpha[i], r[i], flags);
    c.flags = flags;
    c.x = x;
    c.drop_mask = nullptr;
    c.lora_a = query ? nullptr : lora_a[i];
    c.lora_b = query ? nullptr : lora_b[i];
    c.bias = nullptr;
    c.ws = ws;
    c.ws_bytes = ws_bytes;
    c.stream = (hipStream_t)stream;
    gc.off[i] = off;
    gc.toff[i] = toff;
    off += w[i]->rows;
    toff += round_up(r[i], 8);
  }
  gc.off[g] = off;
  gc.toff[g] = toff;
  gc.N = off;
  gc.R8 = toff;
  gc.RP = round_up(toff, 64);
  return QLORA_OK;
}

int check_group_ptrs(const char* who, int32_t g, float* const* a, const char* name) {
  if (!a) return QLORA_OK;
  for (int i = 0; i < g; ++i)
    if (a[i] && !aligned16(a[i])) return set_error(QLORA_ERR_INVALID_ARG, "%s: %s[%d] must be 16-byte aligned", who, name, i);
  return QLORA_OK;
}
}  // namespace

int qlora_linear_fwd_group(int32_t g, const qlora_nf4_t* const* w, const void* x, int64_t m,
                           const void* const* lora_a, const void* const* lora_b, const int32_t* r,
                           const float* alpha, int32_t flags, const void* bias, int32_t cd, void* y,
                           float* const* t_save, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "linear_fwd_group";
  GroupCall gc;
  int rc = build_group(g, w, x, m, lora_a, lora_b, r, alpha, flags, cd, ws, ws_bytes, stream, false, who, gc);
  if (rc) return rc;
  if (!y) return set_error(QLORA_ERR_INVALID_ARG, "%s: null y", who);
  if ((rc = check_aligned(who, "y and bias", {y, bias}))) return rc;
  if ((rc = check_group_ptrs(who, g, t_save, "t_save"))) return rc;
  if (m == 0) return QLORA_OK;
  if ((rc = check_ws(ws, ws_bytes, group_workspace_bytes(QLORA_OP_FWD, gc), who))) return rc;
  if ((rc = check_tables(who))) return rc;
  return launch_forward_group(gc, bias, y, t_save, ws, (hipStream_t)stream);
}

int qlora_linear_bwd_group(int32_t g, const qlora_nf4_t* const* w, const void* x, const void* dy, int64_t m,
                           const void* const* lora_a, const void* const* lora_b, const int32_t* r,
                           const float* alpha, int32_t flags, int32_t cd, const float* const* t_saved,
                           void* dx, float* const* d_a, float* const* d_b, void* ws, size_t ws_bytes,
                           void* stream) {
  g_err[0] = 0;
  const char* who = "linear_bwd_group";
  GroupCall gc;
  int rc = build_group(g, w, x, m, lora_a, lora_b, r, alpha, flags, cd, ws, ws_bytes, stream, false, who, gc);
  if (rc) return rc;
  if (!dy || !d_a || !d_b) return set_error(QLORA_ERR_INVALID_ARG, "%s: null dy / d_a / d_b", who);
  for (int i = 0; i < g; ++i)
    if (!d_a[i] || !d_b[i]) return set_error(QLORA_ERR_INVALID_ARG, "%s: null d_a[%d] / d_b[%d]", who, i, i);
  if ((rc = check_aligned(who, "dy and dx", {dy, dx}))) return rc;
  if ((rc = check_group_ptrs(who, g, d_a, "d_a")) || (rc = check_group_ptrs(who, g, d_b, "d_b")) ||
      (rc = check_group_ptrs(who, g, (float* const*)t_saved, "t_saved")))
    return rc;
  if (m == 0) return set_error(QLORA_ERR_SHAPE, "%s: m must be >= 1 (dA, dB would be all zero)", who);
  if ((rc = check_ws(ws, ws_bytes, group_workspace_bytes(QLORA_OP_BWD, gc), who))) return rc;
  if ((rc = check_tables(who))) return rc;
  return launch_backward_group(gc, dy, t_saved, dx, d_a, d_b, ws, (hipStream_t)stream);
}

size_t qlora_group_workspace_bytes(int32_t op, int32_t g, const qlora_nf4_t* const* w, int64_t m,
                                   const int32_t* r, int32_t cd) {
  if (op != QLORA_OP_FWD && op != QLORA_OP_BWD) return 0;
  GroupCall gc;
  if (build_group(g, w, nullptr, m, nullptr, nullptr, r, nullptr, 0, cd, nullptr, 0, nullptr, true, "group_workspace",
                  gc))
    return 0;
  return group_workspace_bytes(op, gc);
}

int qlora_linear_bwd_dropout(const qlora_nf4_t* w, const void* x, const void* dy, int64_t m,
                             const void* lora_a, const void* lora_b, int32_t r, float alpha, int32_t flags,
                             int32_t cd, const uint8_t* mask, float p, const float* t_saved, void* dx,
                             float* d_a, float* d_b, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int rc = check_dropout(mask, p, "linear_bwd_dropout");
  if (rc) return rc;
  return bwd_impl(w, x, dy, m, lora_a, lora_b, r, alpha, flags, cd, mask, p, t_saved, dx, d_a, d_b, ws, ws_bytes,
                  stream, "linear_bwd_dropout");
}

int qlora_merge(const qlora_nf4_t* w, const void* lora_a, const void* lora_b, int32_t r, float alpha,
                int32_t flags, int32_t cd, void* out, void* stream) {
  g_err[0] = 0;
  int rc = validate_desc(w, true, "merge");
  if (rc) return rc;
  if (!valid_cd(cd)) return set_error(QLORA_ERR_DTYPE, "merge: bad dtype %d", cd);
  if (r < 1) return set_error(QLORA_ERR_INVALID_ARG, "merge: rank r must be >= 1 (got %d)", r);
  if (!isfinite(alpha)) return set_error(QLORA_ERR_INVALID_ARG, "merge: alpha must be finite");
  if (flags & ~QLORA_FLAG_RSLORA) return set_error(QLORA_ERR_INVALID_ARG, "merge: unknown flags 0x%x", flags);
  if (w->rows * w->cols == 0) return QLORA_OK;
  if (!lora_a || !lora_b || !out) return set_error(QLORA_ERR_INVALID_ARG, "merge: null lora_a / lora_b / out");
  if (w->rows > 4194240) return set_error(QLORA_ERR_UNSUPPORTED, "merge: %lld rows (at most 4194240)", (long long)w->rows);
  if ((rc = check_tables("merge"))) return rc;
  return launch_merge(make_w(w), lora_a, lora_b, r, lora_scale(alpha, r, flags), cd, out, (hipStream_t)stream);
}

namespace {
int check_adamw(const qlora_adamw_t* o, int32_t step, const char* who) {
  if (!o) return set_error(QLORA_ERR_INVALID_ARG, "%s: null optimizer settings", who);
  if (step < 1) return set_error(QLORA_ERR_INVALID_ARG, "%s: step must be >= 1 (got %d)", who, step);
  const bool ok = isfinite(o->lr) && o->lr >= 0.f && isfinite(o->beta1) && o->beta1 >= 0.f && o->beta1 < 1.f &&
                  isfinite(o->beta2) && o->beta2 >= 0.f && o->beta2 < 1.f && isfinite(o->eps) && o->eps > 0.f &&
                  isfinite(o->weight_decay) && o->weight_decay >= 0.f;
  if (!ok) return set_error(QLORA_ERR_INVALID_ARG, "%s: AdamW settings out of range", who);
  return QLORA_OK;
}
}  // namespace

int qlora_mse_loss_grad(const void* y, const void* target, int64_t n, int32_t cd, float* loss, void* dy,
                        void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!valid_cd(cd)) return set_error(QLORA_ERR_DTYPE, "mse: bad dtype %d", cd);
  if (n < 0) return set_error(QLORA_ERR_INVALID_ARG, "mse: negative n");
  if (n == 0) return QLORA_OK;
  if (!y || !target || !loss || !dy) return set_error(QLORA_ERR_INVALID_ARG, "mse: null pointer");
  int rc = check_ws(ws, ws_bytes, QLORA_MSE_WORKSPACE_BYTES, "mse");
  if (rc) return rc;
  return launch_mse(y, target, n, cd, loss, dy, (float*)ws, (hipStream_t)stream);
}

int qlora_adamw_step(float* param, const float* grad, float* m, float* v, int64_t n, const qlora_adamw_t* opt,
                     int32_t step, void* param_cd, int32_t cd, void* stream) {
  g_err[0] = 0;
  if (!valid_cd(cd)) return set_error(QLORA_ERR_DTYPE, "adamw: bad dtype %d", cd);
  if (n < 0) return set_error(QLORA_ERR_INVALID_ARG, "adamw: negative n");
  int rc = check_adamw(opt, step, "adamw");
  if (rc) return rc;
  if (n == 0) return QLORA_OK;
  if (!param || !grad || !m || !v) return set_error(QLORA_ERR_INVALID_ARG, "adamw: null pointer");
  return launch_adamw(param, grad, m, v, n, *opt, step, param_cd, cd, (hipStream_t)stream);
}

namespace {
int check_stack(const qlora_stack_layer_t* layers, int32_t L, int64_t m, int32_t r, int32_t cd, const char* who) {
  if (!layers || L < 1) return set_error(QLORA_ERR_SHAPE, "%s: need at least one layer", who);
  if (m < 1) return set_error(QLORA_ERR_SHAPE, "%s: m must be >= 1", who);
  if (r < 1) return set_error(QLORA_ERR_INVALID_ARG, "%s: rank r must be >= 1", who);
  if (!valid_cd(cd)) return set_error(QLORA_ERR_DTYPE, "%s: bad dtype %d", who, cd);
  for (int l = 0; l < L; ++l) {
    if (!layers[l].w) return set_error(QLORA_ERR_INVALID_ARG, "%s: layer %d has no weight", who, l);
    if (l && layers[l].w->cols != layers[l - 1].w->rows)
      return set_error(QLORA_ERR_SHAPE, "%s: layer %d takes %lld inputs, layer %d gives %lld", who, l,
                       (long long)layers[l].w->cols, l - 1, (long long)layers[l - 1].w->rows);
  }
  return QLORA_OK;
}
}  // namespace

size_t qlora_stack_workspace_bytes(const qlora_stack_layer_t* layers, int32_t n_layers, int64_t m, int32_t r,
                                   int32_t cd, int32_t flags) {
  if (check_stack(layers, n_layers, m, r, cd, "stack_workspace")) return 0;
  if (flags & ~(QLORA_FLAG_RSLORA | QLORA_FLAG_FUSED | QLORA_FLAG_DEQUANT_GEMM)) return 0;
  return stack_workspace_bytes(layers, n_layers, m, r, cd, flags);
}

int qlora_stack_train_step(const qlora_stack_layer_t* layers, int32_t n_layers, const void* x, int64_t m,
                           const void* target, int32_t r, float alpha, int32_t flags, int32_t cd,
                           const qlora_adamw_t* opt, int32_t step, float* loss, void* ws, size_t ws_bytes,
                           void* stream) {
  g_err[0] = 0;
  int rc = check_stack(layers, n_layers, m, r, cd, "stack_step");
  if (rc) return rc;
  if (!x || !target || !loss) return set_error(QLORA_ERR_INVALID_ARG, "stack_step: null x / target / loss");
  if (flags & QLORA_FLAG_DROPOUT) return set_error(QLORA_ERR_INVALID_ARG, "stack_step: no dropout in the stack step");
  if ((rc = check_adamw(opt, step, "stack_step"))) return rc;
  for (int l = 0; l < n_layers; ++l) {
    const qlora_stack_layer_t& S = layers[l];
    if ((rc = validate_layer(S.w, x, m, S.lora_a, S.lora_b, r, alpha, flags, cd, "stack_step"))) return rc;
    if (!S.a32 || !S.b32 || !S.m_a || !S.v_a || !S.m_b || !S.v_b || !S.grad_a || !S.grad_b)
      return set_error(QLORA_ERR_INVALID_ARG, "stack_step: layer %d has a null adapter buffer", l);
  }
  if ((rc = check_ws(ws, ws_bytes, stack_workspace_bytes(layers, n_layers, m, r, cd, flags), "stack_step")))
    return rc;
  if ((rc = check_tables("stack_step"))) return rc;
  return launch_stack_step(layers, n_layers, x, m, target, r, lora_scale(alpha, r, flags), flags, cd, *opt, step,
                           loss, ws, (hipStream_t)stream);
}

}  // extern "C"
