// group.hip -- projections that read the same input (q / k / v of an attention
// block, gate / up of an MLP) in one call, on gfx950:
//
//   forward   y [m, N] = [y_0 | y_1 | ...],  y_i = x W~_i^T + s_i (x A_i^T) B_i^T (+ bias)
//   backward  dX = sum_i (dY_i W~_i + dT_i A_i),  dT_i = s_i dY_i B_i,
//             dA_i = dT_i^T x,  dB_i = s_i dY_i^T T0_i
//
// ("LoRA and QLoRA, mathematically", "Rank, alpha, and target modules": the adapted
// modules of a block; each projection is the layer of gemm.hip.)
//
// Tiled path (bf16 / f16, more than 64 tokens, every W_i on the tiled layouts with
// rows a multiple of 64, r_i <= 64): the projections' W~ are written side by side
// into one workspace matrix, their rank products into column slices of one operand,
// and a single 256 x 256 dense GEMM runs over the concatenation:
//   forward  y = [x | T] [W~ | B]^T with T = [s_0 T0_0 | s_1 T0_1 | ...] (each slice
//            r_i rounded up to 8 columns) and B block-diagonal (row n of projection i
//            holds B_i[n] in the columns of T_i, zeros elsewhere), so every output
//            column sees exactly its own projection's low-rank term;
//   dX       dX = [dY | dT] [W~ ; A] with W~^T [cols][N] written slice by slice and A
//            stacked (A^T slices side by side): the contraction runs over every
//            projection's rows and T's slices in one fp32 accumulation.
// Small projections (k / v) then share the rounds of large ones instead of running
// short cut launches, and the block's last round is cut once.  Otherwise each
// projection runs through the single-layer call into the workspace and small
// kernels place its output columns (forward) or add its dX in fp32 (backward).
#include <algorithm>

#include "common.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;

struct DiagArgs {
  const void* b[kGroupMax];   // lora_b of projection i [rows_i][r_i]
  int64_t off[kGroupMax + 1]; // first row of projection i; off[g] = N
  int32_t toff[kGroupMax];    // first column of projection i's slice
  int32_t r[kGroupMax];
  int32_t g;
  int64_t N;
  int32_t R8;                 // columns of the block-diagonal matrix
};

// bd [N][R8] (cd): row n of projection i holds B_i[n - off_i] in columns toff_i ..
// toff_i + r_i, zeros elsewhere.  One thread per 8 columns (one 16-byte store).
template <int CD>
__global__ __launch_bounds__(kThreads) void k_block_diag(DiagArgs a, void* __restrict__ bd) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t chunks = a.R8 / 8;
  const int64_t n = idx / chunks, t0 = (idx - n * chunks) * 8;
  if (n >= a.N) return;
  int i = 0;
  for (int k = 1; k < a.g; ++k) i = n >= a.off[k] ? k : i;
  const int64_t row = n - a.off[i];
  const int64_t t = t0 - a.toff[i];  // column within the slice (a multiple of 8)
  u32x4_t o = {0u, 0u, 0u, 0u};
  if (t >= 0 && t + 8 <= a.r[i] && (a.r[i] & 7) == 0) {
    o = *(const u32x4_t*)((const uint16_t*)a.b[i] + row * a.r[i] + t);  // 16-byte aligned: r % 8 == 0
  } else if (t >= 0 && t < a.r[i]) {
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t + e < a.r[i] ? ((const uint16_t*)a.b[i])[row * a.r[i] + t + e] : (uint16_t)0;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (uint32_t)v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
  }
  *(u32x4_t*)((uint16_t*)bd + n * a.R8 + t0) = o;
}

// dst[row * ld_dst + c] = src[row * ld_src + c] for row < rows, c < cols (elements of
// ES bytes): a projection's columns into or out of the concatenated matrix.
template <int ES>
__global__ __launch_bounds__(kThreads) void k_copy_cols(const void* __restrict__ src, int64_t ld_src,
                                                        void* __restrict__ dst, int64_t ld_dst, int64_t rows,
                                                        int64_t cols) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = idx / cols, c = idx - row * cols;
  if (row >= rows) return;
  if constexpr (ES == 2) ((uint16_t*)dst)[row * ld_dst + c] = ((const uint16_t*)src)[row * ld_src + c];
  else ((uint32_t*)dst)[row * ld_dst + c] = ((const uint32_t*)src)[row * ld_src + c];
}

// acc = (first ? 0 : acc) + v in fp32; on the last term also out = cd(acc).
template <int CD>
__global__ __launch_bounds__(kThreads) void k_acc_terms(const void* __restrict__ v, float* __restrict__ acc,
                                                        void* __restrict__ out, int64_t n, int first, int last) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= n) return;
  const float s = (first ? 0.f : acc[e]) + load_cd<CD>(v, e);
  if (last) store_cd<CD>(out, e, s);
  else acc[e] = s;
}

int64_t al(int64_t b) { return round_up(b, 256); }

// The tiled path's concatenated call: W~ [N, cols] (or [cols][N] for dX) with the
// first projection's layout, rank R8, the workspace's operands.
LayerCall concat_call(const GroupCall& gc) {
  LayerCall c = gc.c[0];
  c.w.rows = gc.N;
  c.r = (int32_t)gc.R8;
  c.scale = 1.f;
  c.lora_a = nullptr;
  c.lora_b = nullptr;
  c.bias = nullptr;
  return c;
}

bool tiled(const GroupCall& gc, bool dx) {
  const LayerCall& c0 = gc.c[0];
  if ((c0.cd != CD_BF16 && c0.cd != CD_F16) || c0.m <= 64 || gc.RP > 512) return false;
  for (int i = 0; i < gc.g; ++i) {
    const LayerCall& c = gc.c[i];
    if (!fast_layout(c.w) || c.w.rows % 64 || !skinny_ok(c.cd, c.r) || !dense256_ok(c, false) ||
        !dense256_ok(c, true))
      return false;
  }
  return dense256_ok(concat_call(gc), dx);
}

// Workspace plans.  Tiled forward: W~ [N][cols], T [m][RP], the block-diagonal B
// [N][R8], every projection's rank-product partial sums, the cut last round's
// partial sums.
struct GFwd {
  bool tiled;
  int64_t wd, tcd, bd, part, part_each, split, single, tmp, total;
  DenseSplit sp;
};
GFwd plan_gfwd(const GroupCall& gc) {
  GFwd P = {};
  const LayerCall& c0 = gc.c[0];
  const int64_t m = c0.m, K = c0.w.cols, es = cd_bytes(c0.cd);
  P.tiled = tiled(gc, false);
  int64_t o = 0;
  if (P.tiled) {
    P.wd = o; o += al(gc.N * K * es);
    P.tcd = o; o += al(m * gc.RP * es);
    P.bd = o; o += al(gc.N * gc.R8 * es);
    P.part_each = al((int64_t)skinny_part_bytes(m, K));
    P.part = o; o += gc.g * P.part_each;
    P.sp = dense_split(m, gc.N, K);
    P.split = o; o += al((int64_t)dense_split_bytes(P.sp));
  } else {
    int64_t single = 0, rows = 0;
    for (int i = 0; i < gc.g; ++i) {
      const LayerCall& c = gc.c[i];
      single = std::max<int64_t>(single, (int64_t)fwd_workspace_bytes(m, c.w.rows, K, c.r, c.cd, c.flags));
      rows = std::max<int64_t>(rows, c.w.rows);
    }
    P.tmp = o; o += al(m * rows * es);
    P.single = o; o += al(single);
  }
  P.total = o;
  return P;
}

// Tiled backward: W~^T [cols][N], dT [m][RP], A^T [cols][RP], per projection dT^T
// and T0^T [r_i][m64], one B^T and one recomputed T0 at a time, the rank-product
// partial sums (two products at once), the dX GEMM's cut round.
struct GBwd {
  bool tiled;
  int64_t wdt, dtcd, at, dtt[kGroupMax], t0t[kGroupMax], bt, t0, part, part2, split;
  int64_t single, dy, dxi, acc, total;
  DenseSplit sp;
};
GBwd plan_gbwd(const GroupCall& gc) {
  GBwd P = {};
  const LayerCall& c0 = gc.c[0];
  const int64_t m = c0.m, K = c0.w.cols, es = cd_bytes(c0.cd), m64 = round_up(m, 64);
  P.tiled = tiled(gc, true);
  int64_t o = 0;
  if (P.tiled) {
    P.wdt = o; o += al(K * gc.N * es);
    P.dtcd = o; o += al(m * gc.RP * es);
    P.at = o; o += al(K * gc.RP * es);
    int64_t bt = 0, part = (int64_t)skinny_part_bytes(m, K), part2 = 0;
    for (int i = 0; i < gc.g; ++i) {
      const LayerCall& c = gc.c[i];
      const int64_t n64 = round_up(c.w.rows, 64);
      P.dtt[i] = o; o += al(c.r * m64 * es);
      P.t0t[i] = o; o += al(c.r * m64 * es);
      bt = std::max<int64_t>(bt, c.r * n64 * es);
      part = std::max<int64_t>(part, (int64_t)skinny_part_bytes(m, n64));   // dT
      part = std::max<int64_t>(part, (int64_t)skinny_part_bytes(K, m64));   // dA
      part2 = std::max<int64_t>(part2, (int64_t)skinny_part_bytes(c.w.rows, m64));  // dB
    }
    P.bt = o; o += al(bt);
    P.t0 = o; o += al(m * 64 * 4);
    P.part = o; o += al(part);
    P.part2 = o; o += al(part2);
    P.sp = dense_split(m, K, gc.N);
    P.split = o; o += al((int64_t)dense_split_bytes(P.sp));
  } else {
    int64_t single = 0, rows = 0;
    for (int i = 0; i < gc.g; ++i) {
      const LayerCall& c = gc.c[i];
      single = std::max<int64_t>(single, (int64_t)bwd_workspace_bytes(m, c.w.rows, K, c.r, c.cd, c.flags));
      rows = std::max<int64_t>(rows, c.w.rows);
    }
    P.dy = o; o += al(m * rows * es);
    P.dxi = o; o += al(m * K * es);
    P.acc = o; o += al(m * K * 4);
    P.single = o; o += al(single);
  }
  P.total = o;
  return P;
}

int copy_cols(int cd, const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t rows, int64_t cols,
              hipStream_t s) {
  const int64_t n = rows * cols;
  if (n == 0) return QLORA_OK;
  const dim3 g((unsigned)ceil_div(n, kThreads)), b(kThreads);
  if (cd_bytes(cd) == 2) k_copy_cols<2><<<g, b, 0, s>>>(src, ld_src, dst, ld_dst, rows, cols);
  else k_copy_cols<4><<<g, b, 0, s>>>(src, ld_src, dst, ld_dst, rows, cols);
  return check_launch("k_copy_cols");
}

int acc_terms(int cd, const void* v, float* acc, void* out, int64_t n, bool first, bool last, hipStream_t s) {
  const dim3 g((unsigned)ceil_div(n, kThreads)), b(kThreads);
  if (cd == CD_BF16) k_acc_terms<CD_BF16><<<g, b, 0, s>>>(v, acc, out, n, first, last);
  else if (cd == CD_F16) k_acc_terms<CD_F16><<<g, b, 0, s>>>(v, acc, out, n, first, last);
  else k_acc_terms<CD_F32><<<g, b, 0, s>>>(v, acc, out, n, first, last);
  return check_launch("k_acc_terms");
}

// Columns of the cd copy of projection i's rank slice that its reduction writes:
// its r_i rounded up to 8, and for the last projection the zero columns up to RP.
int64_t slice_width(const GroupCall& gc, int i) {
  return i + 1 < gc.g ? gc.toff[i + 1] - gc.toff[i] : gc.RP - gc.toff[i];
}

}  // namespace

size_t group_workspace_bytes(int op, const GroupCall& gc) {
  return (size_t)(op == QLORA_OP_BWD ? plan_gbwd(gc).total : plan_gfwd(gc).total);
}

int launch_forward_group(const GroupCall& gc, const void* bias, void* y, float* const* t_save, void* ws,
                         hipStream_t s) {
  const GFwd P = plan_gfwd(gc);
  char* w = (char*)ws;
  const LayerCall& c0 = gc.c[0];
  const int64_t m = c0.m, K = c0.w.cols, es = cd_bytes(c0.cd);
  int rc;
  if (!P.tiled) {
    // each projection by itself: the decode GEMV writes its columns of y in place (row
    // stride N), the other forwards into the workspace and a copy places them
    for (int i = 0; i < gc.g; ++i) {
      LayerCall c = gc.c[i];
      c.bias = bias ? (const char*)bias + gc.off[i] * es : nullptr;
      c.ws = w + P.single;
      if (gemv_route(c)) {
        c.ldy = gc.N;
        if ((rc = launch_forward(c, (char*)y + gc.off[i] * es, t_save ? t_save[i] : nullptr))) return rc;
        continue;
      }
      if ((rc = launch_forward(c, w + P.tmp, t_save ? t_save[i] : nullptr))) return rc;
      if ((rc = copy_cols(c.cd, w + P.tmp, c.w.rows, (char*)y + gc.off[i] * es, gc.N, m, c.w.rows, s))) return rc;
    }
    return QLORA_OK;
  }
  // T_i = s_i x A_i^T into its slice of T: the group's products in one launch (they
  // read the same x), their reductions riding on one dequantize launch that writes
  // each W~_i into rows off_i .. of the concatenated W~
  SkSpec specs[kGroupMax];
  float* parts[kGroupMax];
  int Ss[kGroupMax];
  for (int i = 0; i < gc.g; ++i) {
    const LayerCall& c = gc.c[i];
    specs[i].a = c.x;
    specs[i].lda = K;
    specs[i].arows = m;
    specs[i].b = c.lora_a;
    specs[i].ldb = K;
    specs[i].P = m;
    specs[i].R = c.r;
    specs[i].Kc = K;
    parts[i] = (float*)(w + P.part + i * P.part_each);
  }
  if ((rc = skinny_many(c0.cd, specs, parts, Ss, gc.g, s, QLORA_K_LORA_DOWN))) return rc;
  Nf4W wts[kGroupMax];
  void* outs[kGroupMax];
  SkRed reds[kGroupMax];
  for (int i = 0; i < gc.g; ++i) {
    const LayerCall& c = gc.c[i];
    SkRed& red = reds[i];
    red.part = parts[i];
    red.S = Ss[i];
    red.P = m;
    red.R = c.r;
    red.out32 = t_save ? t_save[i] : nullptr;
    red.sccd = c.scale;
    red.outcd = w + P.tcd + gc.toff[i] * es;
    red.ldcd = gc.RP;
    red.wcd = slice_width(gc, i);
    wts[i] = c.w;
    outs[i] = w + P.wd + gc.off[i] * K * es;
  }
  if ((rc = dequant_group_into(wts, gc.g, c0.cd, outs, reds, s))) return rc;
  DiagArgs a = {};
  a.g = gc.g;
  a.N = gc.N;
  a.R8 = (int32_t)gc.R8;
  for (int i = 0; i < gc.g; ++i) {
    a.b[i] = gc.c[i].lora_b;
    a.off[i] = gc.off[i];
    a.toff[i] = (int32_t)gc.toff[i];
    a.r[i] = gc.c[i].r;
  }
  a.off[gc.g] = gc.N;
  {
    ProfScope prof(QLORA_K_REDUCE, s);
    const dim3 g((unsigned)ceil_div(gc.N * (gc.R8 / 8), kThreads)), b(kThreads);
    if (c0.cd == CD_BF16) k_block_diag<CD_BF16><<<g, b, 0, s>>>(a, w + P.bd);
    else k_block_diag<CD_F16><<<g, b, 0, s>>>(a, w + P.bd);
    if ((rc = check_launch("k_block_diag"))) return rc;
  }
  LayerCall cc = concat_call(gc);
  cc.lora_b = w + P.bd;
  cc.bias = bias;
  return dense256_forward(cc, w + P.wd, w + P.tcd, gc.RP, y, P.sp, w + P.split);
}

int launch_backward_group(const GroupCall& gc, const void* dy, const float* const* t_saved, void* dx,
                          float* const* d_a, float* const* d_b, void* ws, hipStream_t s) {
  const GBwd P = plan_gbwd(gc);
  char* w = (char*)ws;
  const LayerCall& c0 = gc.c[0];
  const int64_t m = c0.m, K = c0.w.cols, es = cd_bytes(c0.cd), m64 = round_up(m, 64);
  int rc;
  if (!P.tiled) {
    for (int i = 0; i < gc.g; ++i) {
      LayerCall c = gc.c[i];
      c.ws = w + P.single;
      if ((rc = copy_cols(c.cd, (const char*)dy + gc.off[i] * es, gc.N, w + P.dy, c.w.rows, m, c.w.rows, s)))
        return rc;
      if ((rc = launch_backward(c, w + P.dy, t_saved ? t_saved[i] : nullptr, dx ? w + P.dxi : nullptr, d_a[i],
                                d_b[i])))
        return rc;
      if (dx && (rc = acc_terms(c.cd, w + P.dxi, (float*)(w + P.acc), dx, m * K, i == 0, i + 1 == gc.g, s)))
        return rc;
    }
    return QLORA_OK;
  }
  float* part = (float*)(w + P.part);
  float* part2 = (float*)(w + P.part2);
  for (int i = 0; i < gc.g; ++i) {
    const LayerCall& c = gc.c[i];
    const int64_t Ni = c.w.rows, n64 = round_up(Ni, 64);
    const void* dyi = (const char*)dy + gc.off[i] * es;
    // T0_i = x A_i^T (the forward's, or recomputed)
    const float* T0 = t_saved ? t_saved[i] : nullptr;
    if (!T0) {
      int S;
      if ((rc = skinny(c.cd, false, c.x, K, m, c.lora_a, K, m, c.r, K, part, &S, s, QLORA_K_LORA_DOWN))) return rc;
      if ((rc = skinny_reduce(c.cd, part, S, m, c.r, 1.0f, (float*)(w + P.t0), false, 0.f, nullptr, 0, s))) return rc;
      T0 = (const float*)(w + P.t0);
    }
    // A_i^T into its slice of the stacked A^T [cols][RP]
    TransposeSpec ta;
    ta.src = c.lora_a;
    ta.ld_src = K;
    ta.rows = c.r;
    ta.cols = K;
    ta.dst = w + P.at + gc.toff[i] * es;
    ta.ld_dst = gc.RP;
    ta.w_dst = slice_width(gc, i);
    // dT_i = s_i dY_i B_i: its slice of dT (cd) for the dX GEMM's tail, dT_i^T and T0_i^T
    // for dA_i and dB_i; the reduction rides on W_i's transposed dequantize.  lora_b_i
    // is read as stored when r_i is a multiple of 8 (A_i^T's transpose then rides on
    // the same launch), else through B_i^T [r_i][n64]
    SkSpec sd;
    sd.a = dyi;
    sd.lda = gc.N;
    sd.arows = m;
    sd.P = m;
    sd.R = c.r;
    sd.Kc = n64;
    const TransposeSpec* ride = nullptr;
    if (c.r % 8 == 0) {
      sd.b = c.lora_b;
      sd.ldb = c.r;
      sd.bt = true;
      sd.brows = Ni;
      ride = &ta;
    } else {
      TransposeSpec tb;
      tb.src = c.lora_b;
      tb.ld_src = c.r;
      tb.rows = Ni;
      tb.cols = c.r;
      tb.dst = w + P.bt;
      tb.ld_dst = n64;
      if ((rc = transpose_jobs(c.cd, tb, &ta, s))) return rc;
      sd.b = w + P.bt;
      sd.ldb = n64;
    }
    int S;
    if ((rc = skinny_jobs(c.cd, false, sd, part, &S, nullptr, nullptr, nullptr, s, QLORA_K_BWD_DT, ride))) return rc;
    SkRed red;
    red.part = part;
    red.S = S;
    red.P = m;
    red.R = c.r;
    red.sccd = c.scale;
    red.outcd = w + P.dtcd + gc.toff[i] * es;
    red.ldcd = gc.RP;
    red.wcd = slice_width(gc, i);
    red.outt = w + P.dtt[i];
    red.ldt = m64;
    red.side = T0;
    red.side_t = w + P.t0t[i];
    if (dx) {
      if ((rc = dequant_into(c.w, c.cd, w + P.wdt + gc.off[i] * es, true, s, &red, gc.N))) return rc;
    } else if ((rc = skinny_reduce_jobs(c.cd, red, nullptr, s))) {
      return rc;
    }
  }
  if (dx) {
    LayerCall cc = concat_call(gc);
    if ((rc = dense256_dx(cc, dy, w + P.wdt, w + P.dtcd, gc.RP, dx, P.sp, w + P.split, w + P.at))) return rc;
  }
  // dA_i = dT_i^T x and dB_i = s_i dY_i^T T0_i: both products in one launch, both
  // reductions in the next
  for (int i = 0; i < gc.g; ++i) {
    const LayerCall& c = gc.c[i];
    SkSpec pa, pb;
    pa.a = c.x;
    pa.lda = K;
    pa.arows = m;
    pa.b = w + P.dtt[i];
    pa.ldb = m64;
    pa.P = K;
    pa.R = c.r;
    pa.Kc = m64;
    pb.a = (const char*)dy + gc.off[i] * es;
    pb.lda = gc.N;
    pb.arows = m;
    pb.b = w + P.t0t[i];
    pb.ldb = m64;
    pb.P = c.w.rows;
    pb.R = c.r;
    pb.Kc = m64;
    int Sa, Sb;
    if ((rc = skinny_jobs(c.cd, true, pa, part, &Sa, &pb, part2, &Sb, s, QLORA_K_BWD_DA))) return rc;
    SkRed ra, rb;
    ra.part = part;
    ra.S = Sa;
    ra.P = K;
    ra.R = c.r;
    ra.out32 = d_a[i];
    ra.trans = true;
    rb.part = part2;
    rb.S = Sb;
    rb.P = c.w.rows;
    rb.R = c.r;
    rb.sc32 = c.scale;
    rb.out32 = d_b[i];
    if ((rc = skinny_reduce_jobs(c.cd, ra, &rb, s))) return rc;
  }
  return QLORA_OK;
}

}  // namespace qnf4
