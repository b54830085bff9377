/*
 * qlora_nf4.h -- C ABI of libqlora_nf4.so: the QLoRA NF4 linear layer on AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (pages: qlora-rs README "Honest capability matrix" and "Quick Start";
 * rust_ai_core QLoraConfig docs; "LoRA and QLoRA, mathematically"):
 *
 *   W  [rows, cols] fp32, frozen, stored as NF4: the flattened weight is cut into
 *      blocks of block_size consecutive elements; each block keeps its absmax a_b
 *      and every element its 4-bit code = the nearest of 16 normal-quantile levels
 *      L[0..15] to w / a_b (ties to the lower code).  Two codes share a byte,
 *      element 2k in the high nibble.  With double quantization the block scales
 *      are themselves stored as u8 q_b with one fp32 scale S per group of dq_group
 *      consecutive blocks: S = fl32(max a / 255), q_b = round-half-even(a_b / S).
 *   deq  w_hat = fl32(L[code] * s_b) with s_b = a_b, or fl32(q_b * S) with DQ.
 *   fwd  y = x W~^T + s (x A^T) B^T (+ bias),  W~ = deq(W) rounded to the compute
 *        dtype, s = alpha / r (alpha / sqrt(r) with QLORA_FLAG_RSLORA).
 *   bwd  with W frozen: dT = s dY B, dX = dY W~ + dT A, dA = dT^T x,
 *        dB = s dY^T T0 where T0 = x A^T.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates or frees device memory.  Matrices are row-major and dense.
 *     The fp32 weight and the codes of quantize / dequantize, the dequantized
 *     output, and every array of a layer call (x, dy, adapters, bias, outputs,
 *     masks, saved T0, gradients) start on a 16-byte boundary: the kernels move
 *     16-byte vectors, and an unaligned pointer is refused with
 *     QLORA_ERR_INVALID_ARG.  Workspaces are 256-byte aligned.  The merge, MSE
 *     and AdamW calls take any element-aligned arrays.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = null stream).
 *   - Arguments are validated on the host before anything is launched: on any
 *     error nothing is written and no work is queued.  Errors: a negative
 *     qlora_status_t; qlora_last_error() (thread-local) gives the reason.
 *   - Launch failures surface as QLORA_ERR_HIP.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_NF4_ABI_VERSION 1

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_INVALID_ARG = -1, /* null pointer, r < 1, non-finite alpha, bad enum   */
  QLORA_ERR_SHAPE = -2,       /* n % block_size != 0, odd block_size, empty dims     */
  QLORA_ERR_DTYPE = -3,       /* dtype not one of qlora_dtype_t                      */
  QLORA_ERR_UNSUPPORTED = -4, /* valid layer outside what the kernels implement      */
  QLORA_ERR_WORKSPACE = -5,   /* workspace too small (see qlora_workspace_bytes)     */
  QLORA_ERR_HIP = -6          /* a HIP launch failed                                 */
} qlora_status_t;

/* Compute / storage dtype of activations, adapters and outputs. */
typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1, QLORA_F16 = 2 } qlora_dtype_t;

/* Flags for the forward / backward calls.  The two path flags (at most one) pick
 * how W~ meets the activations when m > 16 (m <= 16 always takes the decode GEMV;
 * without a path flag, 17 to 64 tokens take its MFMA form where it applies):
 *   default                  the forward of 65 to 768 tokens with r a multiple
 *                            of 8 takes the fused kernels (faster there: W~ is
 *                            not written and read back); every other call with
 *                            m > 16 takes dequantize-then-GEMM
 *   QLORA_FLAG_FUSED         the fused kernels decode W~ on the fly, tile by tile
 *                            (no dequantized copy of W anywhere)
 *   QLORA_FLAG_DEQUANT_GEMM  W~ (forward) or W~^T (dX) is first written in cd into
 *                            the workspace, then a dense GEMM reads it; the copy
 *                            lives only in the workspace, for the call.
 * Both paths give the same W~ bits; the sums differ only in accumulation order. */
enum {
  QLORA_FLAG_RSLORA = 1,       /* scale = alpha / sqrt(r) instead of alpha / r */
  QLORA_FLAG_FUSED = 2,
  QLORA_FLAG_DEQUANT_GEMM = 4,
  QLORA_FLAG_DROPOUT = 8       /* workspace queries only: size for the *_dropout calls */
};

/* Workspace queries: op is QLORA_OP_FWD, QLORA_OP_BWD or QLORA_OP_FWD_CACHED, OR'ed with the call's
 * flags shifted left by QLORA_OP_FLAGS_SHIFT (the path decides the size). */
enum { QLORA_OP_FWD = 0, QLORA_OP_BWD = 1, QLORA_OP_FWD_CACHED = 2, QLORA_OP_FLAGS_SHIFT = 8 };

/*
 * An NF4-quantized frozen weight W [rows, cols].  Descriptor memory is the
 * caller's; the pointers inside are device pointers the caller allocated:
 *   codes          u8   [rows*cols/2]        two 4-bit codes per byte, high nibble first
 *   absmax         f32  [nb]                 when double_quant == 0 (else NULL)
 *   absmax_q       u8   [nb]                 when double_quant != 0 (else NULL)
 *   absmax_scale2  f32  [ceil(nb/dq_group)]  when double_quant != 0 (else NULL)
 * with nb = rows*cols/block_size.  Blocks run over the flattened tensor.
 */
typedef struct {
  int64_t rows;
  int64_t cols;
  int32_t block_size;   /* any even size; powers of two from 8 to 512 take the vectorized kernels */
  int32_t double_quant; /* 0 or 1 */
  int32_t dq_group;     /* blocks per second-level scale when double_quant (>= 1; a value
                           >= rows*cols/block_size gives one scale for the whole tensor) */
  int32_t reserved;     /* must be 0 */
  uint8_t* codes;
  float* absmax;
  uint8_t* absmax_q;
  float* absmax_scale2;
} qlora_nf4_t;

/*
 * Quantize W (device fp32 [q->rows * q->cols], row-major) into *q: per-block absmax,
 * nearest NF4 level of w / absmax (binary32 division, correctly rounded), nibble
 * packing and, if q->double_quant, the u8 + fp32 encoding of the block scales.
 * Pages: qlora-rs README "Honest capability matrix" (NF4 pack/unpack, block absmax,
 * double quant that drops the resident fp32 scales) and "NF4 Quantization".
 * Writes q->codes and either q->absmax or q->absmax_q + q->absmax_scale2.  Block
 * sizes that are powers of two from 8 to 512 run on a vectorized kernel (groups of
 * up to 4096 blocks are encoded in one pass over W; larger ones, one group for the
 * whole tensor included: the "global" scale-of-scales, take a second pass); every
 * other even block size on a one-wavefront-per-block kernel (with double
 * quantization in two passes).  The results are the same bits either way.
 * An empty tensor (rows * cols == 0) is a no-op that returns QLORA_OK.
 * Errors: QLORA_ERR_SHAPE (n % block_size, odd block_size, negative dims),
 * QLORA_ERR_INVALID_ARG (null or unaligned pointers, reserved != 0).
 * NaN / Inf in W are outside the contract (codes are then unspecified, no fault).
 */
int qlora_nf4_quantize(const float* w, qlora_nf4_t* q, void* stream);

/*
 * Dequantize *q into out [rows, cols] of dtype out_dtype: w_hat = fl32(L[c] * s_b),
 * then rounded to nearest-even into bf16 / f16 (fp32 is stored as is).
 * Pages: qlora-rs README "Honest capability matrix" (dequant honours compute_dtype).
 * Errors: QLORA_ERR_DTYPE, QLORA_ERR_SHAPE, QLORA_ERR_INVALID_ARG.
 */
int qlora_nf4_dequantize(const qlora_nf4_t* q, int32_t out_dtype, void* out, void* stream);

/*
 * Forward of the QLoRA linear layer:
 *   y [m, rows] = x [m, cols] . W~^T + s (x . A^T) . B^T (+ bias [rows])
 * x, lora_a [r, cols], lora_b [rows, r], bias, y are in dtype cd; accumulation is
 * fp32.  t_save (nullable) receives T0 = x A^T in fp32 [m, r] for the backward.
 * Pages: qlora-rs README "Quick Start" (QuantizedLinear::forward) and "Honest
 * capability matrix"; rust_ai_core QLoraConfig scale() = alpha / r; "LoRA and QLoRA,
 * mathematically" eq. (6.3.6) and "Tooling" (dequant fused with the matmul).
 * How W~ meets x (see the path flags): m <= 16 runs the decode GEMV (split
 * contraction, W~ decoded in registers; 17 to 64 tokens too when no path flag is
 * given and cols is a multiple of 1024); from 65 to 768 tokens with r a multiple
 * of 8, by default, the fused 256 x 256 MFMA GEMM decodes W~ tile by tile; above
 * that W~ is dequantized once into the workspace and a dense 256 x 256 MFMA GEMM
 * reads it (dequantize-then-GEMM).  The path flags force either.  These kernels take bf16 / f16 layers whose block size is a multiple of
 * 32 dividing cols, with cols a multiple of 64.  Every other layer (f32, any even
 * block size, any cols, blocks that run across rows) runs on a generic MFMA tile
 * engine that decodes W~ per element: the same W~ bits, the sums in another order.
 * ws: device workspace of at least qlora_workspace_bytes(QLORA_OP_FWD, ...) bytes,
 * 256-byte aligned.  m == 0 is a no-op.  Errors: QLORA_ERR_INVALID_ARG (null
 * x/lora_a/lora_b/y, unaligned pointers, r < 1, non-finite alpha, unknown flags,
 * both path flags), QLORA_ERR_SHAPE (m < 0, empty weight), QLORA_ERR_DTYPE,
 * QLORA_ERR_WORKSPACE, QLORA_ERR_UNSUPPORTED (a buffer beyond the kernels' 32-bit
 * offsets, where no generic form exists).
 */
int qlora_linear_fwd(const qlora_nf4_t* w, const void* x, int64_t m, const void* lora_a,
                     const void* lora_b, int32_t r, float alpha, int32_t flags,
                     const void* bias, int32_t cd, void* y, float* t_save, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * Backward of the same layer with the base weight frozen (only A and B train):
 *   dT = s dY B,  dX = dY W~ + dT A  [m, cols] (cd; skipped when dx == NULL),
 *   dA = dT^T x  [r, cols] fp32,  dB = s dY^T T0  [rows, r] fp32.
 * dA and dB are overwritten, not accumulated.  t_saved (nullable) is T0 from the
 * forward; when NULL it is recomputed.  Pages: qlora-rs README "Honest capability
 * matrix" / "Training" (adapters update, base frozen); "LoRA and QLoRA,
 * mathematically" (only the low-rank factors are trained).
 * Errors: as qlora_linear_fwd, plus null dy / d_a / d_b and QLORA_ERR_SHAPE for
 * m == 0 (there is nothing to differentiate).
 */
int qlora_linear_bwd(const qlora_nf4_t* w, const void* x, const void* dy, int64_t m,
                     const void* lora_a, const void* lora_b, int32_t r, float alpha,
                     int32_t flags, int32_t cd, const float* t_saved, void* dx, float* d_a,
                     float* d_b, void* ws, size_t ws_bytes, void* stream);

/*
 * A group of g QLoRA projections that read the same input x (the q / k / v
 * projections of an attention block, the gate / up projections of an MLP), in one
 * call.  Projection i has weight w[i] [rows_i, cols] (cols the same for all),
 * adapters lora_a[i] [r[i], cols], lora_b[i] [rows_i, r[i]] and scale alpha[i] / r[i]
 * (alpha[i] / sqrt(r[i]) with QLORA_FLAG_RSLORA).  The outputs sit side by side:
 *   y [m, N] with N = sum rows_i, columns off_i .. off_i + rows_i of projection i
 *   (off_i = rows_0 + ... + rows_{i-1}), each exactly what qlora_linear_fwd gives for
 *   that projection up to the order of its fp32 sums; bias (nullable) is [N].
 * t_save (nullable array of g nullable pointers): T0_i = x A_i^T fp32 [m, r[i]].
 * Page: "LoRA and QLoRA, mathematically", "Rank, alpha, and target modules" (the
 * adapted modules of a block: q, k, v, o, gate, up, down); the layer itself as in
 * qlora_linear_fwd.
 * How: bf16 / f16, more than 64 tokens, layouts the 256 x 256 kernels take, rows_i
 * multiples of 64 and r[i] <= 64: every W~_i is dequantized into one [N, cols] buffer of the workspace,
 * the rank products write T_i side by side, and one dense GEMM reads
 * [x | T] [W~ | B]^T with B block-diagonal (row n of projection i holds B_i[n] in
 * the columns of T_i), so the short launches of small projections and the cut last
 * rounds of large ones merge.  Otherwise each projection runs through
 * qlora_linear_fwd into the workspace and a copy places its columns.
 * Flags: QLORA_FLAG_RSLORA only.  ws: qlora_group_workspace_bytes(QLORA_OP_FWD, ...)
 * bytes, 256-byte aligned.  Arrays 16-byte aligned as for qlora_linear_fwd.
 * Errors: as qlora_linear_fwd for each projection, plus QLORA_ERR_INVALID_ARG for
 * g < 1, g > QLORA_GROUP_MAX, null arrays or other flags, and QLORA_ERR_SHAPE for
 * differing cols.
 */
#define QLORA_GROUP_MAX 8
int qlora_linear_fwd_group(int32_t g, const qlora_nf4_t* const* w, const void* x, int64_t m,
                           const void* const* lora_a, const void* const* lora_b, const int32_t* r,
                           const float* alpha, int32_t flags, const void* bias, int32_t cd, void* y,
                           float* const* t_save, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of the group with the base weights frozen:
 *   dX = sum_i (dY_i W~_i + dT_i A_i)  [m, cols] (cd; skipped when dx == NULL),
 *   dA_i = dT_i^T x,  dB_i = s_i dY_i^T T0_i  (fp32, overwritten),  dT_i = s_i dY_i B_i,
 * with dy [m, N] laid out like the forward's y (dY_i its columns off_i ..).  dX is the
 * gradient of the block input the projections share.  On the tiled path one fp32
 * accumulation runs over every projection's contraction and is rounded once;
 * otherwise each projection's dX from qlora_linear_bwd (rounded to cd) is added in
 * fp32 and the sum rounded.
 * t_saved (nullable array, or array of nullable pointers): the forward's T0_i.
 * How: as the forward (one dense dX GEMM over the concatenated contraction
 * [dY | dT] [W~ ; A]), otherwise per projection and an fp32 sum of the dX terms.
 * ws: qlora_group_workspace_bytes(QLORA_OP_BWD, ...) bytes.
 * Errors: as qlora_linear_bwd for each projection, and as qlora_linear_fwd_group.
 */
int qlora_linear_bwd_group(int32_t g, const qlora_nf4_t* const* w, const void* x, const void* dy, int64_t m,
                           const void* const* lora_a, const void* const* lora_b, const int32_t* r,
                           const float* alpha, int32_t flags, int32_t cd, const float* const* t_saved,
                           void* dx, float* const* d_a, float* const* d_b, void* ws, size_t ws_bytes,
                           void* stream);

/* Workspace bytes for qlora_linear_fwd_group (op QLORA_OP_FWD) or
 * qlora_linear_bwd_group (QLORA_OP_BWD) on these g weights; 0 for an invalid query.
 * Pure host function. */
size_t qlora_group_workspace_bytes(int32_t op, int32_t g, const qlora_nf4_t* const* w, int64_t m,
                                   const int32_t* r, int32_t cd);

/*
 * Fold the trained adapter into a dense weight (the step after training):
 *   out [rows, cols] = RNE_cd(w_hat + s (B . A)),  s = alpha / r (alpha / sqrt(r)
 *   with QLORA_FLAG_RSLORA),
 * w_hat = fl32(L[code] * s_b) exactly as qlora_nf4_dequantize computes it.  B . A is
 * summed in fp32 (bf16 / f16 products are exact in fp32), added to w_hat with one
 * fp32 fused multiply-add and rounded to nearest-even into cd.  The result stays
 * dense and is never re-quantized to NF4, which would round the update away.
 * lora_a [r, cols], lora_b [rows, r] and out [rows, cols] are row-major device
 * arrays of dtype cd owned by the caller; out must not overlap the inputs.
 * Pages: "LoRA and QLoRA, mathematically", "The merge math, and when merging changes
 * behavior", eq. (6.3.6); qlora-rs README "Honest capability matrix" (dense merge
 * helper with the LoRA scaling, rsLoRA included) and "Deploy".
 * bf16 / f16 with r, cols and block_size multiples of 8 and 16-byte aligned arrays
 * run on the MFMA kernel; other shapes and fp32 on a generic kernel (same w_hat, the
 * rank sum in another order).  An empty weight is a no-op.
 * Errors: QLORA_ERR_INVALID_ARG (null pointers, r < 1, non-finite alpha, flags other
 * than QLORA_FLAG_RSLORA), QLORA_ERR_SHAPE (as qlora_nf4_dequantize), QLORA_ERR_DTYPE,
 * QLORA_ERR_UNSUPPORTED (more than 4194240 rows).
 */
int qlora_merge(const qlora_nf4_t* w, const void* lora_a, const void* lora_b, int32_t r, float alpha,
                int32_t flags, int32_t cd, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Training a stack of QLoRA layers (qlora-rs README, "Training (layer stack)": stacked
 * QuantizedLinear layers, an MSE training_step, AdamW updating the adapters while the
 * NF4 bases stay frozen).
 * ------------------------------------------------------------------------- */

/* AdamW hyper-parameters (decoupled weight decay). */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
} qlora_adamw_t;

/* Bytes of workspace qlora_mse_loss_grad needs (a fixed small size). */
#define QLORA_MSE_WORKSPACE_BYTES 4096

/*
 * loss = mean((y - target)^2) over n elements and dy = dL/dy = 2 (y - target) / n.
 * y, target, dy: device arrays of n elements of dtype cd (dy may alias y); loss: one
 * device float.  The squares are summed in fp32 in a fixed order (deterministic);
 * dy is rounded once more from fp32 into cd.  ws: device workspace of at least
 * QLORA_MSE_WORKSPACE_BYTES bytes, 256-byte aligned.  n == 0 is a no-op.
 * Errors: QLORA_ERR_INVALID_ARG (null pointers, n < 0), QLORA_ERR_DTYPE,
 * QLORA_ERR_WORKSPACE.
 */
int qlora_mse_loss_grad(const void* y, const void* target, int64_t n, int32_t cd, float* loss, void* dy,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * One AdamW step on n fp32 parameters in place, step t >= 1 (1-based):
 *   m = b1 m + (1 - b1) g,  v = b2 v + (1 - b2) g^2,
 *   param = param (1 - lr wd) - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps),
 * all in fp32 (the bias corrections are formed in fp64 and rounded once).  When
 * param_cd is not NULL it receives RNE_cd(param) (the copy the layer kernels read).
 * m and v start at zero.  Errors: QLORA_ERR_INVALID_ARG (null pointers, n < 0,
 * step < 1, non-finite or out-of-range hyper-parameters), QLORA_ERR_DTYPE.
 */
int qlora_adamw_step(float* param, const float* grad, float* m, float* v, int64_t n, const qlora_adamw_t* opt,
                     int32_t step, void* param_cd, int32_t cd, void* stream);

/* One layer of a stack: its frozen base and its adapter state (all device memory,
 * owned by the caller; shapes from w: A [r, cols], B [rows, r]). */
typedef struct {
  const qlora_nf4_t* w;  /* frozen NF4 base [rows, cols] (host descriptor) */
  void* lora_a;          /* [r, cols] cd: the copy the kernels read, rewritten by each step */
  void* lora_b;          /* [rows, r] cd */
  float* a32;            /* [r, cols] fp32 master copy of A (updated by AdamW) */
  float* b32;            /* [rows, r] fp32 master copy of B */
  float* m_a;            /* AdamW moments of A and B, fp32, zero before the first step */
  float* v_a;
  float* m_b;
  float* v_b;
  float* grad_a;         /* [r, cols] fp32: dL/dA of the step, written by the step */
  float* grad_b;         /* [rows, r] fp32: dL/dB */
} qlora_stack_layer_t;

/*
 * One training step of a stack of n_layers QLoRA layers, h_{l+1} = layer_l(h_l) with
 * h_0 = x [m, cols_0] and layer l's cols equal to layer l-1's rows (no activation
 * between layers):  forward through the stack (qlora_linear_fwd, keeping T0),
 * loss = mean((h_L - target)^2) into *loss (device float), backward through the stack
 * (qlora_linear_bwd; dX of layer 0 is skipped), then AdamW (qlora_adamw_step) on every
 * A and B with step t, refreshing the cd copies.  Activations and the gradients
 * between layers are stored in cd.  All layers share r, alpha, flags and cd.
 * ws: at least qlora_stack_workspace_bytes(...) bytes, 256-byte aligned.
 * Errors: those of qlora_linear_fwd / _bwd for any layer, QLORA_ERR_SHAPE (layers
 * that do not chain, m < 1, n_layers < 1), QLORA_ERR_INVALID_ARG (null pointers, bad
 * hyper-parameters), QLORA_ERR_WORKSPACE.
 */
int qlora_stack_train_step(const qlora_stack_layer_t* layers, int32_t n_layers, const void* x, int64_t m,
                           const void* target, int32_t r, float alpha, int32_t flags, int32_t cd,
                           const qlora_adamw_t* opt, int32_t step, float* loss, void* ws, size_t ws_bytes,
                           void* stream);

/* Workspace bytes of qlora_stack_train_step (reads only the layers' shapes); 0 for an
 * invalid query.  Pure host function. */
size_t qlora_stack_workspace_bytes(const qlora_stack_layer_t* layers, int32_t n_layers, int64_t m, int32_t r,
                                   int32_t cd, int32_t flags);

/*
 * The layer with LoRA dropout (rust_ai_core QLoraConfig "Fields": the LoRA
 * configuration holds rank, alpha and dropout; "LoRA and QLoRA, mathematically",
 * "Tooling": PEFT's LoraConfig dropout).  Dropout acts on the input of the low-rank
 * branch only, as inverted dropout with the caller's keep mask M and rate p:
 *   y  = x W~^T + s (x_d A^T) B^T (+ bias),  x_d = x M / (1 - p),
 *   dX = dY W~ + (dT A) M / (1 - p),  dA = dT^T x_d,  dB = s dY^T (x_d A^T),
 * with dT = s dY B.  mask: device u8 [m, cols], nonzero = kept (the caller draws it,
 * e.g. Bernoulli(1 - p), and passes the same mask to both calls); 0 <= p < 1.
 * t_save / t_saved hold x_d A^T (1 - p), i.e. (x M) A^T.  The arguments are otherwise
 * those of qlora_linear_fwd / qlora_linear_bwd; the workspace is
 * qlora_workspace_bytes(op | (flags | QLORA_FLAG_DROPOUT) << QLORA_OP_FLAGS_SHIFT, ...)
 * (x M is staged there; calls with m <= 16 take the GEMM path, not the decode GEMV).
 * Errors: those of qlora_linear_fwd / _bwd, plus QLORA_ERR_INVALID_ARG for a null
 * mask or p outside [0, 1).
 */
int qlora_linear_fwd_dropout(const qlora_nf4_t* w, const void* x, int64_t m, const void* lora_a,
                             const void* lora_b, int32_t r, float alpha, int32_t flags, const void* bias,
                             int32_t cd, const uint8_t* mask, float p, void* y, float* t_save, void* ws,
                             size_t ws_bytes, void* stream);
int qlora_linear_bwd_dropout(const qlora_nf4_t* w, const void* x, const void* dy, int64_t m,
                             const void* lora_a, const void* lora_b, int32_t r, float alpha, int32_t flags,
                             int32_t cd, const uint8_t* mask, float p, const float* t_saved, void* dx,
                             float* d_a, float* d_b, void* ws, size_t ws_bytes, void* stream);

/* Cached-dequant forward (qlora-rs CONFIG "cache_dequantized"; the memory-for-speed
 * trade-off of BOOK "Tooling" and the README's on-the-fly versus cached dequant):
 * the caller dequantizes the frozen weight once with qlora_nf4_dequantize(w, cd,
 * w_cd) and keeps w_cd; each call then computes
 *   y = x w_cd^T + s (x A^T) B^T (+ bias)
 * with the dense GEMM reading w_cd in place (no NF4 decode, no copy of W~ in the
 * workspace; the resident copy costs rows x cols x 2 bytes instead of the packed
 * 0.5 + scales).  Given w_cd from qlora_nf4_dequantize, y equals qlora_linear_fwd
 * with QLORA_FLAG_DEQUANT_GEMM bit for bit for m > 16.
 * w_cd: device [rows, cols] in cd (bf16 or f16), row-major.  Other arguments as for
 * qlora_linear_fwd; flags: 0 or QLORA_FLAG_RSLORA.  ws: at least
 * qlora_workspace_bytes(QLORA_OP_FWD_CACHED, m, rows, cols, r, cd) bytes.
 * Errors: QLORA_ERR_DTYPE unless cd is bf16 / f16; QLORA_ERR_UNSUPPORTED if cols is
 * not a multiple of 64 or w_cd (or x) spans 2 GiB or more; QLORA_ERR_INVALID_ARG for
 * null pointers, r < 1, non-finite alpha or other flags; QLORA_ERR_WORKSPACE. */
int qlora_linear_fwd_cached(const void* w_cd, int64_t rows, int64_t cols, const void* x, int64_t m,
                            const void* lora_a, const void* lora_b, int32_t r, float alpha, int32_t flags,
                            const void* bias, int32_t cd, void* y, float* t_save, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * The forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and errors as qlora_linear_fwd without the workspace: the call uses a
 * scratch array of qlora_noalloc_scratch_bytes() bytes (32 MiB) that the library
 * holds in each GPU's memory for the life of the process, and calls no allocating
 * routine.  Above 16 tokens it takes the fused kernels (no copy of W~) unless
 * flags has QLORA_FLAG_DEQUANT_GEMM.  A call whose workspace
 * (qlora_workspace_bytes of the same path) exceeds the scratch array is refused
 * with QLORA_ERR_WORKSPACE before anything runs (the decode calls of the
 * Llama-3-8B-shaped projections need at most a few MiB; fused forwards fit while
 * their rank products and cut last round stay under the limit).  The scratch array is looked
 * up on the current device (the one the stream and arrays belong to) on its first
 * use there.  Calls on one GPU share its array: two calls that overlap on one GPU
 * (concurrent streams, or threads) race and give undefined results; calls on one
 * stream are ordered and safe.  Nothing in the array needs to start at zero.
 */
int qlora_linear_fwd_noalloc(const qlora_nf4_t* w, const void* x, int64_t m, const void* lora_a,
                             const void* lora_b, int32_t r, float alpha, int32_t flags, const void* bias,
                             int32_t cd, void* y, float* t_save, void* stream);

/* Bytes of the scratch array qlora_linear_fwd_noalloc uses on each GPU.  Pure host. */
size_t qlora_noalloc_scratch_bytes(void);

/* Workspace size in bytes for op (QLORA_OP_FWD / QLORA_OP_BWD, optionally OR'ed
 * with flags << QLORA_OP_FLAGS_SHIFT) on this layer shape; 0 for an invalid query.
 * Pure host function. */
size_t qlora_workspace_bytes(int32_t op, int64_t m, int64_t rows, int64_t cols, int32_t r,
                             int32_t cd);

/* Thread-local message for the last error returned on this thread ("" if none). */
const char* qlora_last_error(void);

/* Host copy of the 16 fp32 NF4 levels the kernels use, ascending.  Pure host. */
int qlora_nf4_levels(float out[16]);

/* QLORA_NF4_ABI_VERSION of the built library. */
int qlora_abi_version(void);

/*
 * Kernel timing (off by default).  While enabled, every kernel the library
 * launches is bracketed by a pair of HIP events recorded on the caller's stream,
 * and the elapsed times are summed per kernel kind.  Used by the benchmark to time
 * individual kernels inside a multi-kernel call; costs one event pair per launch.
 *   qlora_profile_enable(1) resets the totals and starts recording; (0) stops.
 *   qlora_profile_read(kind, &ms, &launches) waits for the recorded events and
 *   returns the summed milliseconds and launch count of that kind.
 *   qlora_kernel_name(kind) names a kind ("" when out of range).
 * Errors: QLORA_ERR_INVALID_ARG (bad kind / null output), QLORA_ERR_HIP.
 */
enum {
  QLORA_K_QUANTIZE = 0,
  QLORA_K_DEQUANTIZE,
  QLORA_K_LORA_DOWN,  /* T = s x A^T (prologue of the forward; T0 in the backward) */
  QLORA_K_REDUCE,     /* fixed-order sum of split-contraction partials */
  QLORA_K_FWD_GEMM,   /* forward GEMM y = [x | T][W~ | B]^T, m > 16 (dense or fused) */
  QLORA_K_GEMV,       /* decode forward, m <= 16 (its LoRA prologue counts as LORA_DOWN) */
  QLORA_K_BWD_DT,     /* dT = s dY B */
  QLORA_K_BWD_DX,     /* backward GEMM dX = dY W~ + dT A (dense or fused) */
  QLORA_K_BWD_DA,     /* dA = dT^T x */
  QLORA_K_BWD_DB,     /* dB = s dY^T T0 */
  QLORA_K_MERGE,      /* adapter merge into the dense weight */
  QLORA_K_LOSS,       /* MSE loss and its gradient */
  QLORA_K_OPTIM,      /* AdamW update of an adapter */
  QLORA_K_COUNT
};
int qlora_profile_enable(int32_t on);
int qlora_profile_read(int32_t kind, double* ms, int64_t* launches);
const char* qlora_kernel_name(int32_t kind);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_NF4_H */
