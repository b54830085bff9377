"""QLoRA NF4 linear layer for AMD Instinct MI355X (gfx950).

Thin Python binding over libqlora_nf4.so (C ABI in include/qlora_nf4.h).  This
module only marshals arguments: it checks devices / dtypes / contiguity, passes
raw device pointers and the current HIP stream, and allocates outputs and
workspaces with torch.  Every step of the computation runs in the library's
hand-written HIP kernels; there is no CPU or PyTorch fallback.

Public API (names follow the pages' problem statement):
    quantize(w, block_size=64, double_quant=False, dq_group=256 | "global") -> NF4Weight
    dequantize(q, dtype=torch.bfloat16) -> Tensor [rows, cols]
    linear_fwd_cached(w_cd, x, lora_a, lora_b, alpha, bias=None, save_t=False, rslora=False)
    linear_fwd_noalloc(q, x, lora_a, lora_b, alpha, bias=None, out=None, t_out=None, rslora=False, path="auto")
    linear_fwd(q, x, lora_a, lora_b, alpha, bias=None, save_t=False, rslora=False, path="auto",
               dropout_mask=None, dropout_p=0.0)
    linear_bwd(q, x, dy, lora_a, lora_b, alpha, t_saved=None, need_dx=True, rslora=False, path="auto",
               dropout_mask=None, dropout_p=0.0)
    merge(q, lora_a, lora_b, alpha, rslora=False, out=None) -> Tensor [rows, cols]
    mse_loss_grad(y, target) -> (loss [1] fp32, dy) ; adamw_step(param, grad, m, v, step, ...)
    StackLayer.create(q, a32, b32, dtype) ; stack_train_step(layers, x, target, alpha, step, ...)
    workspace_bytes(op, m, rows, cols, r, dtype, flags=0) ; levels()

path: "fused" decodes W inside the GEMM kernels; "dequant" writes W~ (or W~^T for
dX) into the workspace first and runs a dense GEMM; "auto" lets the library pick
(dequantize-then-GEMM for bf16 / f16; "fused" saves the rows x cols copy in the
workspace).  Calls with at most 16 tokens take the decode GEMV either way.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

from . import _lib
from ._lib import QloraError, QloraNf4  # noqa: F401

__all__ = ["NF4Weight", "quantize", "dequantize", "linear_fwd", "linear_bwd", "merge", "workspace_bytes",
           "linear_fwd_noalloc", "linear_fwd_cached",
           "levels", "QloraError", "dtype_code", "profile_enable", "profile_read", "mse_loss_grad",
           "adamw_step", "StackLayer", "stack_train_step", "stack_workspace_bytes",
           "linear_fwd_group", "linear_bwd_group", "group_workspace_bytes"]


def _torch():
    import torch
    return torch


def dtype_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return _lib.QLORA_F32
    if dtype == torch.bfloat16:
        return _lib.QLORA_BF16
    if dtype == torch.float16:
        return _lib.QLORA_F16
    raise TypeError("unsupported dtype %s (float32, bfloat16 or float16)" % (dtype,))


def _stream_ptr(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need_cuda(name, t, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


@dataclass
class NF4Weight:
    """An NF4-quantized frozen weight [rows, cols] held in device memory."""
    rows: int
    cols: int
    block_size: int
    double_quant: bool
    dq_group: int
    codes: "object"                      # uint8 [rows*cols/2]
    absmax: "object" = None              # float32 [nb]
    absmax_q: "object" = None            # uint8 [nb]
    absmax_scale2: "object" = None       # float32 [ng]

    @property
    def shape(self) -> Tuple[int, int]:
        return (self.rows, self.cols)

    @property
    def device(self):
        return self.codes.device

    def size_bytes(self) -> int:
        n = self.codes.numel()
        for t in (self.absmax, self.absmax_q, self.absmax_scale2):
            if t is not None:
                n += t.numel() * t.element_size()
        return n

    def descriptor(self) -> QloraNf4:
        return QloraNf4(self.rows, self.cols, self.block_size, int(self.double_quant),
                        self.dq_group, 0, _ptr(self.codes), _ptr(self.absmax),
                        _ptr(self.absmax_q), _ptr(self.absmax_scale2))


def empty_nf4(rows: int, cols: int, block_size: int = 64, double_quant: bool = False,
              dq_group: int = 256, device="cuda") -> NF4Weight:
    torch = _torch()
    n = rows * cols
    nb = n // block_size if block_size > 0 else 0
    codes = torch.empty(n // 2, dtype=torch.uint8, device=device)
    if double_quant:
        ng = (nb + dq_group - 1) // dq_group
        return NF4Weight(rows, cols, block_size, True, dq_group, codes, None,
                         torch.empty(nb, dtype=torch.uint8, device=device),
                         torch.empty(ng, dtype=torch.float32, device=device))
    return NF4Weight(rows, cols, block_size, False, dq_group, codes,
                     torch.empty(nb, dtype=torch.float32, device=device))


def quantize(w, block_size: int = 64, double_quant: bool = False, dq_group=256) -> NF4Weight:
    """Blockwise NF4 quantization of a 2-D fp32 GPU tensor (optionally with the block
    scales double-quantized to u8 + one fp32 scale per dq_group blocks; dq_group
    "global" puts every block in one group)."""
    torch = _torch()
    _need_cuda("w", w, torch.float32)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [rows, cols]")
    rows, cols = w.shape
    if dq_group == "global":
        dq_group = max(1, (rows * cols) // block_size) if block_size > 0 else 1
    if block_size <= 0 or (rows * cols) % block_size:
        desc_bs = block_size  # let the library produce the status and message
        q = NF4Weight(rows, cols, desc_bs, double_quant, dq_group,
                      torch.empty(0, dtype=torch.uint8, device=w.device))
    else:
        q = empty_nf4(rows, cols, block_size, double_quant, dq_group, w.device)
    d = q.descriptor()
    _lib.check(_lib.lib().qlora_nf4_quantize(_ptr(w), ctypes.byref(d), _stream_ptr(w.device)))
    return q


def dequantize(q: NF4Weight, dtype=None):
    """w_hat = fl32(level * block scale), rounded to nearest-even into ``dtype``."""
    torch = _torch()
    dtype = torch.bfloat16 if dtype is None else dtype
    out = torch.empty(q.rows, q.cols, dtype=dtype, device=q.device)
    d = q.descriptor()
    _lib.check(_lib.lib().qlora_nf4_dequantize(ctypes.byref(d), dtype_code(dtype), _ptr(out),
                                              _stream_ptr(q.device)))
    return out


def workspace_bytes(op: int, m: int, rows: int, cols: int, r: int, dtype, flags: int = 0) -> int:
    return int(_lib.lib().qlora_workspace_bytes(op | (flags << _lib.QLORA_OP_FLAGS_SHIFT), m, rows, cols, r,
                                               dtype_code(dtype)))


_PATHS = {"auto": 0, "fused": _lib.QLORA_FLAG_FUSED, "dequant": _lib.QLORA_FLAG_DEQUANT_GEMM}


def _flags(rslora: bool, path: str) -> int:
    if path not in _PATHS:
        raise ValueError("path must be one of %s" % sorted(_PATHS))
    return (_lib.QLORA_FLAG_RSLORA if rslora else 0) | _PATHS[path]


def _workspace(nbytes: int, device, workspace=None):
    torch = _torch()
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), nbytes))
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _flatten(x, cols):
    if x.shape[-1] != cols:
        raise ValueError("last dim of x must be %d, got %d" % (cols, x.shape[-1]))
    lead = tuple(x.shape[:-1])
    return x.reshape(-1, cols), lead


def _dropout_args(dropout_mask, dropout_p, x2):
    torch = _torch()
    if dropout_mask is None:
        return None, 0.0
    mk = dropout_mask.reshape(-1, x2.shape[1]).contiguous()
    _need_cuda("dropout_mask", mk, torch.uint8)
    if mk.shape != x2.shape:
        raise ValueError("dropout_mask must have x's shape")
    return mk, float(dropout_p)


def linear_fwd(q: NF4Weight, x, lora_a, lora_b, alpha: float, bias=None, save_t: bool = False,
               rslora: bool = False, workspace=None, out=None, t_out=None, path: str = "auto",
               dropout_mask=None, dropout_p: float = 0.0):
    """y = x . deq(W)^T + s (x . A^T) . B^T (+ bias), s = alpha / r (alpha / sqrt(r)
    with rslora).  Leading dims of x are flattened to tokens.  Returns y, or
    (y, T0) with T0 = x A^T in fp32 when save_t.  ``out`` / ``t_out`` may supply
    preallocated outputs.  With ``dropout_mask`` (uint8, x's shape, nonzero = kept)
    the low-rank branch reads x * mask / (1 - dropout_p) (LoRA dropout)."""
    torch = _torch()
    dt = x.dtype
    x2, lead = _flatten(x, q.cols)
    x2 = x2.contiguous()
    for name, t in (("x", x2), ("lora_a", lora_a), ("lora_b", lora_b), ("bias", bias)):
        _need_cuda(name, t, dt)
    r = lora_a.shape[0]
    m = x2.shape[0]
    y = out if out is not None else torch.empty(m, q.rows, dtype=dt, device=x.device)
    _need_cuda("out", y, dt)
    if y.numel() != m * q.rows:
        raise ValueError("out must hold %d x %d elements" % (m, q.rows))
    t0 = t_out if t_out is not None else (
        torch.empty(m, r, dtype=torch.float32, device=x.device) if save_t else None)
    _need_cuda("t_out", t0, torch.float32)
    if t0 is not None and t0.numel() != m * r:
        raise ValueError("t_out must hold %d x %d fp32 elements" % (m, r))
    flags = _flags(rslora, path)
    mk, p = _dropout_args(dropout_mask, dropout_p, x2)
    qflags = flags | (_lib.QLORA_FLAG_DROPOUT if mk is not None else 0)
    ws = _workspace(workspace_bytes(_lib.QLORA_OP_FWD, m, q.rows, q.cols, r, dt, qflags), x.device, workspace)
    d = q.descriptor()
    if mk is None:
        _lib.check(_lib.lib().qlora_linear_fwd(
            ctypes.byref(d), _ptr(x2), m, _ptr(lora_a), _ptr(lora_b), r, float(alpha), flags,
            _ptr(bias), dtype_code(dt), _ptr(y), _ptr(t0), _ptr(ws), ws.numel() * ws.element_size(),
            _stream_ptr(x.device)))
    else:
        _lib.check(_lib.lib().qlora_linear_fwd_dropout(
            ctypes.byref(d), _ptr(x2), m, _ptr(lora_a), _ptr(lora_b), r, float(alpha), flags,
            _ptr(bias), dtype_code(dt), _ptr(mk), p, _ptr(y), _ptr(t0), _ptr(ws), ws.numel() * ws.element_size(),
            _stream_ptr(x.device)))
    y = y.reshape(*lead, q.rows)
    return (y, t0) if (save_t or t_out is not None) else y


def linear_fwd_noalloc(q: NF4Weight, x, lora_a, lora_b, alpha: float, bias=None, out=None, t_out=None,
                       rslora: bool = False, path: str = "auto"):
    """The forward through qlora_linear_fwd_noalloc: no workspace, the library's own
    scratch array instead (for graph capture and serving loops that cannot
    allocate).  ``out`` (and ``t_out`` for T0) may be preallocated; returns y, or
    (y, T0) when ``t_out`` is given."""
    torch = _torch()
    dt = x.dtype
    x2, lead = _flatten(x, q.cols)
    x2 = x2.contiguous()
    for name, t in (("x", x2), ("lora_a", lora_a), ("lora_b", lora_b), ("bias", bias)):
        _need_cuda(name, t, dt)
    r = lora_a.shape[0]
    m = x2.shape[0]
    y = out if out is not None else torch.empty(m, q.rows, dtype=dt, device=x.device)
    _need_cuda("out", y, dt)
    _need_cuda("t_out", t_out, torch.float32)
    if y.numel() != m * q.rows or (t_out is not None and t_out.numel() != m * r):
        raise ValueError("out / t_out have the wrong size")
    d = q.descriptor()
    _lib.check(_lib.lib().qlora_linear_fwd_noalloc(
        ctypes.byref(d), _ptr(x2), m, _ptr(lora_a), _ptr(lora_b), r, float(alpha), _flags(rslora, path),
        _ptr(bias), dtype_code(dt), _ptr(y), _ptr(t_out), _stream_ptr(x.device)))
    y = y.reshape(*lead, q.rows)
    return (y, t_out) if t_out is not None else y


def linear_fwd_cached(w_cd, x, lora_a, lora_b, alpha: float, bias=None, save_t: bool = False,
                      rslora: bool = False, workspace=None, out=None, t_out=None):
    """Cached-dequant forward: ``w_cd`` is W~ [rows, cols] in x's dtype (bf16 / f16),
    dequantized once by ``dequantize(q, dtype)`` and kept by the caller; returns
    x . w_cd^T + s (x . A^T) . B^T (+ bias), or (y, T0) when save_t."""
    torch = _torch()
    dt = x.dtype
    rows, cols = w_cd.shape
    _need_cuda("w_cd", w_cd, dt)
    x2, lead = _flatten(x, cols)
    x2 = x2.contiguous()
    for name, t in (("x", x2), ("lora_a", lora_a), ("lora_b", lora_b), ("bias", bias)):
        _need_cuda(name, t, dt)
    r = lora_a.shape[0]
    m = x2.shape[0]
    y = out if out is not None else torch.empty(m, rows, dtype=dt, device=x.device)
    _need_cuda("out", y, dt)
    if y.numel() != m * rows:
        raise ValueError("out must hold %d x %d elements" % (m, rows))
    t0 = t_out if t_out is not None else (
        torch.empty(m, r, dtype=torch.float32, device=x.device) if save_t else None)
    _need_cuda("t_out", t0, torch.float32)
    if t0 is not None and t0.numel() != m * r:
        raise ValueError("t_out must hold %d x %d fp32 elements" % (m, r))
    flags = _lib.QLORA_FLAG_RSLORA if rslora else 0
    ws = _workspace(workspace_bytes(_lib.QLORA_OP_FWD_CACHED, m, rows, cols, r, dt, flags), x.device, workspace)
    _lib.check(_lib.lib().qlora_linear_fwd_cached(
        _ptr(w_cd.contiguous()), rows, cols, _ptr(x2), m, _ptr(lora_a), _ptr(lora_b), r, float(alpha), flags,
        _ptr(bias), dtype_code(dt), _ptr(y), _ptr(t0), _ptr(ws), ws.numel() * ws.element_size(),
        _stream_ptr(x.device)))
    y = y.reshape(*lead, rows)
    return (y, t0) if (save_t or t_out is not None) else y


class _GroupArgs:
    """ctypes arrays for the g projections of a group call (kept alive with it)."""

    def __init__(self, qs, lora_as=None, lora_bs=None, alphas=None):
        g = len(qs)
        if not 1 <= g <= _lib.QLORA_GROUP_MAX:
            raise ValueError("a group holds 1 to %d projections" % _lib.QLORA_GROUP_MAX)
        self.g = g
        self.descs = [q.descriptor() for q in qs]
        self.w = (ctypes.POINTER(_lib.QloraNf4) * g)(*[ctypes.pointer(d) for d in self.descs])
        ranks = [a.shape[0] for a in lora_as] if lora_as is not None else [0] * g
        self.r = (ctypes.c_int32 * g)(*ranks)
        if lora_as is not None:
            self.a = (ctypes.c_void_p * g)(*[_ptr(a) for a in lora_as])
            self.b = (ctypes.c_void_p * g)(*[_ptr(b) for b in lora_bs])
            self.alpha = (ctypes.c_float * g)(*[float(a) for a in alphas])

    @staticmethod
    def ptrs(ts):
        return None if ts is None else (ctypes.c_void_p * len(ts))(*[_ptr(t) for t in ts])


def group_workspace_bytes(op: int, qs, m: int, ranks, dtype) -> int:
    """Workspace bytes of a group call (op QLORA_OP_FWD / QLORA_OP_BWD)."""
    ga = _GroupArgs(qs)
    ga.r = (ctypes.c_int32 * ga.g)(*[int(r) for r in ranks])
    return int(_lib.lib().qlora_group_workspace_bytes(op, ga.g, ga.w, m, ga.r, dtype_code(dtype)))


def linear_fwd_group(qs, x, lora_as, lora_bs, alphas, bias=None, save_t: bool = False, rslora: bool = False,
                     workspace=None, out=None):
    """Projections that read the same x in one call: returns y [m, sum rows_i] with
    projection i's output in its columns (and the list of T0_i = x A_i^T in fp32 when
    save_t).  bias, if given, is [sum rows_i]."""
    torch = _torch()
    dt = x.dtype
    cols = qs[0].cols
    x2, lead = _flatten(x, cols)
    x2 = x2.contiguous()
    _need_cuda("x", x2, dt)
    for i, (a, b) in enumerate(zip(lora_as, lora_bs)):
        _need_cuda("lora_a[%d]" % i, a, dt)
        _need_cuda("lora_b[%d]" % i, b, dt)
    _need_cuda("bias", bias, dt)
    m = x2.shape[0]
    N = sum(q.rows for q in qs)
    y = out if out is not None else torch.empty(m, N, dtype=dt, device=x.device)
    _need_cuda("out", y, dt)
    if y.numel() != m * N:
        raise ValueError("out must hold %d x %d elements" % (m, N))
    ts = [torch.empty(m, a.shape[0], dtype=torch.float32, device=x.device) for a in lora_as] if save_t else None
    ga = _GroupArgs(qs, lora_as, lora_bs, alphas)
    ws = _workspace(group_workspace_bytes(_lib.QLORA_OP_FWD, qs, m, [a.shape[0] for a in lora_as], dt), x.device,
                    workspace)
    _lib.check(_lib.lib().qlora_linear_fwd_group(
        ga.g, ga.w, _ptr(x2), m, ga.a, ga.b, ga.r, ga.alpha, _lib.QLORA_FLAG_RSLORA if rslora else 0, _ptr(bias),
        dtype_code(dt), _ptr(y), _GroupArgs.ptrs(ts), _ptr(ws), ws.numel() * ws.element_size(),
        _stream_ptr(x.device)))
    y = y.reshape(*lead, N)
    return (y, ts) if save_t else y


def linear_bwd_group(qs, x, dy, lora_as, lora_bs, alphas, t_saved=None, need_dx: bool = True,
                     rslora: bool = False, workspace=None):
    """Gradients of a group with the bases frozen: dy [m, sum rows_i] laid out like the
    forward's y.  Returns (dX = sum of the projections' input gradients, or None;
    the list of dA_i fp32; the list of dB_i fp32)."""
    torch = _torch()
    dt = x.dtype
    cols = qs[0].cols
    N = sum(q.rows for q in qs)
    x2, lead = _flatten(x, cols)
    dy2, _ = _flatten(dy, N)
    x2, dy2 = x2.contiguous(), dy2.contiguous()
    _need_cuda("x", x2, dt)
    _need_cuda("dy", dy2, dt)
    m = x2.shape[0]
    dx = torch.empty(m, cols, dtype=dt, device=x.device) if need_dx else None
    das = [torch.empty(a.shape[0], cols, dtype=torch.float32, device=x.device) for a in lora_as]
    dbs = [torch.empty(q.rows, a.shape[0], dtype=torch.float32, device=x.device) for q, a in zip(qs, lora_as)]
    if t_saved is not None:
        for t in t_saved:
            _need_cuda("t_saved", t, torch.float32)
    ga = _GroupArgs(qs, lora_as, lora_bs, alphas)
    ws = _workspace(group_workspace_bytes(_lib.QLORA_OP_BWD, qs, m, [a.shape[0] for a in lora_as], dt), x.device,
                    workspace)
    _lib.check(_lib.lib().qlora_linear_bwd_group(
        ga.g, ga.w, _ptr(x2), _ptr(dy2), m, ga.a, ga.b, ga.r, ga.alpha, _lib.QLORA_FLAG_RSLORA if rslora else 0,
        dtype_code(dt), _GroupArgs.ptrs(t_saved), _ptr(dx), _GroupArgs.ptrs(das), _GroupArgs.ptrs(dbs), _ptr(ws),
        ws.numel() * ws.element_size(), _stream_ptr(x.device)))
    if dx is not None:
        dx = dx.reshape(*lead, cols)
    return dx, das, dbs


def linear_bwd(q: NF4Weight, x, dy, lora_a, lora_b, alpha: float, t_saved=None, need_dx: bool = True,
               rslora: bool = False, workspace=None, dx_out=None, da_out=None, db_out=None, path: str = "auto",
               dropout_mask=None, dropout_p: float = 0.0):
    """Gradients with the base frozen: returns (dX or None, dA fp32 [r, cols], dB fp32 [rows, r]).
    ``*_out`` may supply preallocated outputs; ``dropout_mask`` / ``dropout_p`` as in
    the forward (the same mask)."""
    torch = _torch()
    dt = x.dtype
    x2, lead = _flatten(x, q.cols)
    dy2, _ = _flatten(dy, q.rows)
    x2, dy2 = x2.contiguous(), dy2.contiguous()
    for name, t in (("x", x2), ("dy", dy2), ("lora_a", lora_a), ("lora_b", lora_b)):
        _need_cuda(name, t, dt)
    _need_cuda("t_saved", t_saved, torch.float32)
    r = lora_a.shape[0]
    m = x2.shape[0]
    dx = dx_out if dx_out is not None else (
        torch.empty(m, q.cols, dtype=dt, device=x.device) if need_dx else None)
    da = da_out if da_out is not None else torch.empty(r, q.cols, dtype=torch.float32, device=x.device)
    db = db_out if db_out is not None else torch.empty(q.rows, r, dtype=torch.float32, device=x.device)
    _need_cuda("dx_out", dx, dt)
    _need_cuda("da_out", da, torch.float32)
    _need_cuda("db_out", db, torch.float32)
    if (dx is not None and dx.numel() != m * q.cols) or da.numel() != r * q.cols or db.numel() != q.rows * r:
        raise ValueError("output buffers have the wrong size")
    if t_saved is not None and t_saved.numel() != m * r:
        raise ValueError("t_saved must hold %d x %d fp32 elements" % (m, r))
    flags = _flags(rslora, path)
    mk, p = _dropout_args(dropout_mask, dropout_p, x2)
    qflags = flags | (_lib.QLORA_FLAG_DROPOUT if mk is not None else 0)
    ws = _workspace(workspace_bytes(_lib.QLORA_OP_BWD, m, q.rows, q.cols, r, dt, qflags), x.device, workspace)
    d = q.descriptor()
    if mk is None:
        _lib.check(_lib.lib().qlora_linear_bwd(
            ctypes.byref(d), _ptr(x2), _ptr(dy2), m, _ptr(lora_a), _ptr(lora_b), r, float(alpha), flags,
            dtype_code(dt), _ptr(t_saved), _ptr(dx), _ptr(da), _ptr(db), _ptr(ws),
            ws.numel() * ws.element_size(), _stream_ptr(x.device)))
    else:
        _lib.check(_lib.lib().qlora_linear_bwd_dropout(
            ctypes.byref(d), _ptr(x2), _ptr(dy2), m, _ptr(lora_a), _ptr(lora_b), r, float(alpha), flags,
            dtype_code(dt), _ptr(mk), p, _ptr(t_saved), _ptr(dx), _ptr(da), _ptr(db), _ptr(ws),
            ws.numel() * ws.element_size(), _stream_ptr(x.device)))
    if dx is not None:
        dx = dx.reshape(*lead, q.cols)
    return dx, da, db


def merge(q: NF4Weight, lora_a, lora_b, alpha: float, rslora: bool = False, out=None):
    """Dense merged weight RNE(w_hat + s B A) [rows, cols] in the adapters' dtype
    (never re-quantized to NF4).  ``out`` may supply a preallocated output."""
    torch = _torch()
    dt = lora_a.dtype
    _need_cuda("lora_a", lora_a, dt)
    _need_cuda("lora_b", lora_b, dt)
    r = lora_a.shape[0]
    if lora_a.dim() != 2 or lora_a.shape[1] != q.cols:
        raise ValueError("lora_a must be [r, %d]" % q.cols)
    if lora_b.dim() != 2 or tuple(lora_b.shape) != (q.rows, r):
        raise ValueError("lora_b must be [%d, %d]" % (q.rows, r))
    o = out if out is not None else torch.empty(q.rows, q.cols, dtype=dt, device=lora_a.device)
    _need_cuda("out", o, dt)
    if o.numel() != q.rows * q.cols:
        raise ValueError("out must hold %d x %d elements" % (q.rows, q.cols))
    d = q.descriptor()
    _lib.check(_lib.lib().qlora_merge(ctypes.byref(d), _ptr(lora_a), _ptr(lora_b), r, float(alpha),
                                      _lib.QLORA_FLAG_RSLORA if rslora else 0, dtype_code(dt), _ptr(o),
                                      _stream_ptr(lora_a.device)))
    return o.view(q.rows, q.cols)


def mse_loss_grad(y, target, dy=None):
    """loss = mean((y - target)^2) (a 1-element fp32 GPU tensor) and dy = 2 (y - target) / n
    in y's dtype."""
    torch = _torch()
    dt = y.dtype
    _need_cuda("y", y, dt)
    _need_cuda("target", target, dt)
    if y.numel() != target.numel():
        raise ValueError("y and target differ in size")
    dy = dy if dy is not None else torch.empty_like(y)
    _need_cuda("dy", dy, dt)
    loss = torch.empty(1, dtype=torch.float32, device=y.device)
    ws = torch.empty(_lib.QLORA_MSE_WORKSPACE_BYTES, dtype=torch.uint8, device=y.device)
    _lib.check(_lib.lib().qlora_mse_loss_grad(_ptr(y), _ptr(target), y.numel(), dtype_code(dt), _ptr(loss),
                                              _ptr(dy), _ptr(ws), ws.numel(), _stream_ptr(y.device)))
    return loss, dy


def _adamw(lr, beta1, beta2, eps, weight_decay):
    return _lib.QloraAdamW(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay))


def adamw_step(param, grad, m, v, step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
               eps: float = 1e-8, weight_decay: float = 0.0, param_cd=None):
    """One in-place AdamW update of fp32 ``param`` (moments ``m``, ``v``; 1-based ``step``);
    ``param_cd`` (bf16 / f16 / fp32, optional) receives the rounded copy."""
    torch = _torch()
    for name, t in (("param", param), ("grad", grad), ("m", m), ("v", v)):
        _need_cuda(name, t, torch.float32)
        if t.numel() != param.numel():
            raise ValueError("%s has %d elements, param %d" % (name, t.numel(), param.numel()))
    cd = _lib.QLORA_F32
    if param_cd is not None:
        _need_cuda("param_cd", param_cd)
        cd = dtype_code(param_cd.dtype)
        if param_cd.numel() != param.numel():
            raise ValueError("param_cd has the wrong size")
    o = _adamw(lr, beta1, beta2, eps, weight_decay)
    _lib.check(_lib.lib().qlora_adamw_step(_ptr(param), _ptr(grad), _ptr(m), _ptr(v), param.numel(),
                                           ctypes.byref(o), int(step), _ptr(param_cd), cd,
                                           _stream_ptr(param.device)))


@dataclass
class StackLayer:
    """One layer of a trainable stack: frozen NF4 base, fp32 master adapters, their
    compute-dtype copies, AdamW moments and the gradient buffers the step writes."""
    q: NF4Weight
    lora_a: "object"
    lora_b: "object"
    a32: "object"
    b32: "object"
    m_a: "object"
    v_a: "object"
    m_b: "object"
    v_b: "object"
    grad_a: "object"
    grad_b: "object"

    @staticmethod
    def create(q: NF4Weight, a32, b32, dtype) -> "StackLayer":
        torch = _torch()
        a32 = a32.to(device=q.device, dtype=torch.float32).contiguous().clone()
        b32 = b32.to(device=q.device, dtype=torch.float32).contiguous().clone()
        z = torch.zeros_like
        return StackLayer(q, a32.to(dtype), b32.to(dtype), a32, b32, z(a32), z(a32), z(b32), z(b32), z(a32),
                          z(b32))

    @property
    def r(self) -> int:
        return self.a32.shape[0]

    def _struct(self, desc):
        return _lib.QloraStackLayer(ctypes.pointer(desc), *[_ptr(t) for t in (
            self.lora_a, self.lora_b, self.a32, self.b32, self.m_a, self.v_a, self.m_b, self.v_b,
            self.grad_a, self.grad_b)])


def _stack_structs(layers):
    descs = [L.q.descriptor() for L in layers]
    arr = (_lib.QloraStackLayer * len(layers))(*[L._struct(d) for L, d in zip(layers, descs)])
    return arr, descs


def stack_workspace_bytes(layers, m: int, dtype, rslora: bool = False, path: str = "auto") -> int:
    arr, _descs = _stack_structs(layers)
    return int(_lib.lib().qlora_stack_workspace_bytes(arr, len(layers), m, layers[0].r, dtype_code(dtype),
                                                      _flags(rslora, path)))


def stack_train_step(layers, x, target, alpha: float, step: int, lr: float, beta1: float = 0.9,
                     beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0, rslora: bool = False,
                     path: str = "auto", workspace=None, loss=None):
    """Forward through the stack, MSE loss against ``target``, backward, AdamW on every
    adapter (in place).  Returns the loss as a 1-element fp32 GPU tensor."""
    torch = _torch()
    dt = x.dtype
    x2, _ = _flatten(x, layers[0].q.cols)
    t2, _ = _flatten(target, layers[-1].q.rows)
    x2, t2 = x2.contiguous(), t2.contiguous()
    _need_cuda("x", x2, dt)
    _need_cuda("target", t2, dt)
    m = x2.shape[0]
    if t2.shape[0] != m:
        raise ValueError("target has %d rows, x %d" % (t2.shape[0], m))
    for L in layers:
        _need_cuda("lora_a", L.lora_a, dt)
        _need_cuda("lora_b", L.lora_b, dt)
    arr, _descs = _stack_structs(layers)
    flags = _flags(rslora, path)
    nbytes = int(_lib.lib().qlora_stack_workspace_bytes(arr, len(layers), m, layers[0].r, dtype_code(dt), flags))
    ws = _workspace(nbytes, x.device, workspace)
    loss = loss if loss is not None else torch.empty(1, dtype=torch.float32, device=x.device)
    o = _adamw(lr, beta1, beta2, eps, weight_decay)
    _lib.check(_lib.lib().qlora_stack_train_step(arr, len(layers), _ptr(x2), m, _ptr(t2), layers[0].r, float(alpha),
                                                 flags, dtype_code(dt), ctypes.byref(o), int(step), _ptr(loss),
                                                 _ptr(ws), ws.numel() * ws.element_size(), _stream_ptr(x.device)))
    return loss


def levels():
    """The 16 fp32 NF4 levels the kernels use (host copy)."""
    out = (ctypes.c_float * 16)()
    _lib.check(_lib.lib().qlora_nf4_levels(out))
    return [float(v) for v in out]


def profile_enable(on: bool = True) -> None:
    """Start (resetting the totals) or stop per-kernel event timing in the library."""
    _lib.check(_lib.lib().qlora_profile_enable(1 if on else 0))


def profile_read():
    """{kernel kind: (summed milliseconds, launches)} recorded since profile_enable."""
    out = {}
    for kind, name in enumerate(_lib.KERNEL_KINDS):
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        _lib.check(_lib.lib().qlora_profile_read(kind, ctypes.byref(ms), ctypes.byref(n)))
        out[name] = (ms.value, n.value)
    return out
