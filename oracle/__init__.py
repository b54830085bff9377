"""CPU oracle for the QLoRA NF4 linear layer (numpy front end over nf4_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the HIP library and never imports it.

Every function follows a passage of the pages (cited in nf4_oracle.c):
  * ``levels``      -- the 16 NF4 levels (normal quantiles, printed to 3 d.p.);
  * ``quantize``    -- block absmax, nearest level, two codes per byte, optional
                       double quantization of the block scales to u8 + fp32;
  * ``dequantize``  -- fl32(level * scale);
  * ``round_to``    -- round-to-nearest-even into bf16 / f16;
  * ``forward`` / ``backward`` and their ``*_at`` samplers -- the QLoRA layer in
                       fp64: y = x W~^T + (alpha/r)(x A~^T) B~^T (+ bias) and its
                       gradients with respect to x, A and B (W frozen).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_d = ctypes.c_double
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_round_f64.argtypes = [_f64p, _i64, _i32, _vp]
    lib.orc_round_f64.restype = None
    lib.orc_nf4_levels.argtypes = [_f64p, _f32p]
    lib.orc_nf4_levels.restype = None
    lib.orc_nf4_quantize.argtypes = [_f32p, _i64, _i32, _i32, _i32, _u8p, _vp, _vp, _vp, _vp]
    lib.orc_nf4_quantize.restype = ctypes.c_int
    lib.orc_nf4_dequantize.argtypes = [_u8p, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _f32p]
    lib.orc_nf4_dequantize.restype = ctypes.c_int
    for name, a, b in (("orc_f32_to_bf16", _f32p, _u16p), ("orc_f32_to_f16", _f32p, _u16p),
                       ("orc_bf16_to_f32", _u16p, _f32p), ("orc_f16_to_f32", _u16p, _f32p)):
        fn = getattr(lib, name)
        fn.argtypes = [a, b, _i64]
        fn.restype = None
    lib.orc_qlora_fwd.argtypes = [_f32p, _f32p, _f32p, _f32p, _vp, _i64, _i64, _i64, _i64, _d, _f64p]
    lib.orc_qlora_fwd.restype = None
    lib.orc_qlora_fwd_at.argtypes = [_f32p, _f32p, _f32p, _f32p, _vp, _i64, _i64, _i64, _i64, _d,
                                     _i64p, _i64p, _i64, _f64p]
    lib.orc_qlora_fwd_at.restype = None
    lib.orc_qlora_bwd.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, _d,
                                  _vp, _vp, _vp]
    lib.orc_qlora_bwd.restype = None
    lib.orc_qlora_bwd_dx_at.argtypes = [_f32p, _f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, _d,
                                        _i64p, _i64p, _i64, _f64p]
    lib.orc_qlora_bwd_dx_at.restype = None
    lib.orc_qlora_bwd_da_at.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, _d,
                                        _i64p, _i64p, _i64, _f64p]
    lib.orc_qlora_bwd_da_at.restype = None
    lib.orc_qlora_merge.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _d, _i32, _vp]
    lib.orc_qlora_merge.restype = None
    lib.orc_qlora_bwd_db_at.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, _d,
                                        _i64p, _i64p, _i64, _f64p]
    lib.orc_qlora_bwd_db_at.restype = None
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


# --------------------------------------------------------------------------- levels
def levels():
    """(levels in fp64, levels rounded once to fp32), ascending, L0=-1, L7=0, L15=1."""
    lv64 = np.zeros(16, np.float64)
    lv32 = np.zeros(16, np.float32)
    _load().orc_nf4_levels(lv64, lv32)
    return lv64, lv32


# --------------------------------------------------------------------------- quantize
@dataclass
class NF4Ref:
    """Oracle-side quantized tensor: packed codes and the (possibly double-quantized) scales."""
    shape: tuple
    block_size: int
    double_quant: bool
    dq_group: int
    packed: np.ndarray                      # u8 [n/2]
    absmax: Optional[np.ndarray] = None     # f32 [nb]        (no double quant)
    absmax_q: Optional[np.ndarray] = None   # u8  [nb]        (double quant)
    absmax_scale2: Optional[np.ndarray] = None  # f32 [ng]    (double quant)
    codes: Optional[np.ndarray] = None      # u8 [n], one code per element

    @property
    def n(self) -> int:
        return int(np.prod(self.shape))


def quantize(w, block_size: int = 64, double_quant: bool = False, dq_group: int = 256) -> NF4Ref:
    w = _f32(w)
    n = w.size
    if block_size <= 0 or block_size % 2 or n % block_size:
        raise ValueError("n must be a multiple of an even block_size")
    nb = n // block_size
    packed = np.zeros(n // 2, np.uint8)
    codes = np.zeros(n, np.uint8)
    absmax = absmax_q = scale2 = None
    if double_quant:
        absmax_q = np.zeros(nb, np.uint8)
        scale2 = np.zeros((nb + dq_group - 1) // dq_group, np.float32)
    else:
        absmax = np.zeros(nb, np.float32)
    rc = _load().orc_nf4_quantize(w.reshape(-1), n, block_size, int(bool(double_quant)), dq_group,
                                  packed, _ptr(absmax), _ptr(absmax_q), _ptr(scale2), _ptr(codes))
    if rc != 0:
        raise ValueError("oracle quantize failed with status %d" % rc)
    return NF4Ref(tuple(w.shape), block_size, bool(double_quant), dq_group, packed, absmax,
                  absmax_q, scale2, codes)


def dequantize(q: NF4Ref) -> np.ndarray:
    """w_hat = fl32(L[code] * s_hat) as an fp32 array of the original shape."""
    out = np.zeros(q.n, np.float32)
    rc = _load().orc_nf4_dequantize(q.packed, q.n, q.block_size, int(q.double_quant), q.dq_group,
                                    _ptr(q.absmax), _ptr(q.absmax_q), _ptr(q.absmax_scale2), out)
    if rc != 0:
        raise ValueError("oracle dequantize failed with status %d" % rc)
    return out.reshape(q.shape)


# --------------------------------------------------------------------------- dtypes
def to_bits(a, dtype: str) -> np.ndarray:
    """fp32 -> uint16 bit patterns of bf16 / f16, round-to-nearest-even."""
    a = _f32(a)
    out = np.zeros(a.size, np.uint16)
    fn = {"bf16": _load().orc_f32_to_bf16, "f16": _load().orc_f32_to_f16}[dtype]
    fn(a.reshape(-1), out, a.size)
    return out.reshape(a.shape)


def from_bits(bits, dtype: str) -> np.ndarray:
    """uint16 bit patterns of bf16 / f16 -> the exact fp32 values."""
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    out = np.zeros(bits.size, np.float32)
    fn = {"bf16": _load().orc_bf16_to_f32, "f16": _load().orc_f16_to_f32}[dtype]
    fn(bits.reshape(-1), out, bits.size)
    return out.reshape(bits.shape)


def round_to(a, dtype: str) -> np.ndarray:
    """fp32 values rounded (RNE) to the compute dtype, returned as exact fp32."""
    if dtype == "f32":
        return _f32(a).copy()
    return from_bits(to_bits(a, dtype), dtype)


def round64_to(a, dtype: str) -> np.ndarray:
    """fp64 values rounded once (RNE) to the dtype, returned as exact fp32 values."""
    a = np.ascontiguousarray(a, np.float64)
    kind = {"f32": 0, "bf16": 1, "f16": 2}[dtype]
    out = np.empty(a.shape, np.float32 if kind == 0 else np.uint16)
    _load().orc_round_f64(a.reshape(-1), a.size, kind, out.ctypes.data_as(ctypes.c_void_p))
    return out if kind == 0 else from_bits(out, dtype)


# --------------------------------------------------------------------------- layer
def _dims(x, W, A, B):
    M, K = x.shape
    N, K2 = W.shape
    r, K3 = A.shape
    N2, r2 = B.shape
    if not (K == K2 == K3 and N == N2 and r == r2):
        raise ValueError("shape mismatch: x %s W %s A %s B %s" % (x.shape, W.shape, A.shape, B.shape))
    return M, N, K, r


def forward(x, W, A, B, s: float, bias=None) -> np.ndarray:
    """y = x W^T + s (x A^T) B^T (+ bias) in fp64.  Operands are fp32 arrays that
    already hold the compute-dtype values (see ``round_to``)."""
    x, W, A, B = _f32(x), _f32(W), _f32(A), _f32(B)
    M, N, K, r = _dims(x, W, A, B)
    bias = None if bias is None else _f32(bias)
    y = np.zeros((M, N), np.float64)
    _load().orc_qlora_fwd(x, W, A, B, _ptr(bias), M, N, K, r, float(s), y)
    return y


def forward_at(x, W, A, B, s: float, ii, jj, bias=None) -> np.ndarray:
    x, W, A, B = _f32(x), _f32(W), _f32(A), _f32(B)
    M, N, K, r = _dims(x, W, A, B)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    bias = None if bias is None else _f32(bias)
    out = np.zeros(ii.size, np.float64)
    _load().orc_qlora_fwd_at(x, W, A, B, _ptr(bias), M, N, K, r, float(s), ii, jj, ii.size, out)
    return out


def backward(x, W, A, B, dY, s: float, want=("dx", "da", "db")):
    """(dX [M,K], dA [r,K], dB [N,r]) in fp64 for y = x W^T + s (x A^T) B^T, W frozen."""
    x, W, A, B, dY = _f32(x), _f32(W), _f32(A), _f32(B), _f32(dY)
    M, N, K, r = _dims(x, W, A, B)
    assert dY.shape == (M, N)
    dX = np.zeros((M, K), np.float64) if "dx" in want else None
    dA = np.zeros((r, K), np.float64) if "da" in want else None
    dB = np.zeros((N, r), np.float64) if "db" in want else None
    _load().orc_qlora_bwd(x, W, A, B, dY, M, N, K, r, float(s), _ptr(dX), _ptr(dA), _ptr(dB))
    return dX, dA, dB


def backward_dx_at(dY, W, A, B, s: float, ii, kk) -> np.ndarray:
    dY, W, A, B = _f32(dY), _f32(W), _f32(A), _f32(B)
    M, N = dY.shape
    _, K = W.shape
    r = A.shape[0]
    ii = np.ascontiguousarray(ii, np.int64)
    kk = np.ascontiguousarray(kk, np.int64)
    out = np.zeros(ii.size, np.float64)
    _load().orc_qlora_bwd_dx_at(dY, W, A, B, M, N, K, r, float(s), ii, kk, ii.size, out)
    return out


def backward_da_at(x, dY, B, s: float, tt, kk) -> np.ndarray:
    x, dY, B = _f32(x), _f32(dY), _f32(B)
    M, K = x.shape
    N, r = B.shape
    tt = np.ascontiguousarray(tt, np.int64)
    kk = np.ascontiguousarray(kk, np.int64)
    out = np.zeros(tt.size, np.float64)
    _load().orc_qlora_bwd_da_at(x, dY, B, M, N, K, r, float(s), tt, kk, tt.size, out)
    return out


def backward_db_at(x, A, dY, s: float, nn, tt) -> np.ndarray:
    x, A, dY = _f32(x), _f32(A), _f32(dY)
    M, K = x.shape
    r = A.shape[0]
    N = dY.shape[1]
    nn = np.ascontiguousarray(nn, np.int64)
    tt = np.ascontiguousarray(tt, np.int64)
    out = np.zeros(nn.size, np.float64)
    _load().orc_qlora_bwd_db_at(x, A, dY, M, N, K, r, float(s), nn, tt, nn.size, out)
    return out


# --------------------------------------------------------------------------- helpers
def operand(a, dtype: str) -> np.ndarray:
    """Input tensor (torch or numpy, any float dtype) -> exact fp32 values of it.

    bf16 / f16 tensors are decoded bit-exactly; fp32 passes through."""
    try:
        import torch  # only for unpacking torch tensors handed in by tests
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu()
            if a.dtype == torch.bfloat16:
                return from_bits(a.view(torch.int16).numpy().view(np.uint16), "bf16")
            if a.dtype == torch.float16:
                return from_bits(a.view(torch.int16).numpy().view(np.uint16), "f16")
            return _f32(a.float().numpy())
    except ImportError:  # pragma: no cover
        pass
    return _f32(a)


def weight_operand(q: NF4Ref, cd: str) -> np.ndarray:
    """W~ = RNE_cd(dequantize(q)) as exact fp32 values (the operand of the GEMMs)."""
    return round_to(dequantize(q), cd)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((got - ref).ravel()) / (den if den > 0 else 1.0))


def merge(what, A, B, s: float, dtype: str) -> np.ndarray:
    """W_merged = W_hat + s B A, rounded once to dtype ("LoRA and QLoRA, mathematically",
    "The merge math", eq. 6.3.6).  what: the binary32 dequantized weight [N, K]; A, B the
    adapter values.  Returns float32 values for "f32", else the 16-bit patterns."""
    what, A, B = _f32(what), _f32(A), _f32(B)
    N, K = what.shape
    r = A.shape[0]
    assert A.shape == (r, K) and B.shape == (N, r)
    kind = {"f32": 0, "bf16": 1, "f16": 2}[dtype]
    out = np.empty((N, K), np.float32 if kind == 0 else np.uint16)
    _load().orc_qlora_merge(what, A, B, N, K, r, float(s), kind, out.ctypes.data_as(ctypes.c_void_p))
    return out

