"""ctypes loader for libqlora_nf4.so (the C ABI of include/qlora_nf4.h).

There is no fallback: if the HIP library cannot be built or loaded, every call
raises.  Loading needs no GPU; launching does.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_nf4.so")

QLORA_OK = 0
STATUS_NAMES = {
    0: "QLORA_OK", -1: "QLORA_ERR_INVALID_ARG", -2: "QLORA_ERR_SHAPE", -3: "QLORA_ERR_DTYPE",
    -4: "QLORA_ERR_UNSUPPORTED", -5: "QLORA_ERR_WORKSPACE", -6: "QLORA_ERR_HIP",
}
QLORA_F32, QLORA_BF16, QLORA_F16 = 0, 1, 2
QLORA_FLAG_RSLORA, QLORA_FLAG_FUSED, QLORA_FLAG_DEQUANT_GEMM, QLORA_FLAG_DROPOUT = 1, 2, 4, 8
QLORA_OP_FWD, QLORA_OP_BWD, QLORA_OP_FWD_CACHED, QLORA_OP_FLAGS_SHIFT = 0, 1, 2, 8

# Every function the header declares, for the export check.
EXPORTED = (
    "qlora_nf4_quantize", "qlora_nf4_dequantize", "qlora_linear_fwd", "qlora_linear_bwd",
    "qlora_workspace_bytes", "qlora_last_error", "qlora_nf4_levels", "qlora_abi_version",
    "qlora_profile_enable", "qlora_profile_read", "qlora_kernel_name", "qlora_merge",
    "qlora_mse_loss_grad", "qlora_adamw_step", "qlora_stack_train_step", "qlora_stack_workspace_bytes",
    "qlora_linear_fwd_dropout", "qlora_linear_bwd_dropout", "qlora_linear_fwd_cached",
    "qlora_linear_fwd_noalloc", "qlora_noalloc_scratch_bytes",
    "qlora_linear_fwd_group", "qlora_linear_bwd_group", "qlora_group_workspace_bytes",
)
QLORA_GROUP_MAX = 8
QLORA_MSE_WORKSPACE_BYTES = 4096
KERNEL_KINDS = ("quantize", "dequantize", "lora_down", "reduce", "fwd_gemm", "gemv",
                "bwd_dt", "bwd_dx", "bwd_da", "bwd_db", "merge", "loss", "optim")


class QloraNf4(ctypes.Structure):
    """Mirror of qlora_nf4_t."""
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("double_quant", ctypes.c_int32),
        ("dq_group", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("codes", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("absmax_q", ctypes.c_void_p),
        ("absmax_scale2", ctypes.c_void_p),
    ]


class QloraAdamW(ctypes.Structure):
    """Mirror of qlora_adamw_t."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


class QloraStackLayer(ctypes.Structure):
    """Mirror of qlora_stack_layer_t."""
    _fields_ = [("w", ctypes.POINTER(QloraNf4))] + [
        (name, ctypes.c_void_p) for name in ("lora_a", "lora_b", "a32", "b32", "m_a", "v_a", "m_b", "v_b",
                                             "grad_a", "grad_b")]


class QloraError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__("%s (%d): %s" % (STATUS_NAMES.get(status, "?"), status, message))


_lib = None
_lock = threading.Lock()


def _declare(lib):
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    P = ctypes.POINTER(QloraNf4)
    lib.qlora_nf4_quantize.argtypes = [vp, P, vp]
    lib.qlora_nf4_dequantize.argtypes = [P, i32, vp, vp]
    lib.qlora_linear_fwd.argtypes = [P, vp, i64, vp, vp, i32, f32, i32, vp, i32, vp, vp, vp, sz, vp]
    lib.qlora_linear_bwd.argtypes = [P, vp, vp, i64, vp, vp, i32, f32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.qlora_merge.argtypes = [P, vp, vp, i32, f32, i32, i32, vp, vp]
    PA = ctypes.POINTER(QloraAdamW)
    PS = ctypes.POINTER(QloraStackLayer)
    lib.qlora_mse_loss_grad.argtypes = [vp, vp, i64, i32, vp, vp, vp, sz, vp]
    lib.qlora_adamw_step.argtypes = [vp, vp, vp, vp, i64, PA, i32, vp, i32, vp]
    lib.qlora_stack_train_step.argtypes = [PS, i32, vp, i64, vp, i32, f32, i32, i32, PA, i32, vp, vp, sz, vp]
    lib.qlora_stack_workspace_bytes.argtypes = [PS, i32, i64, i32, i32, i32]
    lib.qlora_stack_workspace_bytes.restype = sz
    lib.qlora_linear_fwd_dropout.argtypes = [P, vp, i64, vp, vp, i32, f32, i32, vp, i32, vp, f32, vp, vp, vp, sz, vp]
    lib.qlora_linear_bwd_dropout.argtypes = [P, vp, vp, i64, vp, vp, i32, f32, i32, i32, vp, f32, vp, vp, vp, vp, vp,
                                             sz, vp]
    lib.qlora_linear_fwd_cached.argtypes = [vp, i64, i64, vp, i64, vp, vp, i32, f32, i32, vp, i32, vp, vp, vp, sz, vp]
    lib.qlora_linear_fwd_noalloc.argtypes = [P, vp, i64, vp, vp, i32, f32, i32, vp, i32, vp, vp, vp]
    lib.qlora_linear_fwd_noalloc.restype = ctypes.c_int
    lib.qlora_noalloc_scratch_bytes.argtypes = []
    lib.qlora_noalloc_scratch_bytes.restype = sz
    lib.qlora_workspace_bytes.argtypes = [i32, i64, i64, i64, i32, i32]
    lib.qlora_workspace_bytes.restype = sz
    lib.qlora_last_error.argtypes = []
    lib.qlora_last_error.restype = ctypes.c_char_p
    lib.qlora_nf4_levels.argtypes = [ctypes.POINTER(ctypes.c_float)]
    lib.qlora_abi_version.argtypes = []
    lib.qlora_profile_enable.argtypes = [i32]
    lib.qlora_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.qlora_kernel_name.argtypes = [i32]
    lib.qlora_kernel_name.restype = ctypes.c_char_p
    # group calls: arrays of g pointers / values
    lib.qlora_linear_fwd_group.argtypes = [i32, vp, vp, i64, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, sz, vp]
    lib.qlora_linear_bwd_group.argtypes = [i32, vp, vp, vp, i64, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.qlora_group_workspace_bytes.argtypes = [i32, i32, vp, i64, vp, i32]
    lib.qlora_group_workspace_bytes.restype = sz
    for name in ("qlora_nf4_quantize", "qlora_nf4_dequantize", "qlora_linear_fwd",
                 "qlora_linear_bwd", "qlora_nf4_levels", "qlora_abi_version",
                 "qlora_profile_enable", "qlora_profile_read", "qlora_merge", "qlora_mse_loss_grad",
                 "qlora_adamw_step", "qlora_stack_train_step", "qlora_linear_fwd_dropout",
                 "qlora_linear_bwd_dropout", "qlora_linear_fwd_group", "qlora_linear_bwd_group"):
        getattr(lib, name).restype = ctypes.c_int


def lib():
    """The loaded library (built in-tree first if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: its HIP runtime (same soname) must be the one this library binds
    # to, so that device pointers and streams are shared.
    import torch  # noqa: F401
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                from . import build as _build
                _build.build()
            handle = ctypes.CDLL(LIB_PATH)
            _declare(handle)
            _lib = handle
    return _lib


def check(status: int) -> None:
    if status != QLORA_OK:
        msg = lib().qlora_last_error()
        raise QloraError(status, msg.decode() if msg else "")
