"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, reports its level table, and refuses invalid calls on the host
before anything is launched (the pointers below are never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from bit_nf4_quantized_nibble_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora_nf4.h")

OK, INVALID, SHAPE, DTYPE, UNSUP, WS = 0, -1, -2, -3, -4, -5
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced by a refused call


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def desc(rows=64, cols=64, bs=64, dq=0, g=256, codes=FAKE, absmax=FAKE, aq=FAKE, s2=FAKE, reserved=0):
    return _lib.QloraNf4(rows, cols, bs, dq, g, reserved, codes, absmax, aq, s2)


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.qlora_abi_version() == 1
    for k, name in enumerate(_lib.KERNEL_KINDS):
        assert lib.qlora_kernel_name(k).decode() == name
    assert lib.qlora_kernel_name(99) == b""


def test_host_level_table_equals_oracle(lib):
    out = (ctypes.c_float * 16)()
    assert lib.qlora_nf4_levels(out) == OK
    _, lv32 = oracle.levels()
    assert np.array_equal(np.array(list(out), np.float32), lv32)


def last_error(lib):
    return lib.qlora_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(bs=63), SHAPE),                    # odd block size
    (dict(rows=10, cols=10, bs=64), SHAPE),  # n not a multiple of the block size
    (dict(dq=1, g=0), INVALID),
    (dict(dq=2), INVALID),
    (dict(reserved=1), INVALID),
    (dict(codes=FAKE + 4), INVALID),         # misaligned codes
    (dict(codes=0), INVALID),
    (dict(absmax=0), INVALID),
    (dict(dq=1, aq=0), INVALID),
    (dict(rows=-1), SHAPE),
])
def test_quantize_refusals(lib, kw, status):
    d = desc(**kw)
    assert lib.qlora_nf4_quantize(FAKE, ctypes.byref(d), None) == status
    assert last_error(lib)


def test_quantize_refuses_null_and_misaligned_weight(lib):
    d = desc()
    assert lib.qlora_nf4_quantize(None, ctypes.byref(d), None) == INVALID
    assert lib.qlora_nf4_quantize(FAKE + 8, ctypes.byref(d), None) == INVALID
    assert lib.qlora_nf4_quantize(FAKE, None, None) == INVALID


def test_empty_tensor_is_a_noop(lib):
    d = desc(rows=0, cols=64, codes=0, absmax=0)
    assert lib.qlora_nf4_quantize(None, ctypes.byref(d), None) == OK
    assert lib.qlora_nf4_dequantize(ctypes.byref(d), 1, None, None) == OK


def test_dequantize_refusals(lib):
    d = desc()
    assert lib.qlora_nf4_dequantize(ctypes.byref(d), 7, FAKE, None) == DTYPE
    assert lib.qlora_nf4_dequantize(ctypes.byref(d), 1, None, None) == INVALID
    assert lib.qlora_nf4_dequantize(ctypes.byref(d), 1, FAKE + 2, None) == INVALID


def fwd(lib, d, x=FAKE, m=128, a=FAKE, b=FAKE, r=8, alpha=16.0, flags=0, bias=None, cd=1, y=FAKE,
        ws=FAKE, ws_bytes=1 << 40):
    return lib.qlora_linear_fwd(ctypes.byref(d), x, m, a, b, r, alpha, flags, bias, cd, y, None, ws,
                                ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(r=0), INVALID),
    (dict(alpha=float("nan")), INVALID),
    (dict(alpha=float("inf")), INVALID),
    (dict(flags=8), INVALID),                # the dropout flag needs the dropout entry point
    (dict(flags=16), INVALID),
    (dict(flags=6), INVALID),                # both path flags
    (dict(x=None), INVALID),
    (dict(a=None), INVALID),
    (dict(b=None), INVALID),
    (dict(y=None), INVALID),
    (dict(cd=3), DTYPE),
    (dict(m=-1), SHAPE),
    (dict(ws_bytes=16), WS),
    (dict(ws=FAKE + 16), WS),
    (dict(x=FAKE + 8), INVALID),             # every device array 16-byte aligned
    (dict(a=FAKE + 4), INVALID),
    (dict(b=FAKE + 2), INVALID),
    (dict(y=FAKE + 8), INVALID),
    (dict(bias=FAKE + 8), INVALID),
])
def test_forward_refusals(lib, kw, status):
    assert fwd(lib, desc(), **kw) == status
    assert last_error(lib)


def test_forward_takes_every_layer_quantize_accepts(lib):
    """No refusal beyond the argument checks: any even block size, any cols, blocks
    that run across rows (m = 0 is a no-op after validation, so nothing launches)."""
    for kw in (dict(rows=64, cols=96, bs=32), dict(rows=64, cols=128, bs=16), dict(rows=64, cols=192, bs=128),
               dict(rows=3, cols=10, bs=6), dict(rows=5, cols=8, bs=40)):
        assert fwd(lib, desc(**kw), m=0) == OK, kw
    assert fwd(lib, desc(), m=0) == OK                          # no tokens: nothing to do


def fwd_cached(lib, w=FAKE, rows=256, cols=512, x=FAKE, m=128, a=FAKE, b=FAKE, r=8, alpha=16.0, flags=0, cd=1,
               y=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.qlora_linear_fwd_cached(w, rows, cols, x, m, a, b, r, alpha, flags, None, cd, y, None, ws, ws_bytes,
                                       None)


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), INVALID),
    (dict(x=None), INVALID),
    (dict(y=None), INVALID),
    (dict(r=0), INVALID),
    (dict(alpha=float("nan")), INVALID),
    (dict(flags=2), INVALID),        # path flags do not apply: W~ is given
    (dict(cd=0), DTYPE),             # f32 has no dense 256 x 256 GEMM
    (dict(cols=96), UNSUP),
    (dict(rows=0), SHAPE),
    (dict(ws_bytes=16), WS),
    (dict(m=0), OK),
])
def test_forward_cached_refusals(lib, kw, status):
    assert fwd_cached(lib, **kw) == status


def test_forward_cached_workspace(lib):
    cached = lib.qlora_workspace_bytes(2, 2048, 4096, 4096, 64, 1)
    dense = lib.qlora_workspace_bytes(0 | (4 << 8), 2048, 4096, 4096, 64, 1)
    assert 0 < cached and dense - cached >= 4096 * 4096 * 2      # no copy of W~ in the workspace
    assert lib.qlora_workspace_bytes(2 | (1 << 8), 2048, 4096, 4096, 64, 1) == cached  # rsLoRA
    assert lib.qlora_workspace_bytes(2 | (2 << 8), 2048, 4096, 4096, 64, 1) == 0       # path flag
    assert lib.qlora_workspace_bytes(2, 2048, 4096, 4096, 64, 0) == 0                  # f32


def test_backward_refusals(lib):
    d = desc()

    def bwd(dy=FAKE, da=FAKE, db=FAKE, m=128, ws_bytes=1 << 40, r=8, dx=FAKE, t=None):
        return lib.qlora_linear_bwd(ctypes.byref(d), FAKE, dy, m, FAKE, FAKE, r, 16.0, 0, 1, t,
                                    dx, da, db, FAKE, ws_bytes, None)

    assert bwd(dy=FAKE + 8) == INVALID      # every device array 16-byte aligned
    assert bwd(dx=FAKE + 2) == INVALID
    assert bwd(da=FAKE + 4) == INVALID
    assert bwd(db=FAKE + 4) == INVALID
    assert bwd(t=FAKE + 4) == INVALID
    assert bwd(dy=None) == INVALID
    assert bwd(da=None) == INVALID
    assert bwd(db=None) == INVALID
    assert bwd(m=0) == SHAPE
    assert bwd(r=0) == INVALID
    assert bwd(ws_bytes=8) == WS


def test_workspace_query(lib):
    assert lib.qlora_workspace_bytes(0, 128, 64, 64, 0, 1) == 0      # r < 1
    assert lib.qlora_workspace_bytes(9, 128, 64, 64, 8, 1) == 0      # bad op
    assert lib.qlora_workspace_bytes(0, 128, 64, 64, 8, 5) == 0      # bad dtype
    small = lib.qlora_workspace_bytes(1, 128, 4096, 4096, 64, 1)
    big = lib.qlora_workspace_bytes(1, 4096, 4096, 4096, 64, 1)
    # a short call can hold more partial sums (its single round is cut into up to 8
    # slices; at most one round of 256 x 256 fp32 tiles, 64 MiB on 256 CUs)
    assert 0 < small and big % 256 == 0 and small % 256 == 0
    assert small <= big + 256 * 256 * 256 * 4
    assert lib.qlora_workspace_bytes(0, 4, 4096, 4096, 16, 1) >= 4 * 16 * 4
    # the dequantize-then-GEMM path holds W~ (forward) or W~^T (dX) in the workspace
    fused = lib.qlora_workspace_bytes(0 | (2 << 8), 2048, 4096, 4096, 64, 1)
    dense = lib.qlora_workspace_bytes(0 | (4 << 8), 2048, 4096, 4096, 64, 1)
    assert dense - fused >= 4096 * 4096 * 2
    assert lib.qlora_workspace_bytes(0, 2048, 4096, 4096, 64, 1) == dense      # the default path
    # the default forward of 65 to 768 tokens takes the fused kernel when r is a multiple
    # of 8 (also for a decode-GEMV candidate whose layout sends it to the GEMM path)
    for m in (32, 512, 768):
        assert lib.qlora_workspace_bytes(0, m, 4096, 4096, 64, 1) == lib.qlora_workspace_bytes(2 << 8, m, 4096, 4096, 64, 1)
        fused, dense = (lib.qlora_workspace_bytes(f, m, 4096, 4096, 64, 1) for f in (0, 4 << 8))
        # never more than dequantize-then-GEMM; at 512 tokens as much: the fused kernel cuts
        # its 32 tiles into eight contraction slices, whose fp32 partial sums take as much as
        # W~ and the dense kernel's four slices together
        assert fused < dense if m != 512 else fused <= dense
        assert lib.qlora_workspace_bytes(0, m, 4096, 4096, 12, 1) == lib.qlora_workspace_bytes(4 << 8, m, 4096, 4096, 12, 1)
    assert lib.qlora_workspace_bytes(0, 769, 4096, 4096, 64, 1) == lib.qlora_workspace_bytes(4 << 8, 769, 4096, 4096, 64, 1)
    # the backward keeps dequantize-then-GEMM by default
    assert lib.qlora_workspace_bytes(1, 512, 4096, 4096, 64, 1) == lib.qlora_workspace_bytes(1 | (4 << 8), 512, 4096, 4096, 64, 1)
    assert lib.qlora_workspace_bytes(1 | (4 << 8), 512, 4096, 4096, 64, 1) >= 4096 * 4096 * 2
    assert lib.qlora_workspace_bytes(0 | (16 << 8), 512, 4096, 4096, 64, 1) == 0  # unknown flag
    # LoRA dropout stages x M (and, in the backward, a zero dT operand) in the workspace
    for op in (0, 1):
        plain = lib.qlora_workspace_bytes(op, 512, 4096, 4096, 64, 1)
        assert lib.qlora_workspace_bytes(op | (8 << 8), 512, 4096, 4096, 64, 1) >= plain + 512 * 4096 * 2
    assert lib.qlora_workspace_bytes(0 | (8 << 8), 4, 4096, 4096, 16, 1) >= 4 * 4096 * 2  # GEMM path, not GEMV
    assert lib.qlora_workspace_bytes(0 | (4 << 8), 512, 4096, 4096, 64, 0) == \
        lib.qlora_workspace_bytes(0 | (2 << 8), 512, 4096, 4096, 64, 0)       # f32 has no dense path


def test_binding_rejects_cpu_tensors():
    import torch

    import bit_nf4_quantized_nibble_amd as q
    with pytest.raises(ValueError):
        q.quantize(torch.zeros(64, 64))
    assert q.dtype_code(torch.bfloat16) == 1 and q.dtype_code(torch.float16) == 2
    with pytest.raises(TypeError):
        q.dtype_code(torch.int8)
    with pytest.raises(ValueError):
        q._flags(False, "fast")
    assert q._flags(True, "dequant") == 5 and q._flags(False, "fused") == 2


def merge(lib, d, a=FAKE, b=FAKE, r=8, alpha=16.0, flags=0, cd=1, out=FAKE):
    return lib.qlora_merge(ctypes.byref(d), a, b, r, alpha, flags, cd, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(r=0), INVALID),
    (dict(alpha=float("nan")), INVALID),
    (dict(flags=2), INVALID),                # path flags mean nothing to the merge
    (dict(flags=4), INVALID),
    (dict(a=None), INVALID),
    (dict(b=None), INVALID),
    (dict(out=None), INVALID),
    (dict(cd=5), DTYPE),
])
def test_merge_refusals(lib, kw, status):
    assert merge(lib, desc(), **kw) == status
    assert last_error(lib)


def test_merge_shape_refusals_and_empty(lib):
    assert merge(lib, desc(rows=3, cols=5, bs=2)) == SHAPE     # 15 elements, block 2
    assert merge(lib, desc(rows=0, cols=64, codes=0, absmax=0), a=None, b=None, out=None) == OK
    assert merge(lib, desc(rows=4194241, cols=64, bs=64)) == UNSUP


def test_training_entry_points_refuse_on_the_host(lib):
    o = _lib.QloraAdamW(1e-3, 0.9, 0.999, 1e-8, 0.0)
    bad = _lib.QloraAdamW(1e-3, 1.0, 0.999, 1e-8, 0.0)
    assert lib.qlora_mse_loss_grad(FAKE, FAKE, 10, 7, FAKE, FAKE, FAKE, 4096, None) == DTYPE
    assert lib.qlora_mse_loss_grad(FAKE, None, 10, 1, FAKE, FAKE, FAKE, 4096, None) == INVALID
    assert lib.qlora_mse_loss_grad(FAKE, FAKE, 10, 1, FAKE, FAKE, FAKE, 16, None) == WS
    assert lib.qlora_mse_loss_grad(None, None, 0, 1, None, None, None, 0, None) == OK
    assert lib.qlora_adamw_step(FAKE, FAKE, FAKE, FAKE, 10, ctypes.byref(o), 0, None, 1, None) == INVALID
    assert lib.qlora_adamw_step(FAKE, FAKE, FAKE, FAKE, 10, ctypes.byref(bad), 1, None, 1, None) == INVALID
    assert lib.qlora_adamw_step(FAKE, None, FAKE, FAKE, 10, ctypes.byref(o), 1, None, 1, None) == INVALID
    assert lib.qlora_adamw_step(FAKE, FAKE, FAKE, FAKE, 10, None, 1, None, 1, None) == INVALID
    d0, d1 = desc(rows=128, cols=64), desc(rows=64, cols=96)
    L = (_lib.QloraStackLayer * 2)(_lib.QloraStackLayer(ctypes.pointer(d0), *([FAKE] * 10)),
                                   _lib.QloraStackLayer(ctypes.pointer(d1), *([FAKE] * 10)))
    args = lambda n: (L, n, FAKE, 16, FAKE, 8, 16.0, 0, 1, ctypes.byref(o), 1, FAKE, FAKE, 1 << 40, None)
    assert lib.qlora_stack_train_step(*args(2)) == SHAPE              # 64 outputs feed 96 inputs
    assert lib.qlora_stack_workspace_bytes(L, 2, 16, 8, 1, 0) == 0
    assert lib.qlora_stack_workspace_bytes(L, 1, 16, 8, 1, 0) > 0
    assert lib.qlora_stack_train_step(*args(0)) == SHAPE


def test_dropout_entry_points_refuse_on_the_host(lib):
    d = desc()
    f = lambda **kw: lib.qlora_linear_fwd_dropout(
        ctypes.byref(d), FAKE, 128, FAKE, FAKE, 8, 16.0, 0, None, 1, kw.get("mask", FAKE), kw.get("p", 0.1), FAKE,
        None, FAKE, 1 << 40, None)
    assert f(mask=None) == INVALID
    assert f(p=1.0) == INVALID
    assert f(p=-0.1) == INVALID
    assert f(p=float("nan")) == INVALID
    b = lambda **kw: lib.qlora_linear_bwd_dropout(
        ctypes.byref(d), FAKE, FAKE, 128, FAKE, FAKE, 8, 16.0, 0, 1, kw.get("mask", FAKE), kw.get("p", 0.1), None,
        FAKE, FAKE, FAKE, FAKE, kw.get("ws_bytes", 1 << 40), None)
    assert b(mask=None) == INVALID
    assert b(p=1.5) == INVALID
    assert b(ws_bytes=16) == WS


def group_args(descs, n=None):
    n = len(descs) if n is None else n
    W = (ctypes.POINTER(_lib.QloraNf4) * len(descs))(*[ctypes.pointer(d) for d in descs])
    A = (ctypes.c_void_p * len(descs))(*([FAKE] * len(descs)))
    R = (ctypes.c_int32 * len(descs))(*([8] * len(descs)))
    AL = (ctypes.c_float * len(descs))(*([16.0] * len(descs)))
    return W, A, R, AL


def group_fwd(lib, descs, g=None, x=FAKE, m=128, flags=0, bias=None, cd=1, y=FAKE, ws=FAKE, ws_bytes=1 << 40):
    W, A, R, AL = group_args(descs)
    return lib.qlora_linear_fwd_group(len(descs) if g is None else g, W, x, m, A, A, R, AL, flags, bias, cd, y,
                                      None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=0), INVALID),
    (dict(g=9), INVALID),
    (dict(flags=2), INVALID),         # the group takes the rsLoRA flag only
    (dict(y=None), INVALID),
    (dict(y=FAKE + 8), INVALID),
    (dict(bias=FAKE + 4), INVALID),
    (dict(cd=5), DTYPE),
    (dict(ws_bytes=16), WS),
])
def test_group_forward_refusals(lib, kw, status):
    assert group_fwd(lib, [desc(), desc(rows=128)], **kw) == status
    assert last_error(lib)


def test_group_refuses_mixed_cols_and_accepts_no_tokens(lib):
    assert group_fwd(lib, [desc(), desc(cols=128)]) == SHAPE
    assert group_fwd(lib, [desc(), desc(rows=128)], m=0) == OK


def test_group_backward_refusals(lib):
    descs = [desc(), desc(rows=128)]
    W, A, R, AL = group_args(descs)
    G = (ctypes.c_void_p * 2)(FAKE, FAKE)
    Z = (ctypes.c_void_p * 2)(FAKE, None)

    def bwd(dy=FAKE, dx=FAKE, da=G, db=G, m=128, ws_bytes=1 << 40):
        return lib.qlora_linear_bwd_group(2, W, FAKE, dy, m, A, A, R, AL, 0, 1, None, dx, da, db, FAKE, ws_bytes,
                                          None)
    assert bwd(m=0) == SHAPE
    assert bwd(dy=None) == INVALID
    assert bwd(da=Z) == INVALID
    assert bwd(dx=FAKE + 2) == INVALID
    assert bwd(ws_bytes=8) == WS


def test_group_workspace_query(lib):
    """The tiled path holds the concatenated W~ (bf16 q / k / v at 4096 tokens);
    invalid queries give 0."""
    descs = [desc(rows=4096, cols=4096), desc(rows=1024, cols=4096), desc(rows=1024, cols=4096)]
    W = (ctypes.POINTER(_lib.QloraNf4) * 3)(*[ctypes.pointer(d) for d in descs])
    R = (ctypes.c_int32 * 3)(64, 64, 64)
    fwd_b = lib.qlora_group_workspace_bytes(0, 3, W, 4096, R, 1)
    bwd_b = lib.qlora_group_workspace_bytes(1, 3, W, 4096, R, 1)
    assert fwd_b >= 6144 * 4096 * 2 and bwd_b >= 6144 * 4096 * 2
    assert lib.qlora_group_workspace_bytes(0, 0, W, 4096, R, 1) == 0
    assert lib.qlora_group_workspace_bytes(2, 3, W, 4096, R, 1) == 0
    mixed = (ctypes.POINTER(_lib.QloraNf4) * 2)(ctypes.pointer(desc()), ctypes.pointer(desc(cols=128)))
    assert lib.qlora_group_workspace_bytes(0, 2, mixed, 16, R, 1) == 0
