"""Shared helpers for the GPU parity tests: move seeded inputs to the device, run
the oracle on the same inputs, and compare to the tolerance the layer is held to.

Tolerance (floating-point outputs, fp32 accumulation): bf16 / f16 compute
  rel-L2 = ||g - r|| / ||r|| <= 5e-3  and  max |g - r| <= 1e-2 * max |r|;
f32 compute: rel-L2 <= 1e-5.  Integer / byte / dequantized outputs are bit-exact.
"""
import sys

import numpy as np
import torch

import oracle

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def say(*args):
    """Name the case before any GPU step so a crash can be attributed."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def assert_close(got, ref, cd, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    rel = oracle.rel_l2(got, ref)
    mx = float(np.max(np.abs(got - ref))) if got.size else 0.0
    ref_max = float(np.max(np.abs(ref))) if ref.size else 0.0
    if cd == "f32":
        assert rel <= 1e-5, "%s: rel-L2 %.3e > 1e-5" % (what, rel)
    else:
        assert rel <= 5e-3, "%s: rel-L2 %.3e > 5e-3" % (what, rel)
        assert mx <= 1e-2 * ref_max, "%s: max abs %.3e > 1e-2 * %.3e" % (what, mx, ref_max)
    return rel, mx


def to_np(t):
    """GPU/CPU tensor -> exact fp32/fp64 numpy values."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.numpy()


def oracle_layer(L, cd=None):
    """Oracle operands for a LayerInputs: quantize W, W~ in the compute dtype, and
    exact fp32 copies of x, A, B, dY, bias."""
    cd = cd or L.cd
    q = oracle.quantize(L.W.numpy(), L.block_size, L.double_quant, L.dq_group)
    Wc = oracle.weight_operand(q, cd)
    ops = dict(q=q, W=Wc, x=oracle.operand(L.x, cd), A=oracle.operand(L.A, cd),
               B=oracle.operand(L.B, cd), s=L.alpha / L.r)
    ops["dY"] = oracle.operand(L.dY, cd) if L.dY is not None else None
    ops["bias"] = oracle.operand(L.bias, cd) if L.bias is not None else None
    return ops


def to_gpu(L):
    dev = "cuda"
    return dict(W=L.W.to(dev), x=L.x.to(dev), A=L.A.to(dev), B=L.B.to(dev),
                dY=None if L.dY is None else L.dY.to(dev),
                bias=None if L.bias is None else L.bias.to(dev))
