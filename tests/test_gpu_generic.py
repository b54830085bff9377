"""GPU parity for every layer the quantize call accepts, beyond the tiled fast paths:
block sizes that are not powers of two from 8 to 512 (quantized one wavefront per
block), layers whose block size is not a multiple of 32, whose cols is not a
multiple of 64, or whose blocks run across rows (the generic tile engine, which
decodes W per element), and adapter ranks above 64 on the fast layouts.

Codes, scales and dequantized weights are compared bit for bit with the oracle;
layer outputs and gradients element by element within the stated tolerance."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
import oracle
from bit_nf4_quantized_nibble_amd import inputs
from parity import TORCH_DT, assert_close, oracle_layer, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols,bs,dq,g", [
    (3, 10, 2, False, 1),        # block 2, n = 30 (not a multiple of 8)
    (3, 10, 6, True, 2),         # block 6, partial last group
    (40, 24, 24, True, 7),
    (64, 96, 96, False, 1),
    (16, 1000, 1000, True, 3),   # one wavefront walks a 1000-element block
    (8, 2048, 2048, True, 256),  # larger than the vectorized kernels take; one global group
    (50, 36, 12, True, 100000),  # group beyond the block count
])
def test_quantize_dequantize_any_block_size(rows, cols, bs, dq, g):
    say("quantize any", rows, cols, bs, dq, g)
    gen = torch.Generator().manual_seed(rows * cols + bs)
    W = torch.randn(rows, cols, generator=gen)
    W.view(-1)[:: max(1, (rows * cols) // 7)] *= 20.0  # a few outliers
    q = qn.quantize(W.cuda(), bs, dq, g)
    torch.cuda.synchronize()
    ref = oracle.quantize(W.numpy(), bs, dq, g)
    assert np.array_equal(q.codes.cpu().numpy(), ref.packed)
    if dq:
        assert np.array_equal(q.absmax_q.cpu().numpy(), ref.absmax_q)
        assert np.array_equal(q.absmax_scale2.cpu().numpy().view(np.uint32), ref.absmax_scale2.view(np.uint32))
    else:
        assert np.array_equal(q.absmax.cpu().numpy().view(np.uint32), ref.absmax.view(np.uint32))
    what = oracle.dequantize(ref)
    for cd in ("f32", "bf16", "f16"):
        out = qn.dequantize(q, TORCH_DT[cd])
        torch.cuda.synchronize()
        exp = oracle.round_to(what, cd)
        got = to_np(out)
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), cd


@pytest.mark.parametrize("M,N,K,r,bs,dq", [
    (40, 72, 40, 8, 8, True),      # cols not a multiple of 64, block 8
    (200, 96, 128, 16, 16, True),  # cols a multiple of 64, block 16
    (33, 64, 96, 5, 6, True),      # block 6, odd rank
    (130, 64, 192, 8, 128, False),  # blocks of 128 run across rows of 192
    (4, 100, 80, 4, 16, True),     # four tokens: the generic engine, not the decode GEMV
])
@pytest.mark.parametrize("cd,path", [("bf16", "auto"), ("bf16", "fused"), ("f16", "auto"), ("f32", "auto")])
def test_layer_generic_layouts(M, N, K, r, bs, dq, cd, path):
    L = inputs.random_layer(M, N, K, r, seed=M + N + K + bs, cd=cd, block_size=bs, double_quant=dq, dq_group=3,
                            with_bias=True)
    say("generic layer", M, N, K, r, bs, dq, cd, path)
    g = to_gpu(L)
    q = qn.quantize(g["W"], bs, dq, 3)
    dt = TORCH_DT[cd]
    y = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    _, t0 = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], path=path, out=y, save_t=True)
    dx, da, db = qn.linear_bwd(q, g["x"], g["dY"], g["A"], g["B"], L.alpha, path=path)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"]), cd, "y")
    ref_t0 = o["x"].astype(np.float64) @ o["A"].astype(np.float64).T
    assert oracle.rel_l2(to_np(t0).astype(np.float64), ref_t0) <= 1e-5, "T0"
    rdx, rda, rdb = oracle.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"])
    assert_close(to_np(dx), rdx, cd, "dX")
    assert_close(to_np(da), rda, cd, "dA")
    assert_close(to_np(db), rdb, cd, "dB")


@pytest.mark.parametrize("r", [96, 128])
@pytest.mark.parametrize("M,N,K", [(300, 256, 512), (4, 320, 1024), (64, 192, 256)])
@pytest.mark.parametrize("path", ["dequant", "fused"])
def test_layer_large_ranks(r, M, N, K, path):
    """Ranks above 64 on the fast layouts: the rank products leave the skinny kernel
    for the generic engine; the low-rank tail of the 256 x 256 GEMMs spans several
    stages; at four tokens the decode GEMV's epilogue takes its general form."""
    L = inputs.random_layer(M, N, K, r, seed=r + M + N, with_bias=True)
    say("large rank", r, M, N, K, path)
    g = to_gpu(L)
    q = qn.quantize(g["W"], L.block_size, L.double_quant, L.dq_group)
    y, t0 = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], path=path, save_t=True)
    dx, da, db = qn.linear_bwd(q, g["x"], g["dY"], g["A"], g["B"], L.alpha, path=path, t_saved=t0)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"]), "bf16", "y")
    rdx, rda, rdb = oracle.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"])
    assert_close(to_np(dx), rdx, "bf16", "dX")
    assert_close(to_np(da), rda, "bf16", "dA")
    assert_close(to_np(db), rdb, "bf16", "dB")
