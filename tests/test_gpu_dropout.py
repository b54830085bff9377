"""GPU parity of the QLoRA layer with LoRA dropout (inverted dropout on the input of
the low-rank branch, caller-drawn keep mask) against the dropout oracle, through
the C ABI; same tolerance as the layer (bf16 / f16 rel-L2 <= 5e-3 and max <= 1e-2
max, f32 rel-L2 <= 1e-5)."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
from oracle import dropout as odrop
from bit_nf4_quantized_nibble_amd import inputs
from parity import assert_close, oracle_layer, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


def f32(v):
    return float(np.float32(v))


def _case(M, N, K, r, cd, p, seed):
    L = inputs.random_layer(M, N, K, r, seed=seed, cd=cd, with_bias=True)
    mask = inputs.dropout_mask(M, K, p, seed=seed + 1)
    g = to_gpu(L)
    q = qn.quantize(g["W"], L.block_size, L.double_quant, L.dq_group)
    return L, g, q, mask


@pytest.mark.parametrize("cd,path", [("bf16", "fused"), ("bf16", "dequant"), ("f16", "fused"), ("f32", "auto")])
@pytest.mark.parametrize("M,N,K,r", [(300, 200, 320, 8), (129, 257, 128, 24), (4, 128, 256, 16)])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_forward_backward(cd, path, M, N, K, r, p):
    L, g, q, mask = _case(M, N, K, r, cd, p, seed=M + N + r)
    say("dropout", cd, path, M, N, K, r, p)
    mk = mask.cuda()
    y = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], path=path, dropout_mask=mk, dropout_p=p)
    dx, da, db = qn.linear_bwd(q, g["x"], g["dY"], g["A"], g["B"], L.alpha, path=path, dropout_mask=mk,
                               dropout_p=p)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    mf, pf = mask.numpy().astype(np.float64), f32(p)
    ref = odrop.forward(o["x"], o["W"], o["A"], o["B"], o["s"], mf, pf, o["bias"])
    assert_close(to_np(y), ref, cd, "fwd")
    rdx, rda, rdb = odrop.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"], mf, pf)
    assert_close(to_np(dx), rdx, cd, "dX")
    assert_close(to_np(da), rda, cd, "dA")
    assert_close(to_np(db), rdb, cd, "dB")


def test_dropout_full_size_dense_path():
    """4096 tokens through the dequantize-then-GEMM path (the library default there)."""
    (L,) = inputs.prefill(with_dy=True, projections=["o_proj"])
    say("dropout o_proj full")
    mask = inputs.dropout_mask(L.M, L.K, 0.1, seed=3)
    g = to_gpu(L)
    q = qn.quantize(g["W"], 64, True, 256)
    mk = mask.cuda()
    y = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, dropout_mask=mk, dropout_p=0.1)
    dx, da, db = qn.linear_bwd(q, g["x"], g["dY"], g["A"], g["B"], L.alpha, dropout_mask=mk, dropout_p=0.1)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    rng = np.random.default_rng(5)
    rows = rng.integers(0, L.M, 48)
    mf = mask.numpy().astype(np.float64)
    ref = odrop.forward(o["x"][rows], o["W"], o["A"], o["B"], o["s"], mf[rows], f32(0.1))
    assert_close(to_np(y)[rows], ref, "bf16", "fwd rows")
    rdx, _, _ = odrop.backward(o["x"][rows], o["W"], o["A"], o["B"], o["dY"][rows], o["s"], mf[rows], f32(0.1))
    assert_close(to_np(dx)[rows], rdx, "bf16", "dX rows")
    _, rda, rdb = odrop.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"], mf, f32(0.1))
    assert_close(to_np(da), rda, "bf16", "dA")
    assert_close(to_np(db), rdb, "bf16", "dB")


def test_keep_everything_matches_the_plain_layer():
    """p = 0 with every element kept: the forward and dA, dB are the plain layer's bit
    for bit (same kernels on x * 1); dX comes from the base GEMM plus the masked
    low-rank add, so it is compared to the plain call within the tolerance."""
    L, g, q, _ = _case(200, 192, 256, 16, "bf16", 0.0, seed=9)
    say("dropout p=0")
    ones = torch.ones(200, 256, dtype=torch.uint8, device="cuda")
    y0, t0 = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, save_t=True)
    y1, t1 = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, save_t=True, dropout_mask=ones, dropout_p=0.0)
    b0 = qn.linear_bwd(q, g["x"], g["dY"], g["A"], g["B"], L.alpha)
    b1 = qn.linear_bwd(q, g["x"], g["dY"], g["A"], g["B"], L.alpha, dropout_mask=ones, dropout_p=0.0)
    b2 = qn.linear_bwd(q, g["x"], g["dY"], g["A"], g["B"], L.alpha, t_saved=t1, dropout_mask=ones, dropout_p=0.0)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(t0, t1)
    assert torch.equal(b0[1], b1[1]) and torch.equal(b0[2], b1[2])
    assert all(torch.equal(u, v) for u, v in zip(b1, b2))
    assert_close(to_np(b1[0]), to_np(b0[0]).astype(np.float64), "bf16", "dX")
