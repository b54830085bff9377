"""GPU parity of the QLoRA layer (fused dequant-GEMM and dequantize-then-GEMM
forward, decode GEMV and the backward) against the fp64 oracle on the same seeded
inputs, through the C ABI.

Small cases compare every element (several tiles plus ragged tails in M, N and
the rank); the decode workload is compared in full.  The full-size prefill and
training workloads are in test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
import oracle
from bit_nf4_quantized_nibble_amd import inputs
from parity import assert_close, oracle_layer, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


def run_fwd(L, g, q, **kw):
    y = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], **kw)
    torch.cuda.synchronize()
    return y


def gpu_q(L, g):
    return qn.quantize(g["W"], L.block_size, L.double_quant, L.dq_group)


# ----------------------------------------------------------------------------- forward
def test_forward_tiny():
    L = inputs.tiny()
    say("fwd tiny")
    g = to_gpu(L)
    y = run_fwd(L, g, gpu_q(L, g))
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"]), "bf16", "tiny fwd")


PATHS = [("bf16", "fused"), ("bf16", "dequant"), ("f16", "fused"), ("f16", "dequant"), ("f32", "auto")]


@pytest.mark.parametrize("cd,path", PATHS)
@pytest.mark.parametrize("M,N,K,r,bs,dq,bias", [
    (300, 200, 320, 8, 64, True, True),     # ragged M and N, 5 K-steps, bias
    (129, 257, 128, 24, 32, False, False),  # ragged by one, rank not a multiple of 16
    (64, 96, 256, 64, 128, True, False),
    (17, 128, 64, 3, 64, False, True),      # smallest GEMM-path M, odd rank
])
def test_forward_ragged(cd, path, M, N, K, r, bs, dq, bias):
    L = inputs.random_layer(M, N, K, r, seed=M + N + r, cd=cd, block_size=bs, double_quant=dq,
                            with_bias=bias, with_dy=False)
    say("fwd ragged", cd, path, M, N, K, r, bs, dq, bias)
    g = to_gpu(L)
    y = run_fwd(L, g, gpu_q(L, g), path=path)
    o = oracle_layer(L)
    ref = oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"])
    assert_close(to_np(y), ref, cd, "fwd %s %dx%dx%d r%d" % (cd, M, N, K, r))


@pytest.mark.parametrize("m", [1, 4, 16])
def test_forward_decode_full(m):
    L = inputs.decode(m)
    say("fwd decode m", m)
    g = to_gpu(L)
    y = run_fwd(L, g, gpu_q(L, g))
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"]), "bf16", "decode m%d" % m)


@pytest.mark.parametrize("m", [2, 7, 13])
@pytest.mark.parametrize("cd", ["f16", "f32"])
def test_forward_decode_small_shapes(m, cd):
    L = inputs.random_layer(m, 320, 512, 16, seed=m, cd=cd, with_bias=True, with_dy=False)
    say("fwd decode small", m, cd)
    g = to_gpu(L)
    y = run_fwd(L, g, gpu_q(L, g))
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"]), cd, "decode small")


@pytest.mark.parametrize("m,N,K,r,bias", [
    (3, 200, 512, 5, True),     # odd rank: the epilogue's general path; ragged N
    (16, 264, 1024, 64, True),  # rank 64: the single-round path at its limit
    (1, 136, 512, 24, False),   # rank 24 (a multiple of 8, not of 16)
])
def test_forward_decode_epilogue_paths(m, N, K, r, bias):
    """Decode (m <= 16) in bf16 with the saved T0 = x A^T, bias on and off, ranks that
    take either path of the split-K GEMV's epilogue."""
    L = inputs.random_layer(m, N, K, r, seed=m * 100 + r, cd="bf16", with_bias=bias, with_dy=False)
    say("fwd decode epilogue", m, N, K, r, bias)
    g = to_gpu(L)
    y, t0 = qn.linear_fwd(gpu_q(L, g), g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], save_t=True)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"]), "bf16", "decode y")
    ref_t0 = np.asarray(o["x"], np.float64) @ np.asarray(o["A"], np.float64).T
    got = to_np(t0).astype(np.float64)
    assert oracle.rel_l2(got, ref_t0) <= 1e-5, "decode T0"


@pytest.mark.parametrize("m,N,K,r,dq,bias", [
    (5, 72, 8192, 16, True, True),     # 8 contraction slices of 1024
    (16, 130, 1536, 12, False, False),  # cols not a multiple of 1024: the VALU GEMV; fp32 block scales, ragged N
    (1, 16, 512, 1, True, True),        # half a slice: the VALU GEMV, one row block, rank 1
    (7, 256, 3072, 8, True, True),      # 3 slices
    (9, 4096, 14336, 64, True, False),  # the down-projection shape: 14 slices
])
def test_forward_decode_more_shapes(m, N, K, r, dq, bias):
    """Decode (m <= 16) with the saved T0 on the slice counts and scale forms the
    full-size cases do not reach."""
    L = inputs.random_layer(m, N, K, r, seed=7 * m + N + r, cd="bf16", double_quant=dq, with_bias=bias,
                            with_dy=False)
    say("fwd decode shapes", m, N, K, r, dq, bias)
    g = to_gpu(L)
    y, t0 = qn.linear_fwd(gpu_q(L, g), g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], save_t=True)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"]), "bf16", "decode y")
    ref_t0 = np.asarray(o["x"], np.float64) @ np.asarray(o["A"], np.float64).T
    assert oracle.rel_l2(to_np(t0).astype(np.float64), ref_t0) <= 1e-5, "decode T0"


@pytest.mark.parametrize("m,N,K,r,bias", [
    (17, 200, 1024, 16, True),    # one past the decode size: two token groups, ragged N
    (32, 4096, 4096, 16, False),  # the decode weight at 32 tokens
    (33, 96, 2048, 5, True),      # three token groups used of four, odd rank
    (48, 320, 8192, 64, True),    # eight slices, rank 64
    (64, 1024, 4096, 24, False),  # the largest count the split-K kernel takes
    (40, 4096, 14336, 64, True),  # the down-projection shape: 14 slices, three token groups
    (24, 14336, 4096, 16, True),  # the gate shape: workgroups loop over 3 or 4 row tiles each
    (64, 6170, 4096, 24, False),  # four token groups looping over a ragged last row tile
])
def test_forward_medium_token_counts(m, N, K, r, bias):
    """17 to 64 tokens without a path flag: the split-K MFMA kernel decodes each W~
    fragment once for up to four 16-token column groups."""
    L = inputs.random_layer(m, N, K, r, seed=3 * m + N + r, cd="bf16", with_bias=bias, with_dy=False)
    say("fwd medium m", m, N, K, r, bias)
    g = to_gpu(L)
    y = torch.full((m, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    _, t0 = qn.linear_fwd(gpu_q(L, g), g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], save_t=True, out=y)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"]), "bf16", "medium y")
    ref_t0 = np.asarray(o["x"], np.float64) @ np.asarray(o["A"], np.float64).T
    assert oracle.rel_l2(to_np(t0).astype(np.float64), ref_t0) <= 1e-5, "medium T0"


@pytest.mark.parametrize("m,N,K,r,bias", [
    (65, 320, 1024, 16, True),     # one past the split-K GEMV's range: the fused kernel
    (512, 1024, 2048, 64, False),  # 512 tokens, one GPU's share of a data-parallel x8 step
    (768, 640, 1024, 8, True),     # the last count the fused kernel takes without a path flag
    (769, 640, 1024, 8, True),     # the first past it: dequantize-then-GEMM
    (700, 512, 1024, 12, False),   # rank not a multiple of 8: dequantize-then-GEMM
])
def test_forward_default_route_65_to_768(m, N, K, r, bias):
    """65 to 768 tokens without a path flag: the fused forward when r is a multiple of 8,
    dequantize-then-GEMM otherwise and above; every element against the oracle, and
    the forced dequantize-then-GEMM path within the same tolerance."""
    L = inputs.random_layer(m, N, K, r, seed=5 * m + N + r, cd="bf16", with_bias=bias, with_dy=False)
    say("fwd default route m", m, N, K, r, bias)
    g = to_gpu(L)
    q = gpu_q(L, g)
    y = torch.full((m, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], out=y)
    yd = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], path="dequant")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "unwritten outputs"
    o = oracle_layer(L)
    ref = oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"])
    assert_close(to_np(y), ref, "bf16", "default route y")
    assert_close(to_np(yd), ref, "bf16", "dequant y")


def test_forward_512_tokens_gate_shape():
    """The gate projection's shape (14336 x 4096, r 64) at 512 tokens on the default
    route (the fused kernel: 2 x 56 tiles cut into 2 slices): outputs NaN-filled and all
    finite, whole rows compared for one row in every band of 32 and both edge rows of
    each 256-row tile."""
    m, N, K, r = 512, 14336, 4096, 64
    L = inputs.random_layer(m, N, K, r, seed=512, cd="bf16", with_bias=False, with_dy=False)
    say("fwd 512 tokens gate shape")
    g = to_gpu(L)
    q = gpu_q(L, g)
    y = torch.full((m, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, out=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "unwritten outputs"
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([np.arange(0, m, 32) + rng.integers(0, 32, m // 32),
                                     np.arange(0, m, 256), np.arange(255, m, 256)]))
    o = oracle_layer(L)
    xs = np.ascontiguousarray(np.asarray(o["x"])[rows])
    ref = oracle.forward(xs, o["W"], o["A"], o["B"], o["s"], None)
    assert_close(to_np(y[torch.from_numpy(rows).cuda()]), ref, "bf16", "gate shape at 512 tokens")


def test_forward_save_t_and_leading_dims():
    L = inputs.random_layer(60, 128, 256, 8, seed=3, with_dy=False)
    say("fwd save_t")
    g = to_gpu(L)
    q = gpu_q(L, g)
    y, t0 = qn.linear_fwd(q, g["x"].reshape(3, 20, 256), g["A"], g["B"], L.alpha, save_t=True)
    torch.cuda.synchronize()
    assert y.shape == (3, 20, 128)
    o = oracle_layer(L)
    T0 = o["x"].astype(np.float64) @ o["A"].astype(np.float64).T
    assert_close(to_np(t0), T0, "f32", "T0")
    assert_close(to_np(y).reshape(60, 128), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"]), "bf16", "y")


def test_forward_b_zero_and_alpha_linearity():
    L = inputs.random_layer(256, 256, 512, 16, seed=4, with_dy=False)
    say("fwd B=0 / alpha")
    g = to_gpu(L)
    q = gpu_q(L, g)
    o = oracle_layer(L)
    base_ref = oracle.forward(o["x"], o["W"], o["A"], np.zeros_like(o["B"]), 0.0)
    y0 = qn.linear_fwd(q, g["x"], g["A"], torch.zeros_like(g["B"]), L.alpha)
    yz = qn.linear_fwd(q, g["x"], g["A"], g["B"], 0.0)
    torch.cuda.synchronize()
    assert torch.equal(y0, yz)  # B = 0 and alpha = 0 both give the base output
    assert_close(to_np(y0), base_ref, "bf16", "base")
    # fp32 outputs of the LoRA delta scale with alpha (f32 compute keeps it exact-ish).
    Lf = inputs.random_layer(128, 128, 256, 8, seed=5, cd="f32", with_dy=False)
    gf = to_gpu(Lf)
    qf = gpu_q(Lf, gf)
    yb = qn.linear_fwd(qf, gf["x"], gf["A"], gf["B"], 0.0)
    y1 = qn.linear_fwd(qf, gf["x"], gf["A"], gf["B"], 8.0)
    y2 = qn.linear_fwd(qf, gf["x"], gf["A"], gf["B"], 16.0)
    torch.cuda.synchronize()
    d1, d2 = (y1 - yb).double().cpu().numpy(), (y2 - yb).double().cpu().numpy()
    assert oracle.rel_l2(d2, 2 * d1) < 1e-4


def test_forward_rslora():
    L = inputs.random_layer(130, 64, 128, 16, seed=6, with_dy=False)
    say("fwd rslora")
    g = to_gpu(L)
    y = qn.linear_fwd(gpu_q(L, g), g["x"], g["A"], g["B"], L.alpha, rslora=True)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    ref = oracle.forward(o["x"], o["W"], o["A"], o["B"], L.alpha / np.sqrt(L.r))
    assert_close(to_np(y), ref, "bf16", "rslora")


# ----------------------------------------------------------------------------- backward
def run_bwd(L, g, q, **kw):
    out = qn.linear_bwd(q, g["x"], g["dY"], g["A"], g["B"], L.alpha, **kw)
    torch.cuda.synchronize()
    return out


def test_backward_tiny():
    L = inputs.tiny()
    say("bwd tiny")
    g = to_gpu(L)
    dx, da, db = run_bwd(L, g, gpu_q(L, g))
    o = oracle_layer(L)
    rdx, rda, rdb = oracle.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"])
    assert_close(to_np(dx), rdx, "bf16", "tiny dX")
    assert_close(to_np(da), rda, "bf16", "tiny dA")
    assert_close(to_np(db), rdb, "bf16", "tiny dB")


@pytest.mark.parametrize("cd,path", PATHS)
@pytest.mark.parametrize("M,N,K,r", [(300, 200, 320, 24), (70, 130, 128, 5), (256, 64, 192, 64),
                                     (130, 256, 384, 16)])
def test_backward_ragged(cd, path, M, N, K, r):
    L = inputs.random_layer(M, N, K, r, seed=M * 7 + r, cd=cd)
    say("bwd ragged", cd, path, M, N, K, r)
    g = to_gpu(L)
    dx, da, db = run_bwd(L, g, gpu_q(L, g), path=path)
    o = oracle_layer(L)
    rdx, rda, rdb = oracle.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"])
    assert_close(to_np(dx), rdx, cd, "dX")
    assert_close(to_np(da), rda, cd, "dA")
    assert_close(to_np(db), rdb, cd, "dB")


@pytest.mark.parametrize("cd", ["bf16", "f16"])
def test_backward_four_tile_transposed_dequantize_partial_slab(cd):
    """dX on the dequantize path with W~^T from the four-tile transposed dequantize
    (4096 x 4160: 64 row slabs x 17 column slabs of 256, the last a quarter full)."""
    L = inputs.random_layer(130, 4096, 4160, 16, seed=41, cd=cd)
    say("bwd multi-tile dequant^T partial slab", cd)
    g = to_gpu(L)
    dx, da, db = run_bwd(L, g, gpu_q(L, g), path="dequant")
    o = oracle_layer(L)
    rdx, rda, rdb = oracle.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"])
    assert_close(to_np(dx), rdx, cd, "dX")
    assert_close(to_np(da), rda, cd, "dA")
    assert_close(to_np(db), rdb, cd, "dB")


def test_backward_saved_t_matches_recompute():
    L = inputs.random_layer(200, 192, 256, 16, seed=9)
    say("bwd saved T0")
    g = to_gpu(L)
    q = gpu_q(L, g)
    _, t0 = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, save_t=True)
    a = run_bwd(L, g, q, t_saved=t0)
    b = run_bwd(L, g, q)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    dx, da, db = run_bwd(L, g, q, need_dx=False)
    assert dx is None and torch.equal(da, a[1]) and torch.equal(db, a[2])


# ----------------------------------------------------------------------------- W~ bits, both paths
@pytest.mark.parametrize("cd", ["bf16", "f16"])
@pytest.mark.parametrize("path", ["fused", "dequant"])
def test_one_hot_reproduces_dequantized_weight_exactly(cd, path):
    """With one-hot activations and B = 0 every output is one product 1 * W~[n, k]
    (plus exact zeros), so y = W~^T and dX = W~ bit for bit: both paths use the
    dequantized weight that qlora_nf4_dequantize writes (W~^T for dX too)."""
    N, K, r = 256, 384, 16
    L = inputs.random_layer(K, N, K, r, seed=31, cd=cd, block_size=64, double_quant=True, with_dy=False)
    say("one-hot", cd, path)
    g = to_gpu(L)
    q = gpu_q(L, g)
    dt = g["x"].dtype
    w_cd = qn.dequantize(q, dt)                                   # [N, K]
    zero_b = torch.zeros_like(g["B"])
    y = qn.linear_fwd(q, torch.eye(K, dtype=dt, device="cuda"), g["A"], zero_b, L.alpha, path=path)
    dx, _, _ = qn.linear_bwd(q, g["x"][:N], torch.eye(N, dtype=dt, device="cuda"), g["A"], zero_b, L.alpha,
                             path=path)
    torch.cuda.synchronize()
    assert torch.equal(y, w_cd.t().contiguous())
    assert torch.equal(dx, w_cd)


# ----------------------------------------------------------------------------- variants
@pytest.mark.parametrize("path", ["fused", "dequant"])
@pytest.mark.parametrize("bs,groups,N,K", [(64, "global", 256, 512), (32, "global", 256, 512), (256, 3, 256, 512),
                                           (128, 64, 256, 512), (32, 5000, 512, 1024)])
def test_layer_block_sizes_and_global_scale(path, bs, groups, N, K):
    """Block sizes 32 / 64 / 128 / 256 and the double-quant group variants (one
    "global" group, a group larger than 4096 blocks, small odd groups) through the
    forward and the backward on both GEMM paths."""
    M, r = 200, 16
    g = N * K // bs if groups == "global" else groups
    L = inputs.random_layer(M, N, K, r, seed=bs + N, block_size=bs, double_quant=True, dq_group=g)
    say("variant", path, bs, groups, g)
    gg = to_gpu(L)
    q = gpu_q(L, gg)
    o = oracle_layer(L)
    y = run_fwd(L, gg, q, path=path)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"]), "bf16", "fwd")
    dx, da, db = run_bwd(L, gg, q, path=path)
    rdx, rda, rdb = oracle.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"])
    assert_close(to_np(dx), rdx, "bf16", "dX")
    assert_close(to_np(da), rda, "bf16", "dA")
    assert_close(to_np(db), rdb, "bf16", "dB")


@pytest.mark.parametrize("m", [1, 4, 16])
def test_decode_global_scale(m):
    L = inputs.random_layer(m, 4096, 4096, 16, seed=m + 40, alpha=32.0, double_quant=True,
                            dq_group=4096 * 4096 // 64, with_dy=False)
    say("decode global", m)
    g = to_gpu(L)
    y = run_fwd(L, g, gpu_q(L, g))
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"]), "bf16", "decode global")
