"""GPU parity of the 256 x 256 GEMMs (dequantize-then-GEMM and fused NF4 decode)
when the tiles of an incomplete last round are cut into contraction slices (two,
four or eight per tile, whose fp32 partial sums a second launch adds in slice
order), against the fp64 oracle through the C ABI.

One round is one tile per compute unit.  A GEMM with T tiles on C units takes
floor(T / C) whole rounds; the R = T mod C tiles left over are cut into the
largest S in {2, 4} (in {2, 4, 8} when all rows fit one 256-row tile row) with
R * S <= C and at least 4 contraction stages of 64 per slice.  Small cases compare every element (ragged M and N, a bias, the low-rank
tail on the last slice); the full projection sizes whose tile counts leave an
incomplete round (gate / up forward, down dX: 16 x 56 tiles) are covered tile by
tile in test_gpu_fullsize.py.  Repeats on a workspace full of stale bytes and outputs filled with NaN
must give the same bits."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
from bit_nf4_quantized_nibble_amd import _lib
import oracle
from bit_nf4_quantized_nibble_amd import inputs
from parity import TORCH_DT, assert_close, oracle_layer, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


def expected_split(M, NB, K1):
    """(whole-tile workgroups, cut tiles, slices) the 256 x 256 GEMMs use on this GPU."""
    C = torch.cuda.get_device_properties(0).multi_processor_count
    T = -(-M // 256) * -(-NB // 256)
    F, R = divmod(T, C)
    if R == 0:
        return T, 0, 1
    cap = min(C // R, (K1 // 64) // 4)
    S = 1
    while S < (8 if M <= 256 else 4) and 2 * S <= cap:
        S *= 2
    return (T, 0, 1) if S == 1 else (F * C, R, S)


def gpu_q(L, g):
    return qn.quantize(g["W"], L.block_size, L.double_quant, L.dq_group)


@pytest.mark.parametrize("path", ["dequant", "fused"])
@pytest.mark.parametrize("cd", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K,r,bias,S", [
    (300, 260, 1024, 16, True, 4),   # 2 x 2 tiles, both ragged, 16 stages -> 4 slices of 4
    (520, 200, 512, 24, False, 2),   # 3 x 1 tiles, 8 stages -> 2 slices
    (257, 64, 1280, 5, True, 4),     # a one-row ragged tile row, odd rank, 20 stages -> 5 per slice
    (300, 1024, 2048, 8, True, 4),   # 2 x 4 tiles, 32 stages, two tile rows -> 4 slices of 8
    (200, 1024, 2048, 8, True, 8),   # 1 x 4 tiles, 32 stages, one tile row -> 8 slices of 4
    (256, 512, 4096, 16, False, 8),  # 1 x 2 tiles, 64 stages -> 8 slices of 8
])
def test_split_forward_every_element(path, cd, M, N, K, r, bias, S):
    assert expected_split(M, N, K)[2] == S
    L = inputs.random_layer(M, N, K, r, seed=M + N + K + r, cd=cd, with_bias=bias, with_dy=False)
    say("split fwd", path, cd, M, N, K, r, "S", S)
    g = to_gpu(L)
    y = qn.linear_fwd(gpu_q(L, g), g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], path=path)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    ref = oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"])
    assert_close(to_np(y), ref, cd, "split fwd %s %dx%dx%d" % (cd, M, N, K))


@pytest.mark.parametrize("path", ["dequant", "fused"])
@pytest.mark.parametrize("cd", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K,r,S", [
    (300, 1024, 320, 16, 4),  # dX [300, 320]: 2 x 2 tiles, contraction 1024 -> 4 slices
    (200, 512, 256, 8, 2),    # dX one tile, contraction 512 -> 2 slices
    (130, 2048, 512, 16, 8),  # dX [130, 512]: 1 x 2 tiles, contraction 2048 -> 8 slices
])
def test_split_backward_dx_every_element(path, cd, M, N, K, r, S):
    assert expected_split(M, K, N)[2] == S
    L = inputs.random_layer(M, N, K, r, seed=3 * M + N + r, cd=cd)
    say("split bwd", path, cd, M, N, K, r, "S", S)
    g = to_gpu(L)
    dx, da, db = qn.linear_bwd(gpu_q(L, g), g["x"], g["dY"], g["A"], g["B"], L.alpha, path=path)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    rdx, rda, rdb = oracle.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"])
    assert_close(to_np(dx), rdx, cd, "split dX")
    assert_close(to_np(da), rda, cd, "split dA")
    assert_close(to_np(db), rdb, cd, "split dB")


@pytest.mark.parametrize("path", ["dequant", "fused"])
def test_split_repeats_bit_identical_on_stale_workspace(path):
    """A workspace left full of 0xff bytes, or holding the partial sums of the
    previous call, gives the same bits, and every output element is written
    (outputs start as NaN)."""
    M, N, K, r = 300, 512, 1024, 16  # forward 2 x 2 tiles in 4 slices, dX 2 x 4 tiles in 2
    assert expected_split(M, N, K)[2] == 4 and expected_split(M, K, N)[2] == 2
    L = inputs.random_layer(M, N, K, r, seed=41, with_bias=True)
    say("split stale workspace", path)
    g = to_gpu(L)
    q = gpu_q(L, g)
    dt = TORCH_DT[L.cd]
    flags = _lib.QLORA_FLAG_DEQUANT_GEMM if path == "dequant" else _lib.QLORA_FLAG_FUSED
    wsf = torch.full((qn.workspace_bytes(_lib.QLORA_OP_FWD, M, N, K, r, dt, flags),), 255, dtype=torch.uint8,
                     device="cuda")
    wsb = torch.full((qn.workspace_bytes(_lib.QLORA_OP_BWD, M, N, K, r, dt, flags),), 255, dtype=torch.uint8,
                     device="cuda")
    ys, dxs = [], []
    for _ in range(3):
        y = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
        qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], path=path, workspace=wsf, out=y)
        dx = torch.full((M, K), float("nan"), dtype=dt, device="cuda")
        qn.linear_bwd(q, g["x"], g["dY"], g["A"], g["B"], L.alpha, path=path, workspace=wsb, dx_out=dx)
        torch.cuda.synchronize()
        ys.append(y.clone())
        dxs.append(dx.clone())
    for i in (1, 2):
        assert torch.equal(ys[i], ys[0]) and torch.equal(dxs[i], dxs[0])
    o = oracle_layer(L)
    assert_close(to_np(ys[0]), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"]), L.cd, "fwd")
    assert_close(to_np(dxs[0]), oracle.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"])[0], L.cd, "dX")


@pytest.mark.parametrize("path", ["dequant", "fused"])
def test_persistent_dense_more_items_than_cus(path):
    """More items (whole tiles + slices of the cut ones) than CUs: the dense kernel runs
    one persistent workgroup per CU that takes items b, b + C, ... and requests the
    next item's first stage before the current epilogue.  Ragged M (the second tile row
    has 8 rows), a cut last round, a bias; forward (2 x 150 tiles) and dX (2 x 150 tiles
    of [M, K]) compared element by element, outputs NaN-filled before the call."""
    C = torch.cuda.get_device_properties(0).multi_processor_count
    M, r = 264, 16
    Nf, Kf = 256 * (C // 2 + 22), 512        # forward: 2 x (C/2 + 22) tiles, contraction 8 stages
    F, R, S = expected_split(M, Nf, Kf)
    assert F + R * S > C and R > 0, (F, R, S)
    L = inputs.random_layer(M, Nf, Kf, r, seed=97, cd="bf16", with_bias=True, with_dy=False)
    say("persistent fwd", path, M, Nf, Kf, "items", F + R * S)
    g = to_gpu(L)
    q = gpu_q(L, g)
    y = torch.full((M, Nf), float("nan"), dtype=torch.bfloat16, device="cuda")
    qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], path=path, out=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "unwritten forward outputs"
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"]), "bf16", "persistent fwd")
    del y, g, q
    # dX [M, Kd]: 2 x (C / 2 + 22) tiles over a contraction of 512 W rows
    Nd, Kd = 512, 256 * (C // 2 + 22)
    F, R, S = expected_split(M, Kd, Nd)
    assert F + R * S > C and R > 0, (F, R, S)
    L = inputs.random_layer(M, Nd, Kd, r, seed=98, cd="bf16")
    say("persistent dX", path, M, Nd, Kd, "items", F + R * S)
    g = to_gpu(L)
    q = gpu_q(L, g)
    dx = torch.full((M, Kd), float("nan"), dtype=torch.bfloat16, device="cuda")
    qn.linear_bwd(q, g["x"], g["dY"], g["A"], g["B"], L.alpha, path=path, dx_out=dx)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dx).all()), "unwritten dX outputs"
    o = oracle_layer(L)
    assert_close(to_np(dx), oracle.backward(o["x"], o["W"], o["A"], o["B"], o["dY"], o["s"], want=("dx",))[0],
                 "bf16", "persistent dX")
