"""GPU parity of the group calls (projections that read the same input, in one call)
against the oracle applied to each projection:

  * forward: the columns of projection i in y equal oracle.forward for it (bias
    included), and T0_i = x A_i^T;
  * backward: dX equals the fp64 sum of the projections' oracle dX, dA_i and dB_i
    equal the projection's own.

Cases: the tiled path (one dense GEMM over the concatenated weights, each rank slice
padded to 8 columns inside the concatenated rank operand, the block-diagonal lora_b,
a cut last round), the per-projection path (64 or fewer tokens, f32, rows that are
not a multiple of 64), and the q / k / v shapes of the Llama-3-8B block at 4096
tokens with outputs NaN-filled before the call and whole rows compared in every band
of 32 rows and at the edges of every 256-row tile."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
import oracle
from bit_nf4_quantized_nibble_amd import inputs
from parity import TORCH_DT, assert_close, say, to_np

pytestmark = pytest.mark.gpu


def make_group(M, K, shapes, cd, seed, bias):
    """Per projection (N_i, r_i): a layer from inputs.random_layer; the group reads the
    first layer's x.  Returns the layers, the shared x and the oracle operands."""
    Ls = [inputs.random_layer(M, N, K, r, seed=seed + 13 * i, cd=cd, with_bias=bias, with_dy=True)
          for i, (N, r) in enumerate(shapes)]
    x = Ls[0].x
    ops = []
    for L in Ls:
        qr = oracle.quantize(L.W.numpy(), L.block_size, L.double_quant, L.dq_group)
        ops.append(dict(W=oracle.weight_operand(qr, cd), A=oracle.operand(L.A, cd), B=oracle.operand(L.B, cd),
                        s=L.alpha / L.r, bias=oracle.operand(L.bias, cd) if bias else None,
                        dY=oracle.operand(L.dY, cd)))
    return Ls, x, ops


def run_group(Ls, x, cd, bias, rows=None):
    dt = TORCH_DT[cd]
    qs = [qn.quantize(L.W.cuda(), L.block_size, L.double_quant, L.dq_group) for L in Ls]
    xg = x.cuda()
    As = [L.A.cuda() for L in Ls]
    Bs = [L.B.cuda() for L in Ls]
    alphas = [L.alpha for L in Ls]
    bcat = torch.cat([L.bias for L in Ls]).cuda() if bias else None
    M, N = x.shape[0], sum(L.N for L in Ls)
    y = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    _, ts = qn.linear_fwd_group(qs, xg, As, Bs, alphas, bias=bcat, save_t=True, out=y)
    dy = torch.cat([L.dY for L in Ls], dim=1).cuda()
    dx, das, dbs = qn.linear_bwd_group(qs, xg, dy, As, Bs, alphas, t_saved=ts)
    torch.cuda.synchronize()
    return y, ts, dx, das, dbs


def check(Ls, x, ops, cd, y, ts, dx, das, dbs, rows=None):
    """rows: the token rows to compare for y and dX (all when None); dA, dB in full."""
    assert bool(torch.isfinite(y).all()), "unwritten or non-finite forward outputs"
    assert bool(torch.isfinite(dx).all()), "non-finite dX"
    xo = oracle.operand(x, cd)
    sel = np.arange(x.shape[0]) if rows is None else rows
    xs = np.ascontiguousarray(xo[sel])
    off = 0
    dx_ref = None
    for i, (L, o) in enumerate(zip(Ls, ops)):
        got = to_np(y[torch.from_numpy(sel).cuda(), off:off + L.N])
        assert_close(got, oracle.forward(xs, o["W"], o["A"], o["B"], o["s"], o["bias"]), cd, "y[%d]" % i)
        ref_t0 = xo.astype(np.float64) @ o["A"].astype(np.float64).T
        assert oracle.rel_l2(to_np(ts[i]).astype(np.float64), ref_t0) <= 1e-5, "T0[%d]" % i
        rdx, _, _ = oracle.backward(xs, o["W"], o["A"], o["B"], np.ascontiguousarray(o["dY"][sel]), o["s"],
                                    want=("dx",))
        dx_ref = rdx if dx_ref is None else dx_ref + rdx
        _, rda, rdb = oracle.backward(xo, o["W"], o["A"], o["B"], o["dY"], o["s"], want=("da", "db"))
        assert_close(to_np(das[i]), rda, cd, "dA[%d]" % i)
        assert_close(to_np(dbs[i]), rdb, cd, "dB[%d]" % i)
        off += L.N
    assert_close(to_np(dx[torch.from_numpy(sel).cuda()]), dx_ref, cd, "dX")


@pytest.mark.parametrize("M,K,shapes,cd,bias", [
    (300, 512, [(256, 16), (64, 8), (64, 8)], "bf16", True),    # q / k / v-like: tiled, ragged last row tile
    (260, 1024, [(512, 5), (128, 12), (192, 64)], "bf16", False),  # ranks padded to 8 inside the rank operand
    (520, 1024, [(1280, 8), (1280, 8)], "f16", True),           # gate / up-like: 30 tiles cut into 4 slices
])
def test_group_tiled(M, K, shapes, cd, bias):
    say("group tiled", M, K, shapes, cd, bias)
    Ls, x, ops = make_group(M, K, shapes, cd, seed=M + K, bias=bias)
    check(Ls, x, ops, cd, *run_group(Ls, x, cd, bias))


@pytest.mark.parametrize("M,K,shapes,cd,bias", [
    (48, 1024, [(256, 16), (64, 8)], "bf16", True),    # few tokens: the split-K GEMV per projection
    (1, 1024, [(512, 16), (128, 8), (128, 8)], "bf16", True),  # decode: each GEMV writes its columns of y
    (16, 2048, [(256, 16), (256, 16)], "f16", False),
    (1, 1024, [(512, 16), (256, 16), (256, 16)], "bf16", True),  # q / k / v-like
    (4, 1024, [(256, 8), (512, 8), (256, 8), (256, 8)], "bf16", False),  # four projections
    (7, 512, [(96, 8), (64, 4)], "f32", True),          # the VALU GEMV, in place as well
    (100, 256, [(200, 8), (72, 4)], "bf16", True),     # rows not a multiple of 64
    (90, 128, [(64, 8), (64, 8), (32, 4)], "f32", False),
])
def test_group_per_projection(M, K, shapes, cd, bias):
    say("group per projection", M, K, shapes, cd, bias)
    Ls, x, ops = make_group(M, K, shapes, cd, seed=3 * M + K, bias=bias)
    check(Ls, x, ops, cd, *run_group(Ls, x, cd, bias))


def test_group_llama_qkv_full_size():
    """q / k / v of the Llama-3-8B-shaped block at 4096 tokens, r 64: 384 tiles of
    256 x 256 for the forward (a whole round and a cut one), a 6144-long contraction
    for dX; rows sampled tile-complete."""
    Ls = inputs.prefill(cd="bf16", with_dy=True, projections=["q_proj", "k_proj", "v_proj"])
    say("group qkv full size")
    x = Ls[0].x
    ops = []
    for L in Ls:
        qr = oracle.quantize(L.W.numpy(), L.block_size, L.double_quant, L.dq_group)
        ops.append(dict(W=oracle.weight_operand(qr, "bf16"), A=oracle.operand(L.A, "bf16"),
                        B=oracle.operand(L.B, "bf16"), s=L.alpha / L.r, bias=None, dY=oracle.operand(L.dY, "bf16")))
    M = x.shape[0]
    rng = np.random.default_rng(5)
    bands = np.arange(0, M, 32)
    picks = bands + rng.integers(0, 32, bands.size)
    edges = np.concatenate([np.arange(0, M, 256), np.arange(255, M, 256)])
    rows = np.unique(np.concatenate([picks, edges]))
    y, ts, dx, das, dbs = run_group(Ls, x, "bf16", False)
    check(Ls, x, ops, "bf16", y, ts, dx, das, dbs, rows=rows)
    # the same call again gives the same bits (the cut round's slices are summed in order)
    y2, _, dx2, _, _ = run_group(Ls, x, "bf16", False)
    assert torch.equal(y, y2) and torch.equal(dx, dx2)


def test_group_llama_gate_up_forward_full_size():
    """gate / up of the Llama-3-8B-shaped block at 4096 tokens, r 64, as one forward
    call (the benchmark's MLP group): 1792 tiles of 256 x 256 over a 28672-wide
    output, seven whole rounds on the persistent form; the output NaN-filled before
    the call and whole rows compared in every band of 32 rows and at the edges of
    every 256-row tile."""
    Ls = inputs.prefill(cd="bf16", with_dy=False, projections=["gate_proj", "up_proj"])
    say("group gate/up forward full size")
    x = Ls[0].x
    ops = []
    for L in Ls:
        qr = oracle.quantize(L.W.numpy(), L.block_size, L.double_quant, L.dq_group)
        ops.append(dict(W=oracle.weight_operand(qr, "bf16"), A=oracle.operand(L.A, "bf16"),
                        B=oracle.operand(L.B, "bf16"), s=L.alpha / L.r))
    M, N = x.shape[0], sum(L.N for L in Ls)
    rng = np.random.default_rng(11)
    bands = np.arange(0, M, 32)
    rows = np.unique(np.concatenate([bands + rng.integers(0, 32, bands.size),
                                     np.arange(0, M, 256), np.arange(255, M, 256)]))
    qs = [qn.quantize(L.W.cuda(), L.block_size, L.double_quant, L.dq_group) for L in Ls]
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    _, ts = qn.linear_fwd_group(qs, x.cuda(), [L.A.cuda() for L in Ls], [L.B.cuda() for L in Ls],
                                [L.alpha for L in Ls], save_t=True, out=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "unwritten or non-finite forward outputs"
    xo = oracle.operand(x, "bf16")
    xs = np.ascontiguousarray(xo[rows])
    sel = torch.from_numpy(rows).cuda()
    off = 0
    for i, (L, o) in enumerate(zip(Ls, ops)):
        got = to_np(y[sel, off:off + L.N])
        assert_close(got, oracle.forward(xs, o["W"], o["A"], o["B"], o["s"], None), "bf16", "y[%d]" % i)
        ref_t0 = xo.astype(np.float64) @ o["A"].astype(np.float64).T
        assert oracle.rel_l2(to_np(ts[i]).astype(np.float64), ref_t0) <= 1e-5, "T0[%d]" % i
        off += L.N
