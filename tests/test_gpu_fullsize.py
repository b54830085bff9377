"""Full-size GPU parity of the QLoRA layer on the seven projections of one
Llama-3-8B-shaped block at 4096 tokens, r 64, alpha 128, NF4 block 64 with double
quantization, in the launch configuration the benchmark times.

Coverage is tile-complete:
  * every output (y, dX) is filled with NaN before the call and must come back
    finite everywhere, so a tile that is skipped or written elsewhere fails;
  * whole output rows are compared with the fp64 oracle for one random row in
    every band of 32 rows plus both edge rows of every 256-row tile, so every
    32 x 32 block of every 256 x 256 tile (and of the cut-round slices) has
    compared elements;
  * dA [r, cols] and dB [rows, r] are compared in full.

Cases: forward in bf16 on the dequantize-then-GEMM and the fused path, forward in
f16 and f32 (the dtype sweep), backward (dX, dA, dB) in bf16 on both paths.  The
oracle quantizes W itself (its codes must equal the library's bit for bit); the
rows of y and dX depend only on the same rows of x and dY, so the oracle runs on
the selected rows alone."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
import oracle
from bit_nf4_quantized_nibble_amd import inputs
from parity import TORCH_DT, assert_close, say, to_np

pytestmark = pytest.mark.gpu

NAMES = [p[0] for p in inputs.PREFILL_PROJECTIONS]
FWD = [("bf16", "dequant"), ("bf16", "fused"), ("f16", "auto"), ("f32", "auto")]
BWD = [("bf16", "dequant"), ("bf16", "fused")]


class _Cache:
    """Inputs of one dtype and the oracle's quantization of one projection at a time
    (the full block holds about a gigabyte of fp32 weights)."""

    def __init__(self):
        self.layers = {}
        self.qref = {}

    def layer(self, cd, name):
        if cd not in self.layers:
            self.layers = {cd: {L.name: L for L in inputs.prefill(cd=cd, with_dy=True)}}
        return self.layers[cd][name]

    def oracle_q(self, name, L):
        if name not in self.qref:
            self.qref = {name: oracle.quantize(L.W.numpy(), L.block_size, L.double_quant, L.dq_group)}
        return self.qref[name]


_cache = _Cache()


def check_rows(M, seed):
    """One random row in every band of 32 rows, plus the first and last row of every
    256-row tile."""
    rng = np.random.default_rng(seed)
    bands = np.arange(0, M, 32)
    picks = bands + rng.integers(0, 32, bands.size)
    edges = np.concatenate([np.arange(0, M, 256), np.minimum(np.arange(255, M + 255, 256), M - 1)])
    return np.unique(np.concatenate([picks[picks < M], edges]))


def _setup(cd, name):
    L = _cache.layer(cd, name)
    qr = _cache.oracle_q(name, L)
    q = qn.quantize(L.W.cuda(), L.block_size, L.double_quant, L.dq_group)
    torch.cuda.synchronize()
    assert np.array_equal(q.codes.cpu().numpy(), qr.packed), "codes differ from the oracle"
    assert np.array_equal(q.absmax_q.cpu().numpy(), qr.absmax_q), "u8 scales differ from the oracle"
    assert np.array_equal(q.absmax_scale2.cpu().numpy(), qr.absmax_scale2), "second-level scales differ"
    W = oracle.weight_operand(qr, cd)
    ops = dict(W=W, A=oracle.operand(L.A, cd), B=oracle.operand(L.B, cd), s=L.alpha / L.r)
    return L, q, ops


@pytest.mark.parametrize("name,cd,path", [(n, c, p) for n in NAMES for c, p in FWD])
def test_forward_full_size_tile_complete(name, cd, path):
    L, q, o = _setup(cd, name)
    say("full fwd", name, cd, path, L.M, L.N, L.K)
    dt = TORCH_DT[cd]
    x, A, B = L.x.cuda(), L.A.cuda(), L.B.cuda()
    y = torch.full((L.M, L.N), float("nan"), dtype=dt, device="cuda")
    qn.linear_fwd(q, x, A, B, L.alpha, path=path, out=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "unwritten or non-finite outputs"
    rows = check_rows(L.M, seed=10 * NAMES.index(name) + len(cd))
    xo = np.ascontiguousarray(oracle.operand(L.x, cd)[rows])
    ref = oracle.forward(xo, o["W"], o["A"], o["B"], o["s"])
    got = to_np(y[torch.from_numpy(rows).cuda()])
    assert_close(got, ref, cd, "fwd %s %s %s (%d rows)" % (name, cd, path, rows.size))
    if name == "gate_proj":
        # cut last round: a second call on the same inputs gives the same bits
        y2 = qn.linear_fwd(q, x, A, B, L.alpha, path=path)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)


@pytest.mark.parametrize("name,cd,path", [(n, c, p) for n in NAMES for c, p in BWD])
def test_backward_full_size_tile_complete(name, cd, path):
    L, q, o = _setup(cd, name)
    say("full bwd", name, cd, path, L.M, L.N, L.K)
    dt = TORCH_DT[cd]
    x, A, B, dY = L.x.cuda(), L.A.cuda(), L.B.cuda(), L.dY.cuda()
    dx = torch.full((L.M, L.K), float("nan"), dtype=dt, device="cuda")
    da = torch.full((L.r, L.K), float("nan"), dtype=torch.float32, device="cuda")
    db = torch.full((L.N, L.r), float("nan"), dtype=torch.float32, device="cuda")
    qn.linear_bwd(q, x, dY, A, B, L.alpha, path=path, dx_out=dx, da_out=da, db_out=db)
    torch.cuda.synchronize()
    for nm, t in (("dX", dx), ("dA", da), ("dB", db)):
        assert bool(torch.isfinite(t).all()), "%s: unwritten or non-finite outputs" % nm
    xo, dYo = oracle.operand(L.x, cd), oracle.operand(L.dY, cd)
    rows = check_rows(L.M, seed=10 * NAMES.index(name) + 7)
    rdx, _, _ = oracle.backward(np.ascontiguousarray(xo[rows]), o["W"], o["A"], o["B"],
                                np.ascontiguousarray(dYo[rows]), o["s"], want=("dx",))
    assert_close(to_np(dx[torch.from_numpy(rows).cuda()]), rdx, cd, "dX %s %s" % (name, path))
    _, rda, rdb = oracle.backward(xo, o["W"], o["A"], o["B"], dYo, o["s"], want=("da", "db"))
    assert_close(to_np(da), rda, cd, "dA %s %s" % (name, path))
    assert_close(to_np(db), rdb, cd, "dB %s %s" % (name, path))
