"""GPU parity of the adapter merge, W_merged = RNE_cd(w_hat + s B A) ("LoRA and QLoRA,
mathematically", "The merge math", eq. 6.3.6), against the oracle's merge on the
same seeded inputs, through the C ABI.

Bar: w_hat is bit-exact on both sides; the kernel sums B A in fp32 and rounds
twice (fp32 fused multiply-add, then the output dtype) where the oracle sums in
fp64 and rounds once.  Each bf16 / f16 element g must satisfy
|g - ref| <= ulp + s gamma_r sum_t |B_nt A_tk|, the textbook bound of an r-term
fp32 sum (gamma_r = r u / (1 - r u), u = 2^-24) plus one unit in the last place
for the two roundings, and >= 99.9 % of them are bit-identical (a mismatch needs
the exact value within the sum error of a rounding boundary).  fp32 output:
rel-L2 <= 1e-6 (the fp32 sum error is far below the weight it is added to)."""
import ctypes

import numpy as np
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
import oracle
from bit_nf4_quantized_nibble_amd import inputs
from parity import say, to_np

pytestmark = pytest.mark.gpu


def _ordered(bits, dtype):
    """Map 16-bit float patterns to integers that count representable values in order."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _ulp(v, dtype):
    """Spacing of the dtype's representable values at |v| (bf16: 8 significant bits)."""
    a = np.abs(v)
    if dtype == "f16":
        return np.spacing(a.astype(np.float16)).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(np.maximum(e - 7, -133))


def assert_merge_close(got_t, ref, dtype, what, A, B, s):
    """ref: the oracle's merge (bits for bf16 / f16, values for fp32); A [r, K], B [N, r]
    the exact adapter values for the error bound of the fp32 rank sum."""
    if dtype == "f32":
        got = to_np(got_t).astype(np.float64)
        rel = oracle.rel_l2(got, ref.astype(np.float64))
        assert rel <= 1e-6, "%s: rel-L2 %.3e" % (what, rel)
        return
    got_bits = got_t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    g = oracle.from_bits(got_bits, dtype).astype(np.float64)
    rv = oracle.from_bits(ref, dtype).astype(np.float64)
    r = A.shape[0]
    u = 2.0 ** -24
    gamma = r * u / (1 - r * u)
    bound = abs(s) * gamma * (np.abs(B.astype(np.float64)) @ np.abs(A.astype(np.float64)))
    allowed = _ulp(np.maximum(np.abs(g), np.abs(rv)), dtype) + bound
    bad = np.abs(g - rv) > allowed
    assert not bad.any(), "%s: %d elements beyond the bound, first at %s: got %r ref %r allowed %r" % (
        what, int(bad.sum()), np.argwhere(bad)[0], g[bad][0], rv[bad][0], allowed[bad][0])
    d = np.abs(_ordered(got_bits, dtype) - _ordered(ref, dtype))
    exact = float(np.mean(d == 0)) if d.size else 1.0
    assert exact >= 0.999, "%s: only %.5f bit-identical" % (what, exact)


def _setup(rows, cols, r, seed, cd, bs, dq, alpha=None):
    L = inputs.random_layer(1, rows, cols, r, seed=seed, cd=cd, alpha=alpha, block_size=bs, double_quant=dq,
                            with_dy=False)
    q = qn.quantize(L.W.cuda(), L.block_size, L.double_quant, L.dq_group)
    oq = oracle.quantize(L.W.numpy(), L.block_size, L.double_quant, L.dq_group)
    return L, q, oracle.dequantize(oq)


@pytest.mark.parametrize("cd", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows,cols,r,bs,dq", [
    (300, 384, 64, 64, True),    # ragged rows, 3 column tiles
    (257, 136, 24, 8, False),    # ragged by one row / 8 columns, rank not a multiple of 16
    (130, 256, 136, 32, True),   # three rank slices (64, 64, 8)
    (64, 96, 3, 32, False),      # odd rank: generic kernel for every dtype
    (1, 64, 8, 64, True),        # a single row
])
def test_merge_ragged(cd, rows, cols, r, bs, dq):
    say("merge", cd, rows, cols, r, bs, dq)
    L, q, what = _setup(rows, cols, r, rows + r, cd, bs, dq)
    out = qn.merge(q, L.A.cuda(), L.B.cuda(), L.alpha)
    torch.cuda.synchronize()
    s = float(np.float32(L.alpha / r))
    A, B = oracle.operand(L.A, cd), oracle.operand(L.B, cd)
    ref = oracle.merge(what, A, B, s, cd)
    assert out.shape == (rows, cols) and out.dtype == L.A.dtype
    assert_merge_close(out, ref, cd, "merge %s %dx%d r%d" % (cd, rows, cols, r), A, B, s)


@pytest.mark.parametrize("cd", ["bf16", "f16"])
def test_merge_rslora_scale(cd):
    say("merge rslora", cd)
    L, q, what = _setup(128, 256, 16, 11, cd, 64, True, alpha=8.0)
    out = qn.merge(q, L.A.cuda(), L.B.cuda(), L.alpha, rslora=True)
    torch.cuda.synchronize()
    s = float(np.float32(8.0 / np.sqrt(16.0)))
    A, B = oracle.operand(L.A, cd), oracle.operand(L.B, cd)
    ref = oracle.merge(what, A, B, s, cd)
    assert_merge_close(out, ref, cd, "merge rslora", A, B, s)


def test_merge_zero_b_equals_dequantize():
    """B = 0: the merge is the dequantized weight, bit for bit (both kernels)."""
    say("merge B=0")
    for r in (64, 5):
        L, q, _ = _setup(192, 320, r, 3, "bf16", 64, True)
        out = qn.merge(q, L.A.cuda(), torch.zeros_like(L.B).cuda(), L.alpha)
        deq = qn.dequantize(q, torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), deq.view(torch.int16)), "r=%d" % r


def test_merged_weight_reproduces_the_layer_forward():
    """eq. (6.3.6): x W_merged^T equals the unmerged layer output up to the bf16
    rounding of the merged weight (within the layer's bf16 tolerance)."""
    say("merge vs forward")
    L = inputs.random_layer(64, 256, 512, 16, seed=5, with_dy=False)
    g = {k: getattr(L, k).cuda() for k in ("W", "x", "A", "B")}
    q = qn.quantize(g["W"], L.block_size, L.double_quant, L.dq_group)
    y = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha)
    wm = qn.merge(q, g["A"], g["B"], L.alpha)
    torch.cuda.synchronize()
    ym = to_np(g["x"]).astype(np.float64) @ to_np(wm).astype(np.float64).T
    yy = to_np(y).astype(np.float64)
    rel = oracle.rel_l2(yy, ym)
    assert rel <= 5e-3, rel


@pytest.mark.parametrize("name", [p[0] for p in inputs.PREFILL_PROJECTIONS])
def test_merge_full_size_sampled_rows(name):
    """The seven projections of the Llama-3-8B-shaped block at r = 64, in the launch
    configuration the benchmark times; one random row in every 64-row tile of the
    kernel (first and last rows included) compared element by element, and the whole
    output (NaN before the call) finite."""
    (L,) = inputs.prefill(m=1, projections=[name])
    say("merge full", name)
    q = qn.quantize(L.W.cuda(), L.block_size, L.double_quant, L.dq_group)
    out = torch.full((L.N, L.K), float("nan"), dtype=torch.bfloat16, device="cuda")
    qn.merge(q, L.A.cuda(), L.B.cuda(), L.alpha, out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "unwritten merge outputs"
    what = oracle.dequantize(oracle.quantize(L.W.numpy(), L.block_size, L.double_quant, L.dq_group))
    rng = np.random.default_rng(9)
    bands = np.arange(0, L.N, 64)
    rows = np.unique(np.concatenate([[0, L.N - 1], np.minimum(bands + rng.integers(0, 64, bands.size), L.N - 1)]))
    A = oracle.operand(L.A, "bf16")
    B = np.ascontiguousarray(oracle.operand(L.B, "bf16")[rows])
    s = L.alpha / L.r
    ref = oracle.merge(np.ascontiguousarray(what[rows]), A, B, s, "bf16")
    assert_merge_close(out[torch.from_numpy(rows).cuda()], ref, "bf16", "merge %s" % name, A, B, s)


def test_merge_rejects_bad_arguments():
    say("merge errors")
    L, q, _ = _setup(64, 128, 8, 1, "bf16", 64, False)
    A, B = L.A.cuda(), L.B.cuda()
    out = torch.empty(64, 128, dtype=torch.bfloat16, device="cuda")
    d = q.descriptor()
    with pytest.raises(qn.QloraError, match="INVALID_ARG"):  # a path flag means nothing here
        qn._lib.check(qn._lib.lib().qlora_merge(ctypes.byref(d), A.data_ptr(), B.data_ptr(), 8, 16.0, 2,
                                                qn._lib.QLORA_BF16, out.data_ptr(), None))
    with pytest.raises(qn.QloraError, match="INVALID_ARG"):
        qn.merge(q, A, B, float("nan"))


def test_merge_global_scale():
    say("merge global")
    nb = 300 * 512 // 64
    L2 = inputs.random_layer(1, 300, 512, 64, seed=8, cd="bf16", block_size=64, double_quant=True, dq_group=nb,
                             with_dy=False)
    q = qn.quantize(L2.W.cuda(), 64, True, nb)
    what = oracle.dequantize(oracle.quantize(L2.W.numpy(), 64, True, nb))
    out = qn.merge(q, L2.A.cuda(), L2.B.cuda(), L2.alpha)
    torch.cuda.synchronize()
    A, B = oracle.operand(L2.A, "bf16"), oracle.operand(L2.B, "bf16")
    ref = oracle.merge(what, A, B, L2.alpha / 64, "bf16")
    assert_merge_close(out, ref, "bf16", "merge global", A, B, L2.alpha / 64)
