"""GPU parity of NF4 quantize / dequantize against the oracle: bit-exact packed
codes, block scales (fp32, or u8 + fp32 with double quantization) and
dequantized values in fp32 / bf16 / f16, through the C ABI on the device."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
import oracle
from bit_nf4_quantized_nibble_amd import inputs
from parity import say

pytestmark = pytest.mark.gpu


def gpu_quant(w_cpu, bs=64, dq=False, g=256):
    q = qn.quantize(w_cpu.cuda(), bs, dq, g)
    torch.cuda.synchronize()
    return q


def assert_same_quant(q, ref, what):
    assert np.array_equal(q.codes.cpu().numpy(), ref.packed), what + ": packed codes differ"
    if ref.double_quant:
        assert np.array_equal(q.absmax_q.cpu().numpy(), ref.absmax_q), what + ": u8 scales differ"
        assert np.array_equal(q.absmax_scale2.cpu().numpy().view(np.uint32),
                              ref.absmax_scale2.view(np.uint32)), what + ": second-level scales differ"
    else:
        assert np.array_equal(q.absmax.cpu().numpy().view(np.uint32),
                              ref.absmax.view(np.uint32)), what + ": absmax differs"


def check(w_cpu, bs=64, dq=False, g=256, what="", deq=("f32", "bf16", "f16")):
    say("quantize", what, tuple(w_cpu.shape), "bs", bs, "dq", dq, "g", g)
    ref = oracle.quantize(w_cpu.numpy(), bs, dq, g)
    q = gpu_quant(w_cpu, bs, dq, g)
    assert_same_quant(q, ref, what)
    if bs % 8 == 0:
        ref_f32 = oracle.dequantize(ref)
        for name in deq:
            say("dequantize", what, name)
            out = qn.dequantize(q, {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name])
            torch.cuda.synchronize()
            if name == "f32":
                assert np.array_equal(out.cpu().numpy().view(np.uint32), ref_f32.view(np.uint32)), what
            else:
                got = out.cpu().view(torch.int16).numpy().view(np.uint16)
                assert np.array_equal(got, oracle.to_bits(ref_f32, name)), what + " " + name
    return q, ref


def test_level_table_on_device():
    # Codes 0..15 with absmax 1 dequantize to the levels themselves.
    _, lv32 = oracle.levels()
    w = torch.from_numpy(np.repeat(lv32, 4).reshape(1, 64).copy())
    q, ref = check(w, 64, False, what="levels")
    assert np.array_equal(ref.codes, np.repeat(np.arange(16, dtype=np.uint8), 4))
    out = qn.dequantize(q, torch.float32).cpu().numpy().reshape(-1)
    assert np.array_equal(out, np.repeat(lv32, 4))


def test_tiny_weight():
    L = inputs.tiny()
    check(L.W, 64, False, what="tiny")
    check(L.W, 64, True, what="tiny-dq")


@pytest.mark.parametrize("dq", [False, True])
@pytest.mark.parametrize("outliers", [False, True])
def test_roundtrip_4096(dq, outliers):
    W = inputs.roundtrip_weight(0, outliers)
    q, ref = check(W, 64, dq, 256, what="roundtrip outliers=%s" % outliers)
    # The absmax element of each block is exactly +-1 after normalisation.
    codes = ref.codes.reshape(-1, 64)
    wb = W.numpy().reshape(-1, 64)
    idx = np.argmax(np.abs(wb), axis=1)
    assert np.all(np.isin(codes[np.arange(codes.shape[0]), idx], (0, 15)))


@pytest.mark.parametrize("bs,g", [(8, 1), (16, 7), (32, 256), (128, 100), (256, 4096), (512, 3)])
def test_block_sizes_and_groups(bs, g):
    g_ = torch.Generator().manual_seed(bs * 31 + g)
    W = torch.randn(300, 512, generator=g_) * 0.5
    check(W, bs, False, what="bs%d" % bs)
    check(W, bs, True, g, what="bs%d-g%d" % (bs, g))


@pytest.mark.parametrize("bs,g", [(64, 262144), (64, 5000), (32, 1 << 30), (256, 4097)])
def test_large_and_global_groups(bs, g):
    """Groups larger than 4096 blocks take the two-pass encoding; g >= nb (and any
    larger value) is the single "global" scale-of-scales."""
    W = inputs.roundtrip_weight(1, outliers=True)
    q, ref = check(W, bs, True, g, what="bs%d-g%d" % (bs, g), deq=("bf16",))
    nb = W.numel() // bs
    assert q.absmax_scale2.numel() == (nb + g - 1) // g


def test_global_group_ragged_span():
    g_ = torch.Generator().manual_seed(9)
    W = torch.randn(1000, 72, generator=g_)
    check(W, 8, True, 9000, what="ragged global bs8")     # 9000 blocks, one group
    check(W, 8, True, 4100, what="ragged bs8 g4100")      # a span crosses a group boundary


def test_ragged_spans():
    # 1125 blocks: the last 16384-element span and the last DQ group are partial.
    g_ = torch.Generator().manual_seed(5)
    W = torch.randn(1000, 72, generator=g_)
    check(W, 64, False, what="ragged")
    check(W, 64, True, 256, what="ragged-dq")
    check(torch.randn(32, 32, generator=g_), 64, True, 256, what="32x32")


def test_special_inputs():
    check(torch.zeros(64, 64), 64, False, what="zeros")
    check(torch.zeros(64, 64), 64, True, what="zeros-dq")
    check(torch.ones(128, 64), 64, False, what="ones")
    check(torch.ones(128, 64), 64, True, what="ones-dq")
    w = torch.zeros(16, 64)
    w[torch.arange(16), torch.arange(16) * 3] = torch.linspace(-5, 5, 16)
    check(w, 64, False, what="single-nonzero")


def test_values_at_every_threshold():
    # Blocks whose absmax is exactly 1 carry every midpoint between levels and its
    # binary32 neighbours; scaled copies move the same values through the division.
    _, lv32 = oracle.levels()
    mids = (lv32[:-1].astype(np.float64) + lv32[1:].astype(np.float64)) / 2
    vals = []
    for m in mids:
        f = np.float32(m)
        for k in range(-3, 4):
            v = f
            for _ in range(abs(k)):
                v = np.nextafter(v, np.float32(np.sign(k) * 2))
            vals.append(v)
    vals = np.array(vals, np.float32)
    per = 63
    nblk = (vals.size + per - 1) // per
    w = np.zeros((nblk, 64), np.float32)
    w[:, 0] = 1.0
    flat = np.zeros(nblk * per, np.float32)
    flat[: vals.size] = vals
    w[:, 1:] = flat.reshape(nblk, per)
    rng = np.random.default_rng(11)
    scales = np.concatenate([[1.0], 2.0 ** rng.integers(-20, 20, 7),
                             rng.uniform(0.1, 10, 8)]).astype(np.float32)
    W = np.concatenate([w * s for s in scales]).astype(np.float32)
    check(torch.from_numpy(W), 64, False, what="thresholds")
    check(torch.from_numpy(W), 64, True, 4, what="thresholds-dq")


def test_extreme_magnitudes():
    # Tiny (including subnormal) and huge blocks take the rescaled division path.
    g_ = torch.Generator().manual_seed(12)
    base = torch.randn(48, 64, generator=g_)
    mags = torch.tensor([1e-42, 1e-39, 1e-30, 1e-20, 1.0, 1e20, 1e30, 3e37] * 6).reshape(48, 1)
    W = (base * mags).float()
    check(W, 64, False, what="magnitudes", deq=("f32", "bf16"))
    check(W, 64, True, 8, what="magnitudes-dq", deq=("f32", "bf16"))


def test_f16_subnormal_outputs():
    g_ = torch.Generator().manual_seed(13)
    W = torch.randn(64, 64, generator=g_) * 1e-6
    check(W, 64, False, what="f16-subnormal")


def test_idempotence_on_device():
    W = inputs.roundtrip_weight(1, False, 1024, 1024).cuda()
    for dq in (False, True):
        q1 = qn.quantize(W, 64, dq)
        q2 = qn.quantize(qn.dequantize(q1, torch.float32), 64, dq)
        torch.cuda.synchronize()
        assert torch.equal(q1.codes, q2.codes)
        if dq:
            assert torch.equal(q1.absmax_q, q2.absmax_q) and torch.equal(q1.absmax_scale2, q2.absmax_scale2)
        else:
            assert torch.equal(q1.absmax, q2.absmax)
