"""Pins for the oracle's NF4 quantize / dequantize (CPU only).

Each test checks the oracle against something other than itself: the level table
printed on the qlora-rs README ("NF4 Quantization"), scipy's normal quantile and
CDF, brute-force nearest-level search, exact rational arithmetic (fractions), numpy
float32 / float16 arithmetic, and the special cases the pages' export tests
quantize (all zeros, all ones, a 32x32 tensor with block 64).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import ndtr, ndtri

import oracle

DELTA = 0.5 * (1 - 1 / 30) + 0.5 * (1 - 1 / 32)


def _printed(golden_dir):
    vals = []
    with open(os.path.join(golden_dir, "nf4_levels_printed.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(float(line))
    return np.array(vals)


# ----------------------------------------------------------------------------- levels
def test_levels_match_printed_table(golden_dir):
    printed = _printed(golden_dir)
    lv64, lv32 = oracle.levels()
    assert printed.shape == (16,)
    assert np.all(np.abs(lv64 - printed) <= 5e-4 + 1e-12)
    assert np.all(np.abs(lv32.astype(np.float64) - printed) <= 5e-4 + 1e-7)
    assert np.array_equal(np.round(lv64, 3), printed)


def test_levels_structure():
    lv64, lv32 = oracle.levels()
    assert lv32[0] == -1.0 and lv32[7] == 0.0 and lv32[15] == 1.0
    assert np.all(np.diff(lv32) > 0)
    assert (lv32 < 0).sum() == 7 and (lv32 > 0).sum() == 8
    assert np.array_equal(lv32, lv64.astype(np.float32))


def test_levels_against_scipy_quantile():
    top = ndtri(DELTA)
    pos = [ndtri(DELTA - j * (DELTA - 0.5) / 8) for j in range(8)]
    neg = [-ndtri(DELTA - j * (DELTA - 0.5) / 7) for j in range(7)]
    ref = np.sort(np.array(pos + neg + [0.0])) / top
    lv64, lv32 = oracle.levels()
    assert np.max(np.abs(lv64 - ref)) < 1e-13
    assert np.array_equal(lv32, ref.astype(np.float32))


def test_levels_are_equal_probability_quantiles():
    # Forward direction: the normal CDF of each un-normalised level is evenly spaced
    # between 1/2 and the offset (8 steps above zero, 7 below).
    lv64, _ = oracle.levels()
    top = ndtri(DELTA)
    p_pos = ndtr(lv64[8:] * top)
    p_neg = ndtr(-lv64[:7] * top)
    assert np.allclose(p_pos, 0.5 + (DELTA - 0.5) * np.arange(1, 9) / 8, atol=1e-13, rtol=0)
    assert np.allclose(p_neg[::-1], 0.5 + (DELTA - 0.5) * np.arange(1, 8) / 7, atol=1e-13, rtol=0)


# ----------------------------------------------------------------------------- codes
def _brute_codes(x):
    """argmin_j |x - L_j| in fp64 (exact for fp32 x, L), ties to the lower index."""
    _, lv32 = oracle.levels()
    d = np.abs(x.astype(np.float64)[:, None] - lv32.astype(np.float64)[None, :])
    return np.argmin(d, axis=1).astype(np.uint8)


def _codes_of_values(x, bs=64):
    """Quantize values x in [-1,1] through blocks whose absmax is exactly 1, so that
    the normalised value is x itself."""
    x = np.asarray(x, np.float32)
    per = bs - 1
    nblk = (x.size + per - 1) // per
    w = np.zeros((nblk, bs), np.float32)
    w[:, 0] = 1.0
    flat = np.zeros(nblk * per, np.float32)
    flat[: x.size] = x
    w[:, 1:] = flat.reshape(nblk, per)
    q = oracle.quantize(w, bs)
    return q.codes.reshape(nblk, bs)[:, 1:].reshape(-1)[: x.size]


def test_nearest_level_brute_force_random():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-1, 1, 200000).astype(np.float32),
                        rng.standard_normal(50000).astype(np.float32) * 0.05,
                        np.array([-1, 0, 1, -0.0], np.float32)])
    x = np.clip(x, -1, 1).astype(np.float32)
    assert np.array_equal(_codes_of_values(x), _brute_codes(x))


def test_nearest_level_ties_and_neighbours():
    _, lv32 = oracle.levels()
    mids = (lv32[:-1].astype(np.float64) + lv32[1:].astype(np.float64)) / 2
    vals = []
    exact_ties = 0
    for m in mids:
        f = np.float32(m)
        if float(f) == m:
            exact_ties += 1
        for v in (f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2)),
                  np.nextafter(np.nextafter(f, np.float32(2)), np.float32(2))):
            vals.append(v)
    assert exact_ties >= 1  # some midpoints are exact in fp32, so real ties occur
    x = np.array(vals, np.float32)
    got = _codes_of_values(x)
    assert np.array_equal(got, _brute_codes(x))
    # An exact tie goes to the lower code.
    for j, m in enumerate(mids):
        if float(np.float32(m)) == m:
            assert _codes_of_values(np.array([m], np.float32))[0] == j


def test_absmax_element_maps_to_plus_minus_one():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((64, 64)).astype(np.float32)
    q = oracle.quantize(w, 64)
    codes = q.codes.reshape(-1, 64)
    wb = w.reshape(-1, 64)
    idx = np.argmax(np.abs(wb), axis=1)
    pick = codes[np.arange(codes.shape[0]), idx]
    sign = np.sign(wb[np.arange(wb.shape[0]), idx])
    assert np.all(pick == np.where(sign > 0, 15, 0))
    deq = oracle.dequantize(q).reshape(-1, 64)
    assert np.array_equal(np.abs(deq[np.arange(deq.shape[0]), idx]), q.absmax)


# ----------------------------------------------------------------------------- special cases
@pytest.mark.parametrize("shape", [(64, 64), (32, 32)])
def test_all_zeros(shape):
    q = oracle.quantize(np.zeros(shape, np.float32), 64)
    assert np.all(q.codes == 7) and np.all(q.packed == 0x77)
    assert np.all(q.absmax == 0)
    assert np.all(oracle.dequantize(q) == 0)
    qd = oracle.quantize(np.zeros(shape, np.float32), 64, double_quant=True)
    assert np.all(qd.absmax_q == 0) and np.all(qd.absmax_scale2 == 0)
    assert np.all(oracle.dequantize(qd) == 0)


def test_all_ones():
    q = oracle.quantize(np.ones((128, 64), np.float32), 64)
    assert np.all(q.codes == 15) and np.all(q.packed == 0xFF)
    assert np.all(q.absmax == 1.0)
    assert np.all(oracle.dequantize(q) == 1.0)
    qd = oracle.quantize(np.ones((128, 64), np.float32), 64, double_quant=True)
    assert np.all(qd.absmax_q == 255)
    assert np.all(oracle.dequantize(qd) == np.float32(255) * np.float32(np.float32(1) / np.float32(255)))


def test_single_nonzero_per_block():
    w = np.zeros((16, 64), np.float32)
    rng = np.random.default_rng(3)
    pos = rng.integers(0, 64, 16)
    vals = rng.standard_normal(16).astype(np.float32) * 3
    w[np.arange(16), pos] = vals
    q = oracle.quantize(w, 64)
    codes = q.codes.reshape(16, 64)
    expect = np.full((16, 64), 7, np.uint8)
    expect[np.arange(16), pos] = np.where(vals > 0, 15, 0)
    assert np.array_equal(codes, expect)
    assert np.array_equal(q.absmax, np.abs(vals))
    assert np.array_equal(oracle.dequantize(q), w)


def test_blocks_run_over_flattened_tensor():
    # 32x32 with block 64: a block spans two rows.
    rng = np.random.default_rng(4)
    w = rng.standard_normal((32, 32)).astype(np.float32)
    q = oracle.quantize(w, 64)
    assert q.absmax.shape == (16,)
    assert np.array_equal(q.absmax, np.abs(w.reshape(16, 64)).max(axis=1))


def test_nibble_order_high_first():
    w = np.zeros(64, np.float32)
    w[0] = 1.0      # element 0 -> code 15, element 1 -> code 7
    w[3] = -1.0     # element 3 -> code 0 (low nibble of byte 1), element 2 -> 7
    q = oracle.quantize(w, 64)
    assert q.packed[0] == 0xF7 and q.packed[1] == 0x70
    assert np.all(q.packed[2:] == 0x77)


def test_refuses_ragged_and_nonfinite():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros(100, np.float32), 64)
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros(63, np.float32), 63)
    w = np.zeros(64, np.float32)
    w[5] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize(w, 64)


# ----------------------------------------------------------------------------- dequant / DQ
def _numpy_dequant(q):
    """Independent dequantization with numpy: unpack high nibble first, then
    fl32(L[c] * s) in numpy float32 arithmetic."""
    _, lv32 = oracle.levels()
    codes = np.empty(q.packed.size * 2, np.uint8)
    codes[0::2] = q.packed >> 4
    codes[1::2] = q.packed & 15
    nb = codes.size // q.block_size
    if q.double_quant:
        grp = np.arange(nb) // q.dq_group
        s = q.absmax_q.astype(np.float32) * q.absmax_scale2[grp]
    else:
        s = q.absmax
    return (lv32[codes].reshape(nb, q.block_size) * s[:, None].astype(np.float32)).astype(np.float32)


@pytest.mark.parametrize("dq", [False, True])
def test_dequant_matches_numpy_float32(dq):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((300, 128)) * 0.02).astype(np.float32)
    q = oracle.quantize(w, 64, double_quant=dq, dq_group=256)
    assert np.array_equal(oracle.dequantize(q).reshape(-1), _numpy_dequant(q).reshape(-1))
    assert np.array_equal(q.codes, np.stack([q.packed >> 4, q.packed & 15], 1).reshape(-1))


def test_double_quant_exact_rounding():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((600, 64)).astype(np.float32)
    w[::7] *= 20  # outlier rows widen the scale range
    g = 256
    q = oracle.quantize(w, 64, double_quant=True, dq_group=g)
    q0 = oracle.quantize(w, 64, double_quant=False)
    nb = q0.absmax.size
    ng = (nb + g - 1) // g
    assert q.absmax_scale2.shape == (ng,)  # last group is partial (600 % 256 != 0)
    assert np.array_equal(q.codes, q0.codes)  # codes use the fp32 absmax either way
    for G in range(ng):
        a = q0.absmax[G * g:(G + 1) * g]
        c = a.max()
        S = q.absmax_scale2[G]
        # S is the binary32 value nearest to c/255 (exact rational check).
        exact = Fraction(float(c)) / 255
        up = np.nextafter(S, np.float32(np.inf))
        dn = np.nextafter(S, np.float32(-np.inf))
        assert abs(Fraction(float(S)) - exact) <= abs(Fraction(float(up)) - exact)
        assert abs(Fraction(float(S)) - exact) <= abs(Fraction(float(dn)) - exact)
        for b, ab in enumerate(a):
            ratio = Fraction(float(ab)) / Fraction(float(S))
            qq = round(ratio)  # Python rounds Fractions half to even
            assert q.absmax_q[G * g + b] == min(max(qq, 0), 255)
        assert q.absmax_q[G * g + int(np.argmax(a))] == 255


def test_idempotence_with_and_without_dq():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((1024, 1024)).astype(np.float32)
    for dq in (False, True):
        q1 = oracle.quantize(w, 64, double_quant=dq)
        q2 = oracle.quantize(oracle.dequantize(q1), 64, double_quant=dq)
        assert np.array_equal(q1.packed, q2.packed)
        if dq:
            assert np.array_equal(q1.absmax_q, q2.absmax_q)
            assert np.array_equal(q1.absmax_scale2, q2.absmax_scale2)
        else:
            assert np.array_equal(q1.absmax, q2.absmax)


def test_roundtrip_error_is_plausible():
    # Not a target from the pages, a regression bound: NF4 on N(0,1) with block 64
    # reconstructs with about 9% relative L2 error.
    rng = np.random.default_rng(8)
    w = rng.standard_normal((512, 512)).astype(np.float32)
    e = oracle.rel_l2(oracle.dequantize(oracle.quantize(w, 64)), w)
    assert 0.08 < e < 0.10


# ----------------------------------------------------------------------------- dtype rounding
def _special_f32():
    rng = np.random.default_rng(9)
    v = [rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 6, 20000)]
    v.append(np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.99, 65520, 65536, 1e6, -1e6,
                       2 ** -14, 2 ** -24, 2 ** -25, 3 * 2 ** -26, 2 ** -26, 1e-30, 3.4e38,
                       1 + 2 ** -11, 1 + 3 * 2 ** -11, 1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32))
    # Exact ties for bf16 (bit 15 set, lower bits zero) and for f16 (halfway mantissas).
    u = rng.integers(0, 2 ** 31, 5000, dtype=np.uint64).astype(np.uint32)
    v.append(((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32))
    v.append(((u & np.uint32(0xC7FFE000)) | np.uint32(0x1000)).view(np.float32))
    with np.errstate(invalid="ignore", over="ignore"):
        x = np.concatenate(v).astype(np.float32)
    return x[~np.isnan(x)]


def test_bf16_rounding_matches_torch():
    x = _special_f32()
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.to_bits(x, "bf16"), ref)
    back = oracle.from_bits(ref, "bf16")
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16).copy()).view(torch.bfloat16).float().numpy())


def test_f16_rounding_matches_numpy():
    x = _special_f32()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.to_bits(x, "f16"), ref)
    assert np.array_equal(oracle.from_bits(ref, "f16"), ref.view(np.float16).astype(np.float32))
