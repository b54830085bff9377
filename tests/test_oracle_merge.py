"""Pins of the oracle's merge, W_merged = W_hat + s B A rounded once to the output
dtype ("LoRA and QLoRA, mathematically", "The merge math", eq. 6.3.6).

Independent routes: exact rational arithmetic with a rounding written out from
the bf16 / f16 formats; B = 0 reduces to the rounding of the dequantized weight;
the merged weight reproduces the unmerged forward (eq. 6.3.6)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _round_exact(v: Fraction, bits: int, qmin: int) -> Fraction:
    """Nearest value with `bits` significant bits and quantum >= 2^qmin, ties to even."""
    if v == 0:
        return v
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # |v| in [2^e, 2^(e+1)): spacing 2^(e + 1 - bits)
    q = max(e + 1 - bits, qmin)
    scaled = abs(v) / Fraction(2) ** q
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    out = Fraction(n) * Fraction(2) ** q
    return out if v > 0 else -out


def _bits(values, dtype):
    a = np.array([float(v) for v in values], np.float64)
    if dtype == "bf16":
        return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return a.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("dtype,bits,qmin", [("bf16", 8, -133), ("f16", 11, -24)])
def test_merge_matches_exact_rational_rounding(dtype, bits, qmin):
    rng = np.random.default_rng(3)
    N, K, r = 5, 12, 3
    what = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = oracle.round_to(rng.standard_normal((r, K)).astype(np.float32), dtype)
    B = oracle.round_to((rng.standard_normal((N, r)) * 0.3).astype(np.float32), dtype)
    s = 2.0
    # a few values placed exactly on a rounding tie of the output format
    what[0, 0] = np.float32(1.0 + 2.0 ** -(bits))  # halfway between two 8/11-bit values
    A[:, 0] = 0
    got = oracle.merge(what, A, B, s, dtype)
    ref = []
    for n in range(N):
        for k in range(K):
            v = Fraction(float(what[n, k])) + Fraction(s) * sum(
                Fraction(float(B[n, t])) * Fraction(float(A[t, k])) for t in range(r))
            ref.append(_round_exact(v, bits, qmin))
    assert np.array_equal(got.reshape(-1), _bits(ref, dtype))
    # the tie rounded to even (down to 1.0)
    assert float(oracle.from_bits(got[:1, :1], dtype)[0, 0]) == 1.0


def test_merge_f32_is_one_rounding_of_the_exact_sum():
    rng = np.random.default_rng(4)
    N, K, r = 4, 6, 5
    what = rng.standard_normal((N, K)).astype(np.float32)
    A = rng.standard_normal((r, K)).astype(np.float32)
    B = rng.standard_normal((N, r)).astype(np.float32)
    got = oracle.merge(what, A, B, 0.5, "f32")
    for n in range(N):
        for k in range(K):
            v = Fraction(float(what[n, k])) + Fraction(0.5) * sum(
                Fraction(float(B[n, t])) * Fraction(float(A[t, k])) for t in range(r))
            assert got[n, k] == np.float32(float(v))  # one rounding of the exact value


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_merge_with_zero_b_is_the_rounded_dequantized_weight(dtype):
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((64, 128)) * 0.02).astype(np.float32)
    q = oracle.quantize(W, 64, True, 256)
    what = oracle.dequantize(q)
    A = oracle.round_to(rng.standard_normal((8, 128)).astype(np.float32), dtype)
    B = np.zeros((64, 8), np.float32)
    assert np.array_equal(oracle.merge(what, A, B, 2.0, dtype), oracle.to_bits(what, dtype))


def test_merged_weight_reproduces_the_forward_eq_6_3_6():
    rng = np.random.default_rng(6)
    M, N, K, r = 7, 48, 64, 4
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    what = oracle.dequantize(oracle.quantize(W, 64, False))
    x = rng.standard_normal((M, K)).astype(np.float32)
    A = rng.standard_normal((r, K)).astype(np.float32)
    B = (rng.standard_normal((N, r)) * 0.1).astype(np.float32)
    s = 4.0
    merged = oracle.merge(what, A, B, s, "f32").astype(np.float64)
    via_merge = torch.from_numpy(x.astype(np.float64)) @ torch.from_numpy(merged).T
    unmerged = oracle.forward(x, what, A, B, s)
    np.testing.assert_allclose(via_merge.numpy(), unmerged, rtol=1e-6, atol=1e-6)
