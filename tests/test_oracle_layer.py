"""Pins for the oracle's QLoRA forward / backward (CPU only).

The oracle's fp64 loops are checked against torch's fp64 matmul and autograd
(library routines), against the special cases the method fixes (B = 0 gives the
base output; the LoRA delta is linear in alpha; scale = alpha / r), and against the
merge identity of "LoRA and QLoRA, mathematically" eq. (6.3.6):
x (W + (alpha/r) B A)^T equals the adapter-on-base output.  Shapes are non-square
with distinct M, N, K, r so a transposed operand or swapped index cannot pass.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_nf4_quantized_nibble_amd import inputs


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _torch64(a):
    return torch.from_numpy(np.asarray(a, np.float64))


SHAPES = [(5, 7, 192, 3), (9, 130, 64, 16), (1, 33, 128, 1)]


@pytest.mark.parametrize("M,N,K,r", SHAPES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_forward_matches_torch_fp64(M, N, K, r, with_bias):
    x, W, A, B = _rand((M, K), 1), _rand((N, K), 2, 0.02), _rand((r, K), 3), _rand((N, r), 4, 0.1)
    bias = _rand((N,), 5) if with_bias else None
    s = 2.5
    y = oracle.forward(x, W, A, B, s, bias)
    ref = _torch64(x) @ _torch64(W).T + s * (_torch64(x) @ _torch64(A).T) @ _torch64(B).T
    if bias is not None:
        ref = ref + _torch64(bias)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_b_zero_gives_base_output_bitwise():
    M, N, K, r = 6, 40, 128, 4
    x, W, A = _rand((M, K), 1), _rand((N, K), 2, 0.02), _rand((r, K), 3)
    y0 = oracle.forward(x, W, A, np.zeros((N, r), np.float32), 2.0)
    ya = oracle.forward(x, W, A, _rand((N, r), 4), 0.0)
    base = oracle.forward(x, W, np.zeros((r, K), np.float32), np.zeros((N, r), np.float32), 2.0)
    assert np.array_equal(y0, base) and np.array_equal(ya, base)
    ref = (_torch64(x) @ _torch64(W).T).numpy()
    np.testing.assert_allclose(base, ref, rtol=1e-13, atol=1e-13)


def test_lora_delta_linear_in_alpha():
    M, N, K, r = 4, 24, 64, 8
    x, W, A, B = _rand((M, K), 1), _rand((N, K), 2, 0.02), _rand((r, K), 3), _rand((N, r), 4)
    base = oracle.forward(x, W, A, B, 0.0)
    d1 = oracle.forward(x, W, A, B, 16.0 / r) - base
    d2 = oracle.forward(x, W, A, B, 32.0 / r) - base
    np.testing.assert_allclose(d2, 2 * d1, rtol=1e-12, atol=1e-14)
    assert np.abs(d1).max() > 0


def test_merge_identity_eq_6_3_6():
    M, N, K, r = 7, 48, 256, 8
    x, W, A, B = _rand((M, K), 1), _rand((N, K), 2, 0.02), _rand((r, K), 3), _rand((N, r), 4, 0.05)
    s = 16.0 / r
    merged = _torch64(W) + s * _torch64(B) @ _torch64(A)
    ref = (_torch64(x) @ merged.T).numpy()
    np.testing.assert_allclose(oracle.forward(x, W, A, B, s), ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("M,N,K,r", SHAPES)
def test_backward_matches_torch_autograd(M, N, K, r):
    x, W, A, B = _rand((M, K), 1), _rand((N, K), 2, 0.02), _rand((r, K), 3), _rand((N, r), 4, 0.1)
    dY = _rand((M, N), 5)
    s = 1.75
    dX, dA, dB = oracle.backward(x, W, A, B, dY, s)
    xt = _torch64(x).requires_grad_(True)
    At = _torch64(A).requires_grad_(True)
    Bt = _torch64(B).requires_grad_(True)
    Wt = _torch64(W)  # frozen
    y = xt @ Wt.T + s * (xt @ At.T) @ Bt.T
    y.backward(_torch64(dY))
    np.testing.assert_allclose(dX, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, At.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dB, Bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_tiny_workload_end_to_end_against_autograd():
    """The tiny workload through the whole oracle: quantize -> dequantize -> bf16
    operands -> forward / backward, checked against torch fp64 autograd of the same
    operands."""
    L = inputs.tiny()
    q = oracle.quantize(L.W.numpy(), L.block_size, L.double_quant)
    Wc = oracle.weight_operand(q, "bf16")
    x, A, B, dY = (oracle.operand(t, "bf16") for t in (L.x, L.A, L.B, L.dY))
    s = L.alpha / L.r
    assert s == 2.0
    y = oracle.forward(x, Wc, A, B, s)
    dX, dA, dB = oracle.backward(x, Wc, A, B, dY, s)
    xt = _torch64(x).requires_grad_(True)
    At = _torch64(A).requires_grad_(True)
    Bt = _torch64(B).requires_grad_(True)
    yt = xt @ _torch64(Wc).T + s * (xt @ At.T) @ Bt.T
    yt.backward(_torch64(dY))
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    for got, ref in ((dX, xt.grad), (dA, At.grad), (dB, Bt.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_samplers_agree_with_full_computation():
    M, N, K, r = 12, 40, 192, 5
    x, W, A, B = _rand((M, K), 1), _rand((N, K), 2, 0.02), _rand((r, K), 3), _rand((N, r), 4, 0.1)
    dY = _rand((M, N), 5)
    bias = _rand((N,), 6)
    s = 3.0
    y = oracle.forward(x, W, A, B, s, bias)
    dX, dA, dB = oracle.backward(x, W, A, B, dY, s)
    rng = np.random.default_rng(0)
    ii, jj = rng.integers(0, M, 50), rng.integers(0, N, 50)
    np.testing.assert_allclose(oracle.forward_at(x, W, A, B, s, ii, jj, bias), y[ii, jj], rtol=1e-13, atol=1e-13)
    kk = rng.integers(0, K, 50)
    np.testing.assert_allclose(oracle.backward_dx_at(dY, W, A, B, s, ii, kk), dX[ii, kk], rtol=1e-13, atol=1e-13)
    tt = rng.integers(0, r, 50)
    np.testing.assert_allclose(oracle.backward_da_at(x, dY, B, s, tt, kk), dA[tt, kk], rtol=1e-13, atol=1e-13)
    nn = rng.integers(0, N, 50)
    np.testing.assert_allclose(oracle.backward_db_at(x, A, dY, s, nn, tt), dB[nn, tt], rtol=1e-13, atol=1e-13)


def test_dtype_operands_are_exact_roundings():
    L = inputs.random_layer(3, 16, 64, 2, cd="f16")
    got = oracle.operand(L.x, "f16")
    assert np.array_equal(got, L.x.float().numpy())
    ref = oracle.round_to(L.x.float().numpy(), "f16")
    assert np.array_equal(got, ref)
