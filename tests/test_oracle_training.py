"""Pins of the training-step oracle (qlora-rs README, "Training (layer stack)":
stacked QuantizedLinear layers, MSE training_step, AdamW on the adapters).

Independent routes: closed forms of the MSE loss and of AdamW's first step,
PyTorch's own AdamW (float64, CPU) over several steps, and central finite
differences of the fp64 loss for the stack's gradients."""
import numpy as np
import pytest
import torch

import oracle
from oracle import training


def _r(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_mse_closed_form():
    t = _r((6, 5), 1)
    loss, dy = training.mse_loss_grad(t + 0.5, t)
    assert loss == pytest.approx(0.25, rel=1e-15)
    np.testing.assert_allclose(dy, np.full((6, 5), 2 * 0.5 / 30), rtol=1e-14)


def test_mse_gradient_finite_differences():
    y, t = _r((4, 7), 2), _r((4, 7), 3)
    _, dy = training.mse_loss_grad(y, t)
    h = 1e-6
    for idx in [(0, 0), (3, 6), (2, 3)]:
        yp, ym = y.copy(), y.copy()
        yp[idx] += h
        ym[idx] -= h
        fd = (training.mse_loss_grad(yp, t)[0] - training.mse_loss_grad(ym, t)[0]) / (2 * h)
        assert fd == pytest.approx(dy[idx], rel=1e-7)


def test_adamw_first_step_closed_form():
    th, g = _r(50, 4), _r(50, 5)
    lr, wd, eps = 1e-2, 0.1, 1e-8
    new, m, v = training.adamw(th, g, np.zeros(50), np.zeros(50), 1, lr, 0.9, 0.999, eps, wd)
    np.testing.assert_allclose(new, th * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-14)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-14)


def test_adamw_matches_torch_adamw_over_steps():
    th0 = _r((8, 9), 6)
    grads = [_r((8, 9), 10 + k) for k in range(4)]
    lr, b1, b2, eps, wd = 3e-3, 0.9, 0.95, 1e-6, 0.05
    p = torch.nn.Parameter(torch.tensor(th0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    th, m, v = th0, np.zeros_like(th0), np.zeros_like(th0)
    for k, g in enumerate(grads):
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        th, m, v = training.adamw(th, g, m, v, k + 1, lr, b1, b2, eps, wd)
        np.testing.assert_allclose(th, p.detach().numpy(), rtol=1e-12, atol=1e-14)


def _stack(seed, dims, r):
    """Random fp64 stack: dims = [K0, N0, N1, ...]."""
    layers = []
    for l in range(len(dims) - 1):
        K, N = dims[l], dims[l + 1]
        layers.append(dict(W=_r((N, K), seed + 10 * l, 0.3), a32=_r((r, K), seed + 10 * l + 1, 0.5),
                           b32=_r((N, r), seed + 10 * l + 2, 0.5), m_a=np.zeros((r, K)), v_a=np.zeros((r, K)),
                           m_b=np.zeros((N, r)), v_b=np.zeros((N, r))))
    return layers


def test_stack_gradients_match_finite_differences():
    dims, r, s = [8, 6, 5, 4], 2, 1.5
    layers = _stack(20, dims, r)
    x, t = _r((5, 8), 30), _r((5, 4), 31)
    kw = dict(step=1, lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0, rounding=False)
    out = training.stack_step(x, t, layers, s, "f32", **kw)

    def loss_with(l, key, idx, delta):
        L2 = [dict(L) for L in layers]
        arr = L2[l][key].copy()
        arr[idx] += delta
        L2[l][key] = arr
        return training.stack_step(x, t, L2, s, "f32", **kw)["loss"]

    h = 1e-6
    for l in range(3):
        for key, gi in (("a32", 0), ("b32", 1)):
            shape = layers[l][key].shape
            for idx in [(0, 0), (shape[0] - 1, shape[1] - 1), (shape[0] // 2, shape[1] // 2)]:
                fd = (loss_with(l, key, idx, h) - loss_with(l, key, idx, -h)) / (2 * h)
                assert fd == pytest.approx(out["grads"][l][gi][idx], rel=1e-6, abs=1e-12), (l, key, idx)


def test_stack_of_one_layer_is_the_layer_backward():
    """With one layer the step's gradients are the layer's (oracle.backward) at
    dY = RNE_cd(2 (y - t) / N), and its loss is the MSE of the rounded output."""
    layers = _stack(40, [64, 32], 4)
    for L in layers:
        L["W"] = oracle.round_to(L["W"].astype(np.float32), "bf16").astype(np.float64)
        L["a32"] = L["a32"].astype(np.float32).astype(np.float64)
        L["b32"] = L["b32"].astype(np.float32).astype(np.float64)
    x = oracle.round_to(_r((16, 64), 41).astype(np.float32), "bf16")
    t = oracle.round_to(_r((16, 32), 42).astype(np.float32), "bf16")
    out = training.stack_step(x, t, layers, 2.0, "bf16", 1, 1e-3, 0.9, 0.999, 1e-8, 0.0)
    A = oracle.round_to(layers[0]["a32"].astype(np.float32), "bf16")
    B = oracle.round_to(layers[0]["b32"].astype(np.float32), "bf16")
    y = oracle.round64_to(oracle.forward(x, layers[0]["W"].astype(np.float32), A, B, 2.0), "bf16")
    loss = np.mean((y.astype(np.float64) - t) ** 2)
    assert out["loss"] == pytest.approx(loss, rel=1e-12)
    dy = oracle.round64_to(2 * (y.astype(np.float64) - t) / y.size, "bf16")
    _, dA, dB = oracle.backward(x, layers[0]["W"].astype(np.float32), A, B, dy, 2.0)
    np.testing.assert_allclose(out["grads"][0][0], dA, rtol=1e-12)
    np.testing.assert_allclose(out["grads"][0][1], dB, rtol=1e-12)


def test_round64_is_one_rounding():
    # 1 + 2^-8 + 2^-30 lies just above the bf16 midpoint 1 + 2^-8: one rounding goes up,
    # a detour through binary32 (which drops the 2^-30) would tie and go down to even.
    v = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, -(1.0 + 2.0 ** -8 + 2.0 ** -30), 1.0 + 2.0 ** -8])
    got = oracle.round64_to(v, "bf16")
    assert list(got) == [1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7), 1.0]
    assert oracle.round64_to(np.array([1.0 + 2.0 ** -11 + 2.0 ** -40]), "f16")[0] == 1.0 + 2.0 ** -10


def test_steps_reduce_the_loss():
    layers = _stack(50, [16, 12, 8], 4)
    x, t = _r((32, 16), 51), _r((32, 8), 52)
    losses = []
    for step in range(1, 6):
        out = training.stack_step(x, t, layers, 1.0, "f32", step, 1e-2, 0.9, 0.999, 1e-8, 0.0, rounding=False)
        losses.append(out["loss"])
        for L, (a, ma, va, b, mb, vb) in zip(layers, out["new"]):
            L.update(a32=a, m_a=ma, v_a=va, b32=b, m_b=mb, v_b=vb)
    assert losses[-1] < losses[0]
