"""CPU oracle for the multi-layer training step: a stack of QLoRA linear layers,
mean-squared-error loss, AdamW on the adapters (the frozen NF4 bases never move).

TEST INFRASTRUCTURE ONLY (same rules as the rest of this package).

Pages: qlora-rs README, "Training (layer stack)": QuantizedLinear layers stacked,
``training_step`` with an MSE loss, AdamW updating the LoRA adapters ("adapters do
update"); "Honest capability matrix": multi-layer training with MSE and AdamW.

Readings where the pages stop short (each listed in the design notes):
  * the stack is a plain composition h_{l+1} = layer_l(h_l), no activation between
    layers (none is named);
  * MSE = mean over every element of (y - target)^2, so dL/dy = 2 (y - target) / N;
  * AdamW is the decoupled-weight-decay form: m = b1 m + (1 - b1) g,
    v = b2 v + (1 - b2) g^2, theta = theta (1 - lr wd) - lr (m / (1 - b1^t)) /
    (sqrt(v / (1 - b2^t)) + eps), with t the 1-based step;
  * the adapters have fp32 master copies (what AdamW updates) and compute-dtype
    copies the layer reads; activations and the gradients passed between layers are
    stored in the compute dtype (``rounding=True``), as a bf16 step keeps them.
    ``rounding=False`` keeps everything in fp64 (for the finite-difference pins).

Arithmetic is fp64; the layer itself is ``oracle.forward`` / ``oracle.backward``.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

from . import backward, forward, round64_to


def mse_loss_grad(y, target):
    """(loss, dL/dy) of loss = mean((y - target)^2), in fp64."""
    d = np.asarray(y, np.float64) - np.asarray(target, np.float64)
    n = d.size
    return float(np.sum(d * d) / n), 2.0 * d / n


def adamw(theta, g, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float, wd: float):
    """One AdamW update in fp64; returns (theta', m', v')."""
    theta = np.asarray(theta, np.float64)
    g = np.asarray(g, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    theta = theta * (1.0 - lr * wd) - lr * mhat / (np.sqrt(vhat) + eps)
    return theta, m, v


def _rd(a, cd: str, rounding: bool):
    """Storage of a value in the compute dtype: one rounding of the fp64 value."""
    if not rounding:
        return np.asarray(a, np.float64)
    return round64_to(a, cd).astype(np.float64)


def _forward64(x, W, A, B, s):
    x, W, A, B = (np.asarray(t, np.float64) for t in (x, W, A, B))
    return x @ W.T + s * (x @ A.T) @ B.T


def _backward64(x, W, A, B, dY, s):
    x, W, A, B, dY = (np.asarray(t, np.float64) for t in (x, W, A, B, dY))
    dT = s * dY @ B
    return dY @ W + dT @ A, dT.T @ x, s * dY.T @ (x @ A.T)


def stack_step(x, target, layers: List[Dict], s: float, cd: str, step: int, lr: float, beta1: float,
               beta2: float, eps: float, wd: float, rounding: bool = True):
    """One training step of the stack.  layers[l]: W (W~ values), a32, b32 (fp32 master
    adapters), m_a, v_a, m_b, v_b (moments).  Returns dict(loss, grads=[(dA, dB)],
    new=[(a, m_a, v_a, b, m_b, v_b)], h=activations).

    With ``rounding`` the layer products go through ``oracle.forward`` /
    ``oracle.backward`` (the C implementation) on compute-dtype operands; without it
    everything is plain fp64 (finite-difference pins)."""
    As = [_rd(L["a32"], cd, rounding) for L in layers]
    Bs = [_rd(L["b32"], cd, rounding) for L in layers]
    Ws = [np.asarray(L["W"], np.float64) for L in layers]
    h = [np.asarray(x, np.float64)]
    for W, A, B in zip(Ws, As, Bs):
        y = forward(h[-1].astype(np.float32), W.astype(np.float32), A.astype(np.float32),
                    B.astype(np.float32), s) if rounding else _forward64(h[-1], W, A, B, s)
        h.append(_rd(y, cd, rounding))
    loss, dy = mse_loss_grad(h[-1], target)
    g = _rd(dy, cd, rounding)
    grads = [None] * len(layers)
    for l in range(len(layers) - 1, -1, -1):
        if rounding:
            dX, dA, dB = backward(h[l].astype(np.float32), Ws[l].astype(np.float32), As[l].astype(np.float32),
                                  Bs[l].astype(np.float32), g.astype(np.float32), s)
        else:
            dX, dA, dB = _backward64(h[l], Ws[l], As[l], Bs[l], g, s)
        grads[l] = (dA, dB)
        g = _rd(dX, cd, rounding)
    new = []
    for L, (dA, dB) in zip(layers, grads):
        a, ma, va = adamw(L["a32"], dA, L["m_a"], L["v_a"], step, lr, beta1, beta2, eps, wd)
        b, mb, vb = adamw(L["b32"], dB, L["m_b"], L["v_b"], step, lr, beta1, beta2, eps, wd)
        new.append((a, ma, va, b, mb, vb))
    return {"loss": loss, "grads": grads, "new": new, "h": h}
