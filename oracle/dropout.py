"""CPU oracle for the QLoRA layer with LoRA dropout (p > 0).

TEST INFRASTRUCTURE ONLY (same rules as the rest of this package).

Pages: rust_ai_core QLoraConfig docs, "Fields" (the LoRA configuration carries rank,
alpha and dropout); "LoRA and QLoRA, mathematically", "Tooling" (PEFT's LoraConfig
with its dropout field).  Reading (PEFT's LoRA dropout, the plainest one the pages
support): dropout acts on the input of the low-rank branch only, as inverted
dropout with a caller-drawn keep mask M (1 = kept) and rate p:

    x_d = x * M / (1 - p)
    y   = x W~^T + s (x_d A^T) B^T (+ bias)

and with W frozen:  dT = s dY B,  dX = dY W~ + (dT A) * M / (1 - p),
dA = dT^T x_d,  dB = s dY^T (x_d A^T).

Arithmetic is fp64 with plain matrix products; operands are the exact values the
kernels read (compute-dtype values as fp32 arrays, the mask as 0/1).
"""
from __future__ import annotations

import numpy as np


def _d(a):
    return np.asarray(a, np.float64)


def forward(x, W, A, B, s: float, mask, p: float, bias=None):
    x, W, A, B, M = _d(x), _d(W), _d(A), _d(B), _d(mask)
    xd = x * M / (1.0 - p)
    y = x @ W.T + s * (xd @ A.T) @ B.T
    return y if bias is None else y + _d(bias)[None, :]


def backward(x, W, A, B, dY, s: float, mask, p: float):
    x, W, A, B, dY, M = _d(x), _d(W), _d(A), _d(B), _d(dY), _d(mask)
    xd = x * M / (1.0 - p)
    dT = s * dY @ B
    dX = dY @ W + (dT @ A) * M / (1.0 - p)
    dA = dT.T @ xd
    dB = s * dY.T @ (xd @ A.T)
    return dX, dA, dB
