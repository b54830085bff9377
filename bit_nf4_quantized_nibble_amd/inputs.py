"""Seeded synthetic inputs for the QLoRA NF4 linear layer.

This module draws random tensors and nothing else: it holds none of the method's
arithmetic (no quantization, no level table, no GEMM), so both the HIP path and
the CPU oracle can be fed from it.  Every tensor comes from a CPU
``torch.Generator`` seeded per workload; values are drawn in fp32 as
``randn * sigma`` and, where the workload names a lower-precision dtype, cast
once to it (round-to-nearest-even) -- that cast is the input's own definition,
not a step of the method.

Shapes and distributions follow the workloads of the pages' problem statement:
  tiny       W 256x256 ~ N(0, 0.02^2), block 64, no double quant; x 8x256 ~ N(0,1);
             r = 8, alpha = 16, A ~ N(0, 1/r), B ~ N(0, 0.01^2), dY 8x256 ~ N(0,1)
  roundtrip  W 4096x4096 ~ N(0,1) (optionally 1% of entries x20 outliers)
  decode     W 4096x4096 ~ N(0, 0.02^2); x Mx4096, M in {1,4,16}; r = 16, alpha = 32
  prefill    the seven projections of one Llama-3-8B-shaped block, M = 4096 tokens,
             r = 64, alpha = 128 (trained weights are not needed: the layer's cost and
             numerics depend on shapes and value ranges, so N(0, 0.02^2) stands in)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# (name, N = out features, K = in features) of one Llama-3-8B-shaped block.
PREFILL_PROJECTIONS = [
    ("q_proj", 4096, 4096),
    ("k_proj", 1024, 4096),
    ("v_proj", 1024, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 14336, 4096),
    ("up_proj", 14336, 4096),
    ("down_proj", 4096, 14336),
]


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def randn(g: torch.Generator, shape, sigma: float = 1.0, dtype: str = "f32") -> torch.Tensor:
    t = torch.randn(*shape, generator=g, dtype=torch.float32) * sigma
    return t.to(_TORCH_DTYPES[dtype]).contiguous()


@dataclass
class LayerInputs:
    """One QLoRA linear layer's inputs (CPU tensors)."""
    name: str
    W: torch.Tensor                 # fp32 [N, K] frozen weight (to be quantized)
    x: torch.Tensor                 # cd   [M, K]
    A: torch.Tensor                 # cd   [r, K]
    B: torch.Tensor                 # cd   [N, r]
    r: int
    alpha: float
    block_size: int = 64
    double_quant: bool = True
    dq_group: int = 256
    cd: str = "bf16"
    dY: Optional[torch.Tensor] = None  # cd [M, N]
    bias: Optional[torch.Tensor] = None

    @property
    def M(self) -> int:
        return self.x.shape[0]

    @property
    def N(self) -> int:
        return self.W.shape[0]

    @property
    def K(self) -> int:
        return self.W.shape[1]


def tiny(seed: int = 0, cd: str = "bf16") -> LayerInputs:
    """Single QLoRA linear, tiny: drawn in the order W, x, A, B, dY."""
    g = _gen(seed)
    r = 8
    W = randn(g, (256, 256), 0.02)
    x = randn(g, (8, 256), 1.0, cd)
    A = randn(g, (r, 256), r ** -0.5, cd)
    B = randn(g, (256, r), 0.01, cd)
    dY = randn(g, (8, 256), 1.0, cd)
    return LayerInputs("tiny", W, x, A, B, r, 16.0, 64, False, 256, cd, dY)


def roundtrip_weight(seed: int = 0, outliers: bool = False, rows: int = 4096,
                     cols: int = 4096) -> torch.Tensor:
    """4096x4096 N(0,1) weight; with ``outliers`` exactly 1% of entries (chosen by a
    random permutation drawn after W) are multiplied by 20."""
    g = _gen(seed)
    W = randn(g, (rows, cols), 1.0)
    if outliers:
        n = W.numel()
        idx = torch.randperm(n, generator=g)[: n // 100]
        W.view(-1)[idx] *= 20.0
    return W


def decode(m: int, seed: int = 0, cd: str = "bf16") -> LayerInputs:
    """Decode-shaped GEMV: drawn in the order W, x, A, B."""
    g = _gen(seed)
    r, N, K = 16, 4096, 4096
    W = randn(g, (N, K), 0.02)
    x = randn(g, (m, K), 1.0, cd)
    A = randn(g, (r, K), r ** -0.5, cd)
    B = randn(g, (N, r), 0.01, cd)
    return LayerInputs("decode_m%d" % m, W, x, A, B, r, 32.0, 64, True, 256, cd)


def prefill(seed: int = 0, cd: str = "bf16", m: int = 4096, with_dy: bool = False,
            projections: Optional[List[str]] = None) -> List[LayerInputs]:
    """The seven projections of one block.  Draw order: x for K=4096 (shared by the
    six K=4096 projections), x for K=14336 (down_proj), then per projection in
    block order W, A, B and (if requested) dY."""
    g = _gen(seed)
    r = 64
    xs: Dict[int, torch.Tensor] = {4096: randn(g, (m, 4096), 1.0, cd),
                                   14336: randn(g, (m, 14336), 1.0, cd)}
    out = []
    for name, N, K in PREFILL_PROJECTIONS:
        W = randn(g, (N, K), 0.02)
        A = randn(g, (r, K), r ** -0.5, cd)
        B = randn(g, (N, r), 0.01, cd)
        dY = randn(g, (m, N), 1.0, cd) if with_dy else None
        if projections is None or name in projections:
            out.append(LayerInputs(name, W, xs[K], A, B, r, 128.0, 64, True, 256, cd, dY))
    return out


def random_layer(M: int, N: int, K: int, r: int, seed: int = 0, cd: str = "bf16",
                 alpha: Optional[float] = None, block_size: int = 64, double_quant: bool = True,
                 dq_group: int = 256, w_sigma: float = 0.02, with_bias: bool = False,
                 with_dy: bool = True) -> LayerInputs:
    """Arbitrary-shape layer for parity cases (ragged tails, other ranks / dtypes).
    Draw order: W, x, A, B, dY, bias."""
    g = _gen(seed)
    W = randn(g, (N, K), w_sigma)
    x = randn(g, (M, K), 1.0, cd)
    A = randn(g, (r, K), r ** -0.5, cd)
    B = randn(g, (N, r), 0.01, cd)
    dY = randn(g, (M, N), 1.0, cd) if with_dy else None
    bias = randn(g, (N,), 0.1, cd) if with_bias else None
    return LayerInputs("random_%dx%dx%d_r%d" % (M, N, K, r), W, x, A, B, r,
                       float(2 * r if alpha is None else alpha), block_size, double_quant,
                       dq_group, cd, dY, bias)


@dataclass
class StackInputs:
    """A stack of QLoRA layers for the training step (CPU tensors): layer l maps
    dims[l] features to dims[l + 1]."""
    Ws: List[torch.Tensor]          # fp32 [dims[l+1], dims[l]] frozen weights (to be quantized)
    As: List[torch.Tensor]          # fp32 master adapters [r, dims[l]]
    Bs: List[torch.Tensor]          # fp32 master adapters [dims[l+1], r]
    x: torch.Tensor                 # cd [M, dims[0]]
    target: torch.Tensor            # cd [M, dims[-1]]
    r: int
    alpha: float
    cd: str = "bf16"


def stack(dims: List[int], M: int, r: int = 16, seed: int = 0, cd: str = "bf16", alpha: Optional[float] = None,
          w_sigma: float = 0.02, t_sigma: float = 0.1) -> StackInputs:
    """Synthetic stack: W ~ N(0, w_sigma^2), A ~ N(0, 1/r), B ~ N(0, 0.01^2) per layer in
    order, then x ~ N(0, 1) and the regression target ~ N(0, t_sigma^2)."""
    g = _gen(seed)
    Ws, As, Bs = [], [], []
    for K, N in zip(dims[:-1], dims[1:]):
        Ws.append(randn(g, (N, K), w_sigma))
        As.append(randn(g, (r, K), r ** -0.5))
        Bs.append(randn(g, (N, r), 0.01))
    x = randn(g, (M, dims[0]), 1.0, cd)
    target = randn(g, (M, dims[-1]), t_sigma, cd)
    return StackInputs(Ws, As, Bs, x, target, r, float(2 * r if alpha is None else alpha), cd)


def dropout_mask(M: int, K: int, p: float, seed: int = 0) -> torch.Tensor:
    """Keep mask of LoRA dropout: uint8 [M, K], 1 with probability 1 - p (uniform draws)."""
    g = _gen(seed)
    return (torch.rand(M, K, generator=g) >= p).to(torch.uint8)
