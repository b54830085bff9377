"""GPU parity of the cached-dequant forward (the caller dequantizes the frozen
weight once and keeps W~ in the compute dtype; each call runs the rank product and
the dense 256 x 256 GEMM on it) against the fp64 oracle through the C ABI, and its
bit-identity with the per-call dequantize-then-GEMM path."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
import oracle
from bit_nf4_quantized_nibble_amd import inputs
from parity import assert_close, oracle_layer, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


def gpu_q(L, g):
    return qn.quantize(g["W"], L.block_size, L.double_quant, L.dq_group)


@pytest.mark.parametrize("cd,M,N,K,r,bias", [
    ("bf16", 300, 260, 512, 16, True),   # ragged M and N, bias
    ("f16", 17, 128, 192, 5, False),     # odd rank: the four-wave kernel's tail
    ("bf16", 4, 64, 256, 8, True),       # a decode-sized call through the dense GEMM
    ("bf16", 520, 200, 1024, 64, False),  # cut last round (3 x 1 tiles, 4 slices)
])
def test_cached_forward_matches_oracle(cd, M, N, K, r, bias):
    L = inputs.random_layer(M, N, K, r, seed=5 * M + N + r, cd=cd, with_bias=bias, with_dy=False)
    say("fwd cached", cd, M, N, K, r, bias)
    g = to_gpu(L)
    q = gpu_q(L, g)
    w_cd = qn.dequantize(q, g["x"].dtype)
    y, t0 = qn.linear_fwd_cached(w_cd, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], save_t=True)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"]), cd, "cached fwd")
    ref_t0 = np.asarray(o["x"], np.float64) @ np.asarray(o["A"], np.float64).T
    assert oracle.rel_l2(to_np(t0).astype(np.float64), ref_t0) <= 1e-5, "cached T0"


@pytest.mark.parametrize("rslora", [False, True])
def test_cached_forward_equals_dequant_path_bitwise(rslora):
    """Same W~ bits, same kernels: the cached call and the per-call dequantize-then-GEMM
    path give identical y, on a repeat as well."""
    L = inputs.random_layer(700, 640, 1280, 24, seed=77, with_bias=True, with_dy=False)
    say("fwd cached == dequant", rslora)
    g = to_gpu(L)
    q = gpu_q(L, g)
    w_cd = qn.dequantize(q, torch.bfloat16)
    y1 = qn.linear_fwd_cached(w_cd, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], rslora=rslora)
    y2 = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], rslora=rslora, path="dequant")
    y3 = qn.linear_fwd_cached(w_cd, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], rslora=rslora)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    o = oracle_layer(L)
    s = L.alpha / (np.sqrt(L.r) if rslora else L.r)
    assert_close(to_np(y1), oracle.forward(o["x"], o["W"], o["A"], o["B"], s, o["bias"]), "bf16", "cached rslora")


def test_cached_forward_full_size_sampled():
    """gate_proj at 4096 tokens with W~ cached: sampled entries against the oracle."""
    (L,) = inputs.prefill(projections=["gate_proj"])
    say("fwd cached full", L.M, L.N, L.K)
    g = to_gpu(L)
    w_cd = qn.dequantize(gpu_q(L, g), torch.bfloat16)
    y = qn.linear_fwd_cached(w_cd, g["x"], g["A"], g["B"], L.alpha)
    torch.cuda.synchronize()
    o = oracle_layer(L)
    rng = np.random.default_rng(23)
    ii, jj = rng.integers(0, L.M, 256), rng.integers(0, L.N, 256)
    ii[:2] = [0, L.M - 1]
    jj[:2] = [L.N - 1, 0]
    ref = oracle.forward_at(o["x"], o["W"], o["A"], o["B"], o["s"], ii, jj)
    assert_close(to_np(y)[ii, jj], ref, "bf16", "gate_proj cached sampled")
