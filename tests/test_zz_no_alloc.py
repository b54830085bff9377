"""qlora_linear_fwd_noalloc (the forward without a workspace, on the library's own
scratch array) against qlora_linear_fwd on the same path, through the C ABI: the
outputs must be the same bits.  Two calls in a row, the second on a smaller input,
so the scratch array holds the first call's leftovers when the second runs; a call
that needs more scratch than the library holds is refused before anything runs."""
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
from bit_nf4_quantized_nibble_amd import _lib, inputs
import oracle
from parity import assert_close, oracle_layer, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


def _case(L):
    g = to_gpu(L)
    q = qn.quantize(g["W"], L.block_size, L.double_quant, L.dq_group)
    return g, q


@pytest.mark.parametrize("cases", [
    # (M, N, K, r) twice: decode GEMV then a smaller decode
    [(16, 4096, 4096, 16), (4, 1024, 2048, 8)],
    # fused forward above 16 tokens, then a smaller one (and a decode after it)
    [(300, 1024, 2048, 64), (100, 256, 512, 16), (1, 512, 1024, 16)],
])
def test_noalloc_matches_workspace_entry_point(cases):
    outs = []
    for i, (M, N, K, r) in enumerate(cases):
        L = inputs.random_layer(M, N, K, r, seed=100 + i + M, with_bias=True, with_dy=False)
        say("noalloc", M, N, K, r)
        assert qn.workspace_bytes(_lib.QLORA_OP_FWD, M, N, K, r, torch.bfloat16, _lib.QLORA_FLAG_FUSED) <= \
            _lib.lib().qlora_noalloc_scratch_bytes()
        g, q = _case(L)
        path = "fused" if M > 16 else "auto"
        y_ref, t_ref = qn.linear_fwd(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], save_t=True, path=path)
        y = torch.full_like(y_ref, float("nan"))
        t = torch.full_like(t_ref, float("nan"))
        qn.linear_fwd_noalloc(q, g["x"], g["A"], g["B"], L.alpha, bias=g["bias"], out=y, t_out=t)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), "y differs from qlora_linear_fwd (%d x %d x %d)" % (M, N, K)
        assert torch.equal(t, t_ref), "T0 differs from qlora_linear_fwd"
        o = oracle_layer(L)
        assert_close(to_np(y), oracle.forward(o["x"], o["W"], o["A"], o["B"], o["s"], o["bias"]), "bf16", "oracle")
        outs.append(y)


def test_noalloc_refuses_calls_beyond_its_scratch():
    lib = _lib.lib()
    cap = lib.qlora_noalloc_scratch_bytes()
    assert cap == 32 << 20
    # gate_proj shape at 4096 tokens on the fused path: its cut last round needs 64 MiB
    need = qn.workspace_bytes(_lib.QLORA_OP_FWD, 4096, 14336, 4096, 64, torch.bfloat16, _lib.QLORA_FLAG_FUSED)
    assert need > cap
    N, K, M, r = 14336, 4096, 4096, 64
    q = qn.empty_nf4(N, K, 64, True, 256)
    x = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(r, K, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(N, r, dtype=torch.bfloat16, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qn.QloraError, match="WORKSPACE"):
        qn.linear_fwd_noalloc(q, x, A, B, 128.0, out=y)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a refused call wrote its output"
