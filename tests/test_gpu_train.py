"""GPU parity of the training step of a QLoRA layer stack (qlora-rs README, "Training
(layer stack)"): the MSE loss / gradient kernel, the AdamW kernel and the whole
stack step (forward, loss, backward, AdamW) against the fp64 oracle in
oracle/training.py, through the C ABI.

Bars: the loss is an fp32 sum in a fixed order (rel <= 1e-5 alone, 5e-3 after a
bf16 stack); dy within one unit in the last place of the oracle's single rounding
and >= 99.9 % bit-identical; AdamW in fp32 against fp64 within a few binary32
rounding units (4e-7) of the terms each value is summed from; gradients and first moments of the stack step at the layer's bf16
bar (rel-L2 <= 5e-3, max <= 1e-2 max); updated parameters equal the oracle's where
the gradient is clearly away from zero (AdamW's first step moves each parameter by
about lr sign(g), so a gradient inside the bf16 noise may flip the step).  The
oracle gets the hyper-parameters as the binary32 values the C ABI carries."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_nibble_amd as qn
import oracle
from oracle import training
from bit_nf4_quantized_nibble_amd import inputs
from parity import TORCH_DT, assert_close, say, to_np

pytestmark = pytest.mark.gpu


def f32(v):
    return float(np.float32(v))


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).astype(np.int64)


def _ulps(got_t, ref_vals, dtype):
    ref_bits = oracle.to_bits(ref_vals.astype(np.float32), dtype).astype(np.int64)
    g = _bits(got_t).reshape(-1)
    r = ref_bits.reshape(-1)
    og = np.where(g & 0x8000, -(g & 0x7FFF), g & 0x7FFF)
    orf = np.where(r & 0x8000, -(r & 0x7FFF), r & 0x7FFF)
    return np.abs(og - orf)


@pytest.mark.parametrize("cd", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", [(1000, 37), (4096, 1024), (3,)])
def test_mse_loss_and_gradient(cd, shape):
    say("mse", cd, shape)
    g = torch.Generator().manual_seed(len(shape) * 100 + shape[0])
    y = (torch.randn(*shape, generator=g)).to(TORCH_DT[cd])
    t = (torch.randn(*shape, generator=g) * 0.5).to(TORCH_DT[cd])
    loss, dy = qn.mse_loss_grad(y.cuda(), t.cuda())
    torch.cuda.synchronize()
    ly, lt = oracle.operand(y, cd), oracle.operand(t, cd)
    ref_loss, ref_dy = training.mse_loss_grad(ly, lt)
    assert float(loss.item()) == pytest.approx(ref_loss, rel=1e-5)
    if cd == "f32":
        got = dy.cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(got, ref_dy, rtol=2 ** -23, atol=0)
    else:
        d = _ulps(dy, oracle.round64_to(ref_dy, cd), cd)
        assert d.max() <= 1 and np.mean(d == 0) >= 0.999


def test_mse_is_deterministic():
    say("mse determinism")
    g = torch.Generator().manual_seed(3)
    y = torch.randn(3000, 700, generator=g).to(torch.bfloat16).cuda()
    t = torch.randn(3000, 700, generator=g).to(torch.bfloat16).cuda()
    a = [qn.mse_loss_grad(y, t)[0].item() for _ in range(3)]
    assert a[0] == a[1] == a[2]


@pytest.mark.parametrize("wd", [0.0, 0.1])
@pytest.mark.parametrize("step", [1, 2, 10, 1000])
def test_adamw_against_oracle(wd, step):
    """One update from a random state (moments included) at several step counts: the
    kernel is an elementwise map (theta, g, m, v) -> (theta', m', v')."""
    say("adamw", wd, step)
    n = 100003
    g = torch.Generator().manual_seed(11 + step)
    th0 = torch.randn(n, generator=g)
    gr = torch.randn(n, generator=g) * 1e-2
    m0 = torch.randn(n, generator=g) * 1e-2
    v0 = torch.rand(n, generator=g) * 1e-4
    lr, b1, b2, eps, wd = f32(1e-3), f32(0.9), f32(0.999), f32(1e-8), f32(wd)
    p, m, v = th0.cuda(), m0.cuda(), v0.cuda()
    pcd = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    qn.adamw_step(p, gr.cuda(), m, v, step, lr, b1, b2, eps, wd, param_cd=pcd)
    torch.cuda.synchronize()
    t64, g64, m64, v64 = (a.numpy().astype(np.float64) for a in (th0, gr, m0, v0))
    rt, rm, rv = training.adamw(t64, g64, m64, v64, step, lr, b1, b2, eps, wd)
    # size of the terms each fp32 result is formed from (a difference can cancel)
    scale = {"m": b1 * np.abs(m64) + (1 - b1) * np.abs(g64), "v": b2 * v64 + (1 - b2) * g64 * g64}
    bc1, bc2 = 1 - b1 ** step, 1 - b2 ** step
    den = np.sqrt(rv / bc2) + eps
    # theta: its own terms, plus the update's sensitivity to the rounding of m and v
    scale["theta"] = (np.abs(t64) + lr * np.abs(rm / bc1) / den
                      + lr * (scale["m"] / bc1) / den + lr * np.abs(rm / bc1) * (scale["v"] / bc2) / (den * den * np.sqrt(rv / bc2) + 1e-30))
    for got, ref, what in ((p, rt, "theta"), (m, rm, "m"), (v, rv, "v")):
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= 4e-7 * scale[what] + 1e-30), (what, float((err / scale[what]).max()))
    # the compute-dtype copy is the rounding of the fp32 master
    assert torch.equal(pcd, p.to(torch.bfloat16))


def _gpu_stack(S, bs=64, dq=True):
    dt = TORCH_DT[S.cd]
    layers, oracle_layers = [], []
    for W, A, B in zip(S.Ws, S.As, S.Bs):
        q = qn.quantize(W.cuda(), bs, dq, 256)
        layers.append(qn.StackLayer.create(q, A, B, dt))
        oq = oracle.quantize(W.numpy(), bs, dq, 256)
        oracle_layers.append(dict(W=oracle.weight_operand(oq, S.cd).astype(np.float64),
                                  a32=A.numpy().astype(np.float64), b32=B.numpy().astype(np.float64),
                                  m_a=np.zeros(A.shape), v_a=np.zeros(A.shape), m_b=np.zeros(B.shape),
                                  v_b=np.zeros(B.shape)))
    return layers, oracle_layers


OPT = dict(lr=f32(1e-3), beta1=f32(0.9), beta2=f32(0.999), eps=f32(1e-8), weight_decay=f32(0.01))


@pytest.mark.parametrize("path", ["fused", "dequant"])
@pytest.mark.parametrize("dims,M", [([256, 512, 256, 128], 200), ([512, 256], 64)])
def test_stack_step_against_oracle(path, dims, M):
    S = inputs.stack(dims, M, r=16, seed=len(dims) * 10 + M)
    say("stack", path, dims, M)
    layers, ol = _gpu_stack(S)
    x, t = S.x.cuda(), S.target.cuda()
    loss = qn.stack_train_step(layers, x, t, S.alpha, 1, path=path, **OPT)
    torch.cuda.synchronize()
    xo, to_ = oracle.operand(S.x, "bf16"), oracle.operand(S.target, "bf16")
    ref = training.stack_step(xo, to_, ol, S.alpha / S.r, "bf16", 1, OPT["lr"], OPT["beta1"], OPT["beta2"],
                              OPT["eps"], OPT["weight_decay"])
    assert float(loss.item()) == pytest.approx(ref["loss"], rel=5e-3)
    for l, (L, (dA, dB), (a, ma, va, b, mb, vb)) in enumerate(zip(layers, ref["grads"], ref["new"])):
        assert_close(to_np(L.grad_a), dA, "bf16", "layer %d dA" % l)
        assert_close(to_np(L.grad_b), dB, "bf16", "layer %d dB" % l)
        assert_close(to_np(L.m_a), ma, "bf16", "layer %d m_a" % l)
        assert_close(to_np(L.m_b), mb, "bf16", "layer %d m_b" % l)
        for got, want, gref, old, what in ((L.a32, a, dA, ol[l]["a32"], "A"), (L.b32, b, dB, ol[l]["b32"], "B")):
            gv = to_np(got).astype(np.float64)
            clear = np.abs(gref) >= 0.05 * np.abs(gref).max()
            assert clear.mean() > 0.5
            err = np.abs(gv - want)[clear]
            assert err.max() <= 0.05 * OPT["lr"] + 1e-6 * np.abs(want[clear]).max(), (l, what, float(err.max()))
            assert np.all(np.abs(gv - old) <= 1.02 * OPT["lr"] * (1 + OPT["weight_decay"] * np.abs(old)) + 1e-6)
        assert torch.equal(L.lora_a, L.a32.to(L.lora_a.dtype))
        assert torch.equal(L.lora_b, L.b32.to(L.lora_b.dtype))


def test_stack_steps_reduce_the_loss():
    S = inputs.stack([256, 256, 128], 256, r=16, seed=77)
    say("stack descent")
    layers, _ = _gpu_stack(S)
    x, t = S.x.cuda(), S.target.cuda()
    losses = [float(qn.stack_train_step(layers, x, t, S.alpha, k, lr=1e-2).item()) for k in range(1, 9)]
    assert losses[-1] < losses[0], losses


def test_stack_rejects_layers_that_do_not_chain():
    S = inputs.stack([256, 128], 8, r=8, seed=1)
    S2 = inputs.stack([256, 128], 8, r=8, seed=2)
    a, _ = _gpu_stack(S)
    b, _ = _gpu_stack(S2)
    with pytest.raises(qn.QloraError, match="SHAPE"):
        qn.stack_train_step([a[0], b[0]], S.x.cuda(), torch.zeros(8, 128, dtype=torch.bfloat16, device="cuda"),
                            S.alpha, 1, lr=1e-3)
