#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 linear layer on one MI355X.

Headline: the training step of the seven projections of one Llama-3-8B-shaped
block (q/o 4096x4096, k/v 1024x4096, gate/up 14336x4096, down 4096x14336; NF4 block
64 with double quantization; 4096 tokens; LoRA r = 64, alpha = 128; bf16 compute):
one step = the forward of all seven projections followed by their backward (dX,
dA, dB).  The projections that read the same x (q / k / v, gate / up) are forwarded
as one qlora_linear_fwd_group call each, as a transformer block calls them; o, down
and every backward are per-projection calls; all on the library's default path (at
4096 tokens: W~ dequantized into the workspace, then the dense MFMA GEMM).  value =
algorithmic TFLOP/s of that step (dequantization is not credited).  Beside it: the
same step with every projection a call of its own (per_projection_step), and forced
onto the fused dequant-GEMM kernels (QLORA_FLAG_FUSED, fused_path_step).

Also reported on the same line, each against its own MI355X roofline:
  gemv      decode forward at m = 1, 4, 16 (4096x4096, r = 16), GB/s over cold weights, and one
            token through the block's seven projections (per projection and grouped)
  quantize  NF4 quantize of a 4096x4096 fp32 weight without / with double quant, GB/s
  dequantize  the double-quantized weight back to bf16 / fp32, GB/s
  dtype_sweep  the prefill forward in bf16, f16 and f32 compute (10 warm-up, 100 timed passes)
  merge     the adapter merge of the block's seven projections, GB/s
  stack_train_step  forward + MSE + backward + AdamW of a 3-layer stack of projection shapes
  share_step  the headline step at 512 tokens (one GPU's share of 8-way data parallelism)
  cpu_baseline  the oracle (plain C, fp64) on a bounded sample of the step's work
  roofline  the dominant kernel of the step, timed with HIP events on its stream

Inputs are seeded synthetic tensors (bit_nf4_quantized_nibble_amd.inputs): trained
weights are not needed because cost and numerics depend on shapes and value ranges.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused NF4 QLoRA linear TFLOP/s (prefill/bwd) + GEMV HBM GB/s, % of roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
SHARE_TOKENS = 512  # one GPU's tokens when 4096 are split data-parallel over 8 GPUs


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def fwd_flops(m, n, k, r):
    return 2.0 * m * n * k + 2.0 * m * r * k + 2.0 * m * n * r


def bwd_flops(m, n, k, r):
    # dX base + dT A, plus dT = s dY B, dA = dT^T x, dB = s dY^T T0
    return 2.0 * m * n * k + 2.0 * m * r * k + 2.0 * m * n * r + 2.0 * r * k * m + 2.0 * n * r * m


class Layer:
    """Device tensors and prebuilt C-ABI argument tuples for one projection."""

    def __init__(self, L, x, ws_f, ws_b, qn, torch, lib, flags=0):
        self.name, self.M, self.N, self.K, self.r, self.alpha = L.name, L.M, L.N, L.K, L.r, L.alpha
        dev = "cuda"
        W = L.W.to(dev)
        self.q = qn.quantize(W, L.block_size, L.double_quant, L.dq_group)
        del W
        self.A, self.B = L.A.to(dev), L.B.to(dev)
        self.dY = L.dY.to(dev) if L.dY is not None else None
        dt = x.dtype
        self.y = torch.empty(self.M, self.N, dtype=dt, device=dev)
        self.t0 = torch.empty(self.M, self.r, dtype=torch.float32, device=dev)
        self.dx = torch.empty(self.M, self.K, dtype=dt, device=dev)
        self.da = torch.empty(self.r, self.K, dtype=torch.float32, device=dev)
        self.db = torch.empty(self.N, self.r, dtype=torch.float32, device=dev)
        self.desc = self.q.descriptor()
        cd = qn.dtype_code(dt)
        stream = torch.cuda.current_stream().cuda_stream
        self.fwd_args = (ctypes.byref(self.desc), x.data_ptr(), self.M, self.A.data_ptr(), self.B.data_ptr(),
                         self.r, float(self.alpha), flags, None, cd, self.y.data_ptr(), self.t0.data_ptr(),
                         ws_f.data_ptr(), ws_f.numel(), stream)
        if self.dY is not None:
            self.bwd_args = (ctypes.byref(self.desc), x.data_ptr(), self.dY.data_ptr(), self.M,
                             self.A.data_ptr(), self.B.data_ptr(), self.r, float(self.alpha), flags, cd,
                             self.t0.data_ptr(), self.dx.data_ptr(), self.da.data_ptr(),
                             self.db.data_ptr(), ws_b.data_ptr(), ws_b.numel(), stream)
        self.lib = lib

    def fwd(self):
        rc = self.lib.qlora_linear_fwd(*self.fwd_args)
        if rc:
            raise RuntimeError("fwd %s: %d %s" % (self.name, rc, self.lib.qlora_last_error()))

    def bwd(self):
        rc = self.lib.qlora_linear_bwd(*self.bwd_args)
        if rc:
            raise RuntimeError("bwd %s: %d %s" % (self.name, rc, self.lib.qlora_last_error()))


class GroupUnit:
    """Layers that read the same x called as one group (qlora_linear_fwd_group /
    qlora_linear_bwd_group): the outputs side by side in one [M, sum N] buffer, dY
    likewise, one dX (the sum of the group's input gradients); adapters, T0, dA and
    dB in the layers' own buffers."""

    def __init__(self, layers, x, torch, lib, qn, group_bwd=True):
        self.layers, self.lib, self.name = layers, lib, "+".join(l.name for l in layers)
        self.group_bwd = group_bwd
        g = len(layers)
        M, K = layers[0].M, layers[0].K
        N = sum(l.N for l in layers)
        vp = ctypes.c_void_p
        self.w = (ctypes.POINTER(qn._lib.QloraNf4) * g)(*[ctypes.pointer(l.desc) for l in layers])
        self.a = (vp * g)(*[l.A.data_ptr() for l in layers])
        self.b = (vp * g)(*[l.B.data_ptr() for l in layers])
        self.r = (ctypes.c_int32 * g)(*[l.r for l in layers])
        self.alpha = (ctypes.c_float * g)(*[float(l.alpha) for l in layers])
        self.t0 = (vp * g)(*[l.t0.data_ptr() for l in layers])
        self.da = (vp * g)(*[l.da.data_ptr() for l in layers])
        self.db = (vp * g)(*[l.db.data_ptr() for l in layers])
        self.y = torch.empty(M, N, dtype=x.dtype, device="cuda")
        cd = qn.dtype_code(x.dtype)
        wsf = lib.qlora_group_workspace_bytes(0, g, self.w, M, self.r, cd)
        self.ws_f = torch.empty(max(wsf, 1), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        self.fwd_args = (g, self.w, x.data_ptr(), M, self.a, self.b, self.r, self.alpha, 0, None, cd,
                         self.y.data_ptr(), self.t0, self.ws_f.data_ptr(), self.ws_f.numel(), stream)
        if layers[0].dY is None:  # forward only
            self.bwd_args = None
            return
        self.dy = torch.cat([l.dY for l in layers], dim=1).contiguous()
        self.dx = torch.empty(M, K, dtype=x.dtype, device="cuda")
        wsb = lib.qlora_group_workspace_bytes(1, g, self.w, M, self.r, cd)
        self.ws_b = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        self.bwd_args = (g, self.w, x.data_ptr(), self.dy.data_ptr(), M, self.a, self.b, self.r, self.alpha, 0, cd,
                         self.t0, self.dx.data_ptr(), self.da, self.db, self.ws_b.data_ptr(), self.ws_b.numel(),
                         stream)

    def fwd(self):
        rc = self.lib.qlora_linear_fwd_group(*self.fwd_args)
        if rc:
            raise RuntimeError("fwd %s: %d %s" % (self.name, rc, self.lib.qlora_last_error()))

    def bwd(self):
        if not self.group_bwd:  # each projection's own backward on the T0 the group forward saved
            for l in self.layers:
                l.bwd()
            return
        rc = self.lib.qlora_linear_bwd_group(*self.bwd_args)
        if rc:
            raise RuntimeError("bwd %s: %d %s" % (self.name, rc, self.lib.qlora_last_error()))


GROUPS = (("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",))


def tensor_sha256(t):
    import hashlib
    return hashlib.sha256(t.contiguous().view(-1).view(__import__("torch").uint8).numpy().tobytes()).hexdigest()


def build_block(cd, with_dy, qn, torch, lib, inputs, m=4096, flags=0, hashes=None):
    Ls = inputs.prefill(seed=0, cd=cd, m=m, with_dy=with_dy)
    if hashes is not None:  # SHA-256 of every input tensor, as generated on the host
        for L in Ls:
            hashes.setdefault("x_K%d" % L.K, tensor_sha256(L.x))
            for name, t in (("W", L.W), ("A", L.A), ("B", L.B), ("dY", L.dY)):
                if t is not None:
                    hashes["%s_%s" % (L.name, name)] = tensor_sha256(t)
    xs = {}
    for L in Ls:
        if L.K not in xs:
            xs[L.K] = L.x.to("cuda")
    op_f, op_b = 0, 1
    wsf = max(qn.workspace_bytes(op_f, L.M, L.N, L.K, L.r, xs[L.K].dtype, flags) for L in Ls)
    wsb = max(qn.workspace_bytes(op_b, L.M, L.N, L.K, L.r, xs[L.K].dtype, flags) for L in Ls) if with_dy else 1
    ws_f = torch.empty(wsf, dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    layers = [Layer(L, xs[L.K], ws_f, ws_b, qn, torch, lib, flags) for L in Ls]
    del Ls
    return layers, (xs, ws_f, ws_b)


def time_loop(fn, iters, torch, per_step=None):
    """Mean seconds per call over `iters` calls between two synchronizations; with
    `per_step` (a list) also the device time of each call from event pairs recorded
    between the calls (no synchronization inside the loop)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)] if per_step is not None else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(iters):
        if evs:
            evs[i].record()
        fn()
    if evs:
        evs[iters].record()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / iters
    if evs:
        per_step.extend(evs[i].elapsed_time(evs[i + 1]) for i in range(iters))
    return sec


def percentiles(ms):
    """median, p10 and p90 of a list of milliseconds (nearest rank)."""
    v = sorted(ms)
    pick = lambda q: v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    return {"median": round(pick(0.5), 4), "p10": round(pick(0.1), 4), "p90": round(pick(0.9), 4), "n": len(v)}


def bench_step(args, qn, torch, lib, inputs, flags=0, hashes=None, grouped=False, m=4096):
    layers, keep = build_block("bf16", True, qn, torch, lib, inputs, m=m, flags=flags, hashes=hashes)
    units = layers
    if grouped:  # projections that read the same x as one call each (q / k / v, gate / up)
        by = {l.name: l for l in layers}
        xs = keep[0]
        units = [GroupUnit([by[n] for n in grp], xs[by[grp[0]].K], torch, lib, qn, grouped == "both")
                 if len(grp) > 1 else by[grp[0]] for grp in GROUPS]
    torch.cuda.synchronize()
    flops = sum(fwd_flops(l.M, l.N, l.K, l.r) + bwd_flops(l.M, l.N, l.K, l.r) for l in layers)
    ff = {k: 0.0 for k in ("fwd_gemm", "lora_down", "bwd_dx", "bwd_dt", "bwd_da", "bwd_db")}
    for l in layers:
        ff["fwd_gemm"] += 2.0 * l.M * l.N * l.K + 2.0 * l.M * l.N * l.r
        ff["lora_down"] += 2.0 * l.M * l.r * l.K
        ff["bwd_dx"] += 2.0 * l.M * l.N * l.K + 2.0 * l.M * l.r * l.K
        ff["bwd_dt"] += 2.0 * l.M * l.N * l.r
        ff["bwd_da"] += 2.0 * l.r * l.K * l.M
        ff["bwd_db"] += 2.0 * l.N * l.r * l.M

    def step():
        for u in units:
            u.fwd()
        for u in units:
            u.bwd()

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timing", args.steps, "steps")
    step_ms = []
    sec = time_loop(step, args.steps, torch, per_step=step_ms)
    # per-kernel times from a second, profiled pass (the event pairs it records around
    # each launch stay out of the timed steps above)
    qn.profile_enable(True)
    time_loop(step, args.steps, torch)
    prof = qn.profile_read()
    qn.profile_enable(False)
    if prof.get("bwd_db", (0.0, 0))[1] == 0:  # dA and dB share one launch on the skinny path
        ff["bwd_da"] += ff.pop("bwd_db")
    kernels = {}
    for kind, (ms, n) in prof.items():
        if n == 0:
            continue
        per_step = ms / args.steps
        ent = {"ms_per_step": round(per_step, 4), "launches_per_step": n // args.steps}
        if kind in ff:
            tf = ff[kind] / (per_step / 1e3) / 1e12
            ent["tflops"] = round(tf, 2)
            ent["frac_bf16_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
        kernels[kind] = ent
    # The dominant kernel: the largest share of the step's time.
    dom = max((k for k in kernels if k in ff), key=lambda k: kernels[k]["ms_per_step"])
    dom_ms = prof[dom][0] / prof[dom][1]  # average launch duration
    dom_flops = ff[dom] / (prof[dom][1] / args.steps)  # algorithmic flops per launch
    achieved = dom_flops / (dom_ms / 1e3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": (measured_traffic(dom, "grouped" if grouped == "fwd" else "per_projection")
                            if flags == 0 and grouped in (False, "fwd") else None),
                "avg_launch_ms": round(dom_ms, 4), "flops_per_launch": dom_flops}
    result = dict(sec=sec, flops=flops, kernels=kernels, roofline=roofline, step_ms=percentiles(step_ms),
                  fwd_ms=sum(kernels.get(k, {}).get("ms_per_step", 0) for k in ("fwd_gemm", "lora_down")),
                  layers=[(l.name, l.N, l.K) for l in layers])
    del layers, keep, units
    torch.cuda.empty_cache()
    return result


def bench_dtype_sweep(qn, torch, lib, inputs, warmup=10, steps=100):
    """The block's prefill forward (seven projections, 4096 tokens) in bf16, f16 and
    f32 compute, timed like the headline: `warmup` untimed passes, then `steps`
    passes with the device time of each from event pairs between them (median,
    p10, p90) and the mean over the whole loop."""
    out = {}
    for cd in ("bf16", "f16", "f32"):
        layers, keep = build_block(cd, False, qn, torch, lib, inputs)
        flops = sum(fwd_flops(l.M, l.N, l.K, l.r) for l in layers)

        def fwd():
            for l in layers:
                l.fwd()

        for _ in range(warmup):
            fwd()
        per = []
        sec = time_loop(fwd, steps, torch, per_step=per)
        pc = percentiles(per)
        tf = flops / (pc["median"] / 1e3) / 1e12
        peak = PEAK_BF16_TFLOPS if cd != "f32" else PEAK_F32_TFLOPS
        out[cd] = {"ms_median": pc["median"], "ms_p10": pc["p10"], "ms_p90": pc["p90"], "ms_mean": round(sec * 1e3, 4),
                   "passes": steps, "warmup": warmup, "tflops": round(tf, 2), "peak": peak, "frac": round(tf / peak, 4)}
        del layers, keep
        torch.cuda.empty_cache()
    return out


def bench_path_sweep(qn, torch, lib, inputs, copies=8, replays=5):
    """Forward of q_proj and gate_proj (r 64, bf16) at several token counts on both
    dequant-GEMM paths: fused (decode inside the GEMM) and dequantize-then-GEMM (W~
    written once into the call's workspace).  The calls cycle through `copies`
    copies of the two quantized weights (about 300 MB of codes and scales, more than
    the 256 MB last-level cache), so each call reads its weight from HBM as a block
    of a real model would.  "auto" is the call without a path flag (up to 64 tokens
    the split-K decode kernel, above that dequantize-then-GEMM).  Reports time per q + gate pair, TFLOP/s and the
    workspace each path needs (the memory side of the trade-off).  A third column,
    "cached", runs qlora_linear_fwd_cached on W~ dequantized once per weight copy
    beforehand (held resident: 2 bytes per weight instead of about 0.53)."""
    ms = (16, 32, 64, 128, 256, 512, 1024, 2048, 4096)
    Ls = inputs.prefill(seed=0, cd="bf16", m=max(ms), projections=["q_proj", "gate_proj"])
    x = Ls[0].x.to("cuda")
    cd = qn.dtype_code(x.dtype)
    stream = torch.cuda.current_stream().cuda_stream
    projs = []
    for L in Ls:
        W = L.W.to("cuda")
        q0 = qn.quantize(W, L.block_size, L.double_quant, L.dq_group)
        del W
        qs = [qn.NF4Weight(q0.rows, q0.cols, q0.block_size, True, q0.dq_group, q0.codes.clone(), None,
                           q0.absmax_q.clone(), q0.absmax_scale2.clone()) for _ in range(copies)]
        wcs = [qn.dequantize(q, x.dtype) for q in qs]
        projs.append((L, qs, [q.descriptor() for q in qs], L.A.to("cuda"), L.B.to("cuda"),
                      torch.empty(max(ms), L.N, dtype=x.dtype, device="cuda"), wcs))
        del q0
    paths = (("auto", 0), ("fused", qn._lib.QLORA_FLAG_FUSED), ("dequant", qn._lib.QLORA_FLAG_DEQUANT_GEMM),
             ("cached", None))

    def ws_need(m, L, flag):
        if flag is None:
            return qn.workspace_bytes(qn._lib.QLORA_OP_FWD_CACHED, m, L.N, L.K, L.r, x.dtype)
        return qn.workspace_bytes(0, m, L.N, L.K, L.r, x.dtype, flag)

    wsb = max(ws_need(m, L, fl) for m in ms for L in Ls for _, fl in paths)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    st = torch.cuda.Stream()
    out = {"weights_cycled": copies, "timing": "HIP graph of the 2 x copies calls, replayed %d times" % replays}
    for m in ms:
        flops = sum(fwd_flops(m, L.N, L.K, L.r) for L in Ls)
        res = {}
        for path, flag in paths:
            if flag is None:
                f = lib.qlora_linear_fwd_cached
                calls = [(wc[c].data_ptr(), L.N, L.K, x.data_ptr(), m, A.data_ptr(), B.data_ptr(), L.r,
                          float(L.alpha), 0, None, cd, y.data_ptr(), None, ws.data_ptr(), ws.numel(), st.cuda_stream)
                         for c in range(copies) for (L, qs, ds, A, B, y, wc) in projs]
            else:
                f = lib.qlora_linear_fwd
                calls = [(ctypes.byref(d), x.data_ptr(), m, A.data_ptr(), B.data_ptr(), L.r, float(L.alpha), flag,
                          None, cd, y.data_ptr(), None, ws.data_ptr(), ws.numel(), st.cuda_stream)
                         for c in range(copies) for (L, qs, ds, A, B, y, wc) in projs for d in (ds[c],)]

            def fwd():
                for a in calls:
                    rc = f(*a)
                    if rc:
                        raise RuntimeError("fwd %s m=%d: %d %s" % (path, m, rc, lib.qlora_last_error()))

            # eager once (the reference outputs), then the same calls as one graph, so
            # that host launch gaps do not hide the kernels' time at small m
            torch.cuda.synchronize()
            with torch.cuda.stream(st):
                fwd()
            st.synchronize()
            eager = [p[5][:m].clone() for p in projs]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                fwd()
            for p in projs:
                p[5][:m].fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            same = all(torch.equal(e, p[5][:m]) for e, p in zip(eager, projs))
            # replay() launches on the current stream: the events go there too
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            same = same and all(torch.equal(e, p[5][:m]) for e, p in zip(eager, projs))
            sec = e0.elapsed_time(e1) / 1e3 / (replays * copies)
            del g
            need = max(ws_need(m, L, flag) for L in Ls)
            res[path] = {"ms": round(sec * 1e3, 4), "tflops": round(flops / sec / 1e12, 1),
                         "workspace_mb": round(need / 2 ** 20, 1), "replay_matches_eager": same}
            if flag is None:
                res[path]["resident_w_mb"] = round(sum(L.N * L.K * 2 for L in Ls) / 2 ** 20, 1)
        res["faster"] = min(("auto", "fused", "dequant"), key=lambda k: res[k]["ms"])
        out["m%d" % m] = res
    del projs, ws, x
    torch.cuda.empty_cache()
    return out


def bench_gemv(qn, torch, lib, inputs, copies=40, iters=400):
    """Decode GEMV over `copies` independent weights (> the 256 MB last-level cache),
    so each call streams its weight from HBM."""
    out = {}
    for m in (1, 4, 16):
        L = inputs.decode(m)
        W = L.W.to("cuda")
        q0 = qn.quantize(W, 64, True, 256)
        del W
        sets = []
        for c in range(copies):
            q = qn.NF4Weight(q0.rows, q0.cols, 64, True, 256, q0.codes.clone(), None,
                             q0.absmax_q.clone(), q0.absmax_scale2.clone())
            x = L.x.to("cuda").clone()
            A, B = L.A.to("cuda").clone(), L.B.to("cuda").clone()
            y = torch.empty(m, 4096, dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(qn.workspace_bytes(0, m, 4096, 4096, 16, torch.bfloat16), dtype=torch.uint8,
                             device="cuda")
            d = q.descriptor()
            args = (ctypes.byref(d), x.data_ptr(), m, A.data_ptr(), B.data_ptr(), 16, 32.0, 0, None, 1,
                    y.data_ptr(), None, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
            sets.append((q, x, A, B, y, ws, d, args))
        f = lib.qlora_linear_fwd
        for s in sets:
            f(*s[7])
        torch.cuda.synchronize()
        qn.profile_enable(True)
        t0 = time.perf_counter()
        for i in range(iters):
            rc = f(*sets[i % copies][7])
            if rc:
                raise RuntimeError("gemv rc %d" % rc)
        torch.cuda.synchronize()
        call_us = (time.perf_counter() - t0) / iters * 1e6
        prof = qn.profile_read()
        qn.profile_enable(False)
        k_ms, k_n = prof["gemv"]
        e_ms = prof["reduce"][0] + prof["lora_down"][0]  # the epilogue (y = partial sums + T B^T + bias)
        kern_us = k_ms / k_n * 1e3
        epi_us = e_ms / k_n * 1e3
        codes = 4096 * 4096 // 2 + 4096 * 4096 // 64 + 4096 * 4096 // 64 // 256 * 4
        # the GEMV kernel must read the packed weight, x and lora_a (the LoRA down-projection
        # rides along); the layer also reads lora_b and writes y
        kern_bytes = codes + 2 * m * 4096 + 2 * 16 * 4096
        layer_bytes = codes + 2 * m * 4096 + 2 * 16 * 4096 * 2 + 2 * m * 4096
        gbs_kernel = kern_bytes / (kern_us * 1e-6) / 1e9
        gbs_layer = layer_bytes / ((kern_us + epi_us) * 1e-6) / 1e9
        out["m%d" % m] = {"kernel_us": round(kern_us, 3), "epilogue_us": round(epi_us, 3),
                          "call_us_wall": round(call_us, 3), "kernel_bytes": kern_bytes,
                          "kernel_gbs": round(gbs_kernel, 1), "kernel_frac": round(gbs_kernel / PEAK_HBM_GBS, 4),
                          "layer_bytes": layer_bytes, "layer_gbs_device": round(gbs_layer, 1),
                          "layer_frac": round(gbs_layer / PEAK_HBM_GBS, 4),
                          "stream": gemv_stream(torch, f, sets, layer_bytes)}
        del sets
        torch.cuda.empty_cache()
    out["move_probe_9mb"] = move_probe(torch)
    return out


def gemv_stream(torch, f, sets, layer_bytes, replays=10):
    """Back-to-back stream of distinct decode GEMVs: one call per weight copy captured
    in a HIP graph (no host launch gaps, no event pairs), replayed; every replay's
    outputs must equal the eager outputs bit for bit."""
    eager = [s[4].clone() for s in sets]  # y of each copy from the eager calls above
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        h = torch.cuda.current_stream().cuda_stream
        for s in sets:
            a = s[7]
            rc = f(*(a[:-1] + (h,)))
            if rc:
                raise RuntimeError("gemv capture rc %d" % rc)
    for s in sets:
        s[4].zero_()
    g.replay()
    torch.cuda.synchronize()
    ok = all(torch.equal(s[4], e) for s, e in zip(sets, eager))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ok = ok and all(torch.equal(s[4], e) for s, e in zip(sets, eager))
    us = e0.elapsed_time(e1) / (replays * len(sets)) * 1e3
    del g
    gbs = layer_bytes / (us * 1e-6) / 1e9
    return {"us_per_call": round(us, 3), "layer_gbs": round(gbs, 1), "layer_frac": round(gbs / PEAK_HBM_GBS, 4),
            "replays_match_eager": ok}


def bench_decode_block(qn, torch, lib, inputs, copies=3, replays=10):
    """Decode (one token) of the block's seven projections, r 64: every projection a
    call of its own, and q / k / v and gate / up as one group call each; `copies`
    copies of the block's weights (more than the 256 MB last-level cache) in turn,
    each form captured in a HIP graph and replayed (every replay's outputs must equal
    the eager ones)."""
    blocks = [build_block("bf16", False, qn, torch, lib, inputs, m=1) for _ in range(copies)]
    nbytes = 0
    for l in blocks[0][0]:
        n, k, r = l.N, l.K, l.r
        nbytes += n * k // 2 + n * k // 64 + n * k // 64 // 256 * 4 + 2 * k + 2 * r * k + 2 * n * r + 2 * n
    out = {"tokens": 1, "bytes_per_block": nbytes}
    for form in ("per_projection", "grouped"):
        calls, outs = [], []
        for layers, keep in blocks:
            if form == "grouped":
                by = {l.name: l for l in layers}
                units = [GroupUnit([by[n] for n in grp], keep[0][by[grp[0]].K], torch, lib, qn, False)
                         if len(grp) > 1 else by[grp[0]] for grp in GROUPS]
            else:
                units = layers
            for u in units:
                grouped = isinstance(u, GroupUnit)
                calls.append((lib.qlora_linear_fwd_group if grouped else lib.qlora_linear_fwd, u.fwd_args))
                outs.append(u.y)
        for f, a in calls:
            if f(*a):
                raise RuntimeError("decode block: %s" % lib.qlora_last_error())
        torch.cuda.synchronize()
        eager = [y.clone() for y in outs]
        st = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            h = torch.cuda.current_stream().cuda_stream
            for f, a in calls:
                if f(*(a[:-1] + (h,))):
                    raise RuntimeError("decode block capture: %s" % lib.qlora_last_error())
        for y in outs:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        ok = all(torch.equal(y, e) for y, e in zip(outs, eager))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ok = ok and all(torch.equal(y, e) for y, e in zip(outs, eager))
        us = e0.elapsed_time(e1) / (replays * copies) * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        out[form] = {"us_per_block": round(us, 2), "calls_per_block": len(calls) // copies, "gbs": round(gbs, 1),
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "replays_match_eager": ok}
        del g
    del blocks
    torch.cuda.empty_cache()
    return out


def move_probe(torch, nbytes=8933376, copies=40, replays=10):
    """Empirical ceiling of one small launch that moves ~9 MB through HBM: a plain
    device copy of nbytes / 2 into another nbytes / 2 (read + write = nbytes), 40
    distinct buffer pairs in a HIP graph, so every copy misses the last-level cache."""
    half = nbytes // 4  # int16 elements in nbytes / 2
    srcs = [torch.ones(half, dtype=torch.int16, device="cuda") for _ in range(copies)]
    dsts = [torch.empty_like(t) for t in srcs]
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for a, b in zip(srcs, dsts):
            b.copy_(a)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for a, b in zip(srcs, dsts):
            b.copy_(a)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (replays * copies) * 1e3
    moved = 4 * half
    del g, srcs, dsts
    torch.cuda.empty_cache()
    gbs = moved / (us * 1e-6) / 1e9
    return {"bytes_moved": moved, "us": round(us, 3), "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}


def bench_merge(qn, torch, inputs, iters=5):
    """Adapter merge W_merged = RNE_bf16(w_hat + s B A) of the seven projections of the
    block (r = 64), cycled so that every call streams its weight from HBM (the seven
    outputs and codes together exceed the last-level cache)."""
    layers = inputs.prefill(m=1)
    sets = []
    for L in layers:
        q = qn.quantize(L.W.to("cuda"), 64, True, 256)
        A, B = L.A.to("cuda"), L.B.to("cuda")
        out = torch.empty(L.N, L.K, dtype=torch.bfloat16, device="cuda")
        sets.append((L, q, A, B, out))
    for L, q, A, B, out in sets:
        qn.merge(q, A, B, L.alpha, out=out)
    torch.cuda.synchronize()
    per = {}
    total_bytes = 0
    # the block: `iters` passes over the seven merges between one event pair
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        for L, q, A, B, out in sets:
            qn.merge(q, A, B, L.alpha, out=out)
    e1.record()
    torch.cuda.synchronize()
    block_us = e0.elapsed_time(e1) * 1e3 / iters
    # the same calls with the library's event pair around each one
    qn.profile_enable(True)
    for _ in range(iters):
        for L, q, A, B, out in sets:
            qn.merge(q, A, B, L.alpha, out=out)
    torch.cuda.synchronize()
    ms, k = qn.profile_read()["merge"]
    qn.profile_enable(False)
    # per-projection times from a second, separately profiled pass
    for L, q, A, B, out in sets:
        qn.profile_enable(True)
        for _ in range(iters):
            qn.merge(q, A, B, L.alpha, out=out)
        torch.cuda.synchronize()
        pms, pk = qn.profile_read()["merge"]
        qn.profile_enable(False)
        n = L.N * L.K
        nb = n // 64
        byts = n // 2 + nb + (nb + 255) // 256 * 4 + 2 * L.r * L.K + 2 * L.N * L.r + 2 * n
        us = pms / pk * 1e3
        per[L.name] = {"us": round(us, 2), "bytes": byts, "gbs": round(byts / (us * 1e-6) / 1e9, 1)}
        total_bytes += byts
    paired_us = ms / k * 1e3 * len(sets)
    gbs = total_bytes / (block_us * 1e-6) / 1e9
    del sets
    torch.cuda.empty_cache()
    return {"block_us": round(block_us, 2), "block_bytes": total_bytes, "gbs": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4), "block_us_per_call_event_pairs": round(paired_us, 2),
            "per_projection": per, "timing": "block: %d passes of the seven merges between one event pair; "
            "per projection: the library's event pair around each of %d calls" % (iters, iters),
            "bytes_per_element": "0.5 codes + 1/64 u8 scale + 2 bf16 out (+ A, B once)"}


STACK_DIMS = [4096, 14336, 4096, 4096]  # up_proj, down_proj and o_proj shapes, chained


def bench_stack(qn, torch, inputs, steps=5, warmup=2, m=4096):
    """Training step of a stack of QLoRA layers (forward, MSE loss, backward, AdamW on
    every adapter) on Llama-3-8B projection shapes 4096 -> 14336 -> 4096 -> 4096,
    4096 tokens, r = 64, bf16, NF4 block 64 with double quantization."""
    S = inputs.stack(STACK_DIMS, m, r=64, seed=5, alpha=128.0)
    layers = []
    for W, A, B in zip(S.Ws, S.As, S.Bs):
        q = qn.quantize(W.to("cuda"), 64, True, 256)
        layers.append(qn.StackLayer.create(q, A, B, torch.bfloat16))
    del S.Ws[:]
    x, t = S.x.to("cuda"), S.target.to("cuda")
    ws = torch.empty(qn.stack_workspace_bytes(layers, m, torch.bfloat16), dtype=torch.uint8, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    opt = dict(lr=1e-4, weight_decay=0.01)
    for k in range(warmup):
        qn.stack_train_step(layers, x, t, S.alpha, k + 1, workspace=ws, loss=loss, **opt)
    torch.cuda.synchronize()
    first = float(loss.item())
    t0 = time.perf_counter()
    for k in range(steps):
        qn.stack_train_step(layers, x, t, S.alpha, warmup + k + 1, workspace=ws, loss=loss, **opt)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    qn.profile_enable(True)  # per-kernel times from a separate profiled pass
    for k in range(steps):
        qn.stack_train_step(layers, x, t, S.alpha, warmup + steps + k + 1, workspace=ws, loss=loss, **opt)
    torch.cuda.synchronize()
    prof = qn.profile_read()
    qn.profile_enable(False)
    flops = 0.0
    for l, (K, N) in enumerate(zip(STACK_DIMS[:-1], STACK_DIMS[1:])):
        flops += fwd_flops(m, N, K, 64) + bwd_flops(m, N, K, 64) - (2.0 * m * N * K + 2.0 * m * 64 * K if l == 0 else 0)
    out = {"workload": "stack 4096-14336-4096-4096, 4096 tokens, r 64, bf16", "ms_per_step": round(sec * 1e3, 4),
           "tflops": round(flops / sec / 1e12, 2), "frac_bf16_peak": round(flops / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
           "loss_first_timed": first, "loss_last": float(loss.item()),
           "kernels_ms_per_step": {k: round(ms / steps, 4) for k, (ms, n) in prof.items() if n}}
    del layers, ws
    torch.cuda.empty_cache()
    return out


def copy_probe(torch, mib=512, iters=10):
    """A plain device copy of known size: the calibration run for the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) and the streaming ceiling of this GPU."""
    a = torch.ones(mib << 19, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / iters * 1e3
    return {"bytes_read": mib << 20, "bytes_written": mib << 20, "us": round(us, 2),
            "gbs": round(2 * (mib << 20) / (us * 1e-6) / 1e9, 1)}


# Counter records of HBM traffic per launch (calibrated FETCH_SIZE + WRITE_SIZE):
# the headline step's forward and dX GEMM launches, and the forward GEMM of the
# per-projection step.
TRAFFIC_FILES = {
    "grouped": os.path.join(ROOT, "profiles", "dense256_hbm_traffic_llama3_8b_block_grouped_fwd_step.md"),
    "per_projection": os.path.join(ROOT, "profiles", "dense256_fwd_hbm_traffic_llama3_8b_block.md"),
}
KERNEL_SOURCES = [os.path.join(ROOT, "bit_nf4_quantized_nibble_amd", "csrc", f) for f in ("gemm256.hip", "common.h")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kind, step):
    """HBM bytes per launch of kernel `kind` in `step` ("grouped" or
    "per_projection") from the committed counter runs (calibrated FETCH_SIZE +
    WRITE_SIZE), or None when there is no record or the kernel sources changed
    since the counters were taken."""
    try:
        vals = {}
        with open(TRAFFIC_FILES[step]) as fh:
            for line in fh:
                if line.startswith("traffic_") or line.startswith("kernel_source_hash"):
                    k, v = line.split(":", 1)
                    vals[k.strip()] = v.strip()
        if vals.get("kernel_source_hash") != kernel_source_hash():
            return None
        return int(float(vals["traffic_%s_bytes_per_launch" % kind]))
    except (OSError, KeyError, ValueError):
        return None


def bench_quant(qn, torch, inputs, copies=5, iters=20):
    """Quantize and dequantize of a 4096 x 4096 weight, cycling through `copies` copies
    (more bytes than the last-level cache).  `us`: `iters` back-to-back calls between one
    event pair on the stream, per call; `us_event_pairs`: the same calls with the
    library's event pair around each one (which adds the pair's own cost)."""
    W0 = inputs.roundtrip_weight(0).to("cuda")
    n = W0.numel()
    Ws = [W0.clone() for _ in range(copies)]
    out = {}

    def stream_us(call):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / iters
    for dq in (False, True):
        qs = [qn.empty_nf4(4096, 4096, 64, dq, 256) for _ in range(copies)]
        ds = [q.descriptor() for q in qs]
        lib = qn._lib.lib()
        stream = torch.cuda.current_stream().cuda_stream
        for i in range(copies):
            lib.qlora_nf4_quantize(Ws[i].data_ptr(), ctypes.byref(ds[i]), stream)
        torch.cuda.synchronize()

        def quant(i):
            rc = lib.qlora_nf4_quantize(Ws[i % copies].data_ptr(), ctypes.byref(ds[i % copies]), stream)
            if rc:
                raise RuntimeError("quantize rc %d" % rc)

        us = stream_us(quant)
        qn.profile_enable(True)
        for i in range(iters):
            quant(i)
        torch.cuda.synchronize()
        ms, k = qn.profile_read()["quantize"]
        qn.profile_enable(False)
        nb = n // 64
        byts = n * 4 + n // 2 + (nb + (nb + 255) // 256 * 4 if dq else nb * 4)
        gbs = byts / (us * 1e-6) / 1e9
        out["dq" if dq else "no_dq"] = {"us": round(us, 2), "bytes": byts, "gbs": round(gbs, 1),
                                        "frac": round(gbs / PEAK_HBM_GBS, 4),
                                        "us_event_pairs": round(ms / k * 1e3, 2)}
        if dq:
            for name, dt, ob in (("bf16", torch.bfloat16, 2), ("f32", torch.float32, 4)):
                outs = [torch.empty(4096, 4096, dtype=dt, device="cuda") for _ in range(copies)]
                code = qn.dtype_code(dt)
                for i in range(copies):
                    lib.qlora_nf4_dequantize(ctypes.byref(ds[i]), code, outs[i].data_ptr(), stream)
                torch.cuda.synchronize()

                def dequant(i):
                    rc = lib.qlora_nf4_dequantize(ctypes.byref(ds[i % copies]), code, outs[i % copies].data_ptr(),
                                                  stream)
                    if rc:
                        raise RuntimeError("dequantize rc %d" % rc)

                us = stream_us(dequant)
                qn.profile_enable(True)
                for i in range(iters):
                    dequant(i)
                torch.cuda.synchronize()
                ms, k = qn.profile_read()["dequantize"]
                qn.profile_enable(False)
                byts = n // 2 + nb + (nb + 255) // 256 * 4 + n * ob
                gbs = byts / (us * 1e-6) / 1e9
                out["dequant_dq_to_" + name] = {"us": round(us, 2), "bytes": byts, "gbs": round(gbs, 1),
                                                "frac": round(gbs / PEAK_HBM_GBS, 4),
                                                "us_event_pairs": round(ms / k * 1e3, 2)}
                del outs
        del qs
    del Ws, W0
    torch.cuda.empty_cache()
    return out


def cpu_baseline(inputs, target_s):
    """The oracle as it is (plain C, fp64, OpenMP over output rows) on a bounded
    sample of the step: forward + backward of q_proj for the first m_s tokens."""
    import numpy as np

    import oracle
    (L,) = inputs.prefill(seed=0, cd="bf16", with_dy=True, projections=["q_proj"])
    q = oracle.quantize(L.W.numpy(), 64, True, 256)
    W = oracle.weight_operand(q, "bf16")
    x, A, B, dY = (oracle.operand(t, "bf16") for t in (L.x, L.A, L.B, L.dY))
    s = L.alpha / L.r

    def run(ms):
        t0 = time.perf_counter()
        oracle.forward(x[:ms], W, A, B, s)
        oracle.backward(x[:ms], W, A, B, dY[:ms], s)
        return time.perf_counter() - t0

    probe = 8
    t = run(probe)
    ms = int(max(8, min(4096, probe * target_s / max(t, 1e-3))))
    t = run(ms)
    flops = fwd_flops(ms, L.N, L.K, L.r) + bwd_flops(ms, L.N, L.K, L.r)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(t, 2),
            "sample": "oracle forward + backward of q_proj (4096x4096, r=64) on the first %d of the "
                      "4096 tokens (%.1f GFLOP), fp64 scalar C with OpenMP" % (ms, flops / 1e9)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["step", "projstep", "fusedstep", "groupstep", "sharestep", "gemv", "decodeblock", "quant", "sweep",
                                       "merge", "stack", "copyprobe", "paths"],
                    default=None,
                    help="run one part (for profiling); the JSON line needs the full run")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the benchmark measures one GPU; --gpus %d is not supported "
              "(the layer would shard data-parallel over tokens)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_nf4_quantized_nibble_amd as qn
    from bit_nf4_quantized_nibble_amd import inputs
    lib = qn._lib.lib()
    torch.cuda.set_device(0)

    if args.only == "gemv":
        print(json.dumps(bench_gemv(qn, torch, lib, inputs)))
        return
    if args.only == "decodeblock":
        print(json.dumps(bench_decode_block(qn, torch, lib, inputs)))
        return
    if args.only == "copyprobe":
        print(json.dumps(copy_probe(torch)))
        return
    if args.only == "quant":
        print(json.dumps(bench_quant(qn, torch, inputs)))
        return
    if args.only == "sweep":
        print(json.dumps(bench_dtype_sweep(qn, torch, lib, inputs)))
        return
    if args.only == "merge":
        print(json.dumps(bench_merge(qn, torch, inputs)))
        return
    if args.only == "paths":
        print(json.dumps(bench_path_sweep(qn, torch, lib, inputs)))
        return
    if args.only == "stack":
        print(json.dumps(bench_stack(qn, torch, inputs)))
        return

    if args.only in ("fusedstep", "groupstep", "projstep", "sharestep"):
        grouped = {"groupstep": "both", "sharestep": "fwd"}.get(args.only, False)
        st = bench_step(args, qn, torch, lib, inputs, flags=qn._lib.QLORA_FLAG_FUSED if args.only == "fusedstep" else 0,
                        grouped=grouped, m=SHARE_TOKENS if args.only == "sharestep" else 4096)
        print(json.dumps({"ms_per_step": st["sec"] * 1e3, "kernels": st["kernels"], "roofline": st["roofline"]}))
        return
    hashes = {} if args.only is None else None
    st = bench_step(args, qn, torch, lib, inputs, hashes=hashes, grouped="fwd")
    log("step %.3f ms" % (st["sec"] * 1e3))
    if args.only == "step":
        print(json.dumps({"ms_per_step": st["sec"] * 1e3, "kernels": st["kernels"], "roofline": st["roofline"]}))
        return
    stp = bench_step(args, qn, torch, lib, inputs)
    log("per-projection step %.3f ms" % (stp["sec"] * 1e3))
    stf = bench_step(args, qn, torch, lib, inputs, flags=qn._lib.QLORA_FLAG_FUSED)
    log("fused step %.3f ms" % (stf["sec"] * 1e3))
    sts = bench_step(args, qn, torch, lib, inputs, grouped="fwd", m=SHARE_TOKENS)
    log("%d-token step %.3f ms" % (SHARE_TOKENS, sts["sec"] * 1e3))
    gemv = bench_gemv(qn, torch, lib, inputs)
    log("gemv done")
    gemv["decode_block"] = bench_decode_block(qn, torch, lib, inputs)
    log("decode block done")
    quant = bench_quant(qn, torch, inputs)
    log("quant done")
    sweep = bench_dtype_sweep(qn, torch, lib, inputs)
    log("sweep done")
    merge = bench_merge(qn, torch, inputs)
    log("merge done")
    stack = bench_stack(qn, torch, inputs)
    log("stack done")
    paths = bench_path_sweep(qn, torch, lib, inputs)
    log("path sweep done")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (~%.0f s)" % args.cpu_seconds)
        cpu = cpu_baseline(inputs, args.cpu_seconds)

    ms = st["sec"] * 1e3
    value = st["flops"] / st["sec"] / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qlora_nf4_block_train_step_llama3_8b_shapes",
                   "tokens": 4096, "projections": [[n, N, K] for n, N, K in st["layers"]],
                   "r": 64, "alpha": 128, "block_size": 64, "double_quant": True, "dq_group": 256,
                   "step": "forward of 7 projections (q/k/v and gate/up each one grouped call) + backward "
                           "(dX, dA, dB) per projection, library default path (dequantize-then-GEMM at 4096 tokens)",
                   "flops_per_step": st["flops"], "parallelism": "single GPU"},
        "frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "step_ms_device": st["step_ms"],
        "roofline": st["roofline"],
        "cpu_baseline": cpu,
        "kernels": st["kernels"],
        "fused_path_step": {"ms_per_step": round(stf["sec"] * 1e3, 4),
                            "tflops": round(stf["flops"] / stf["sec"] / 1e12, 2),
                            "frac_bf16_peak": round(stf["flops"] / stf["sec"] / 1e12 / PEAK_BF16_TFLOPS, 4),
                            "roofline": stf["roofline"], "kernels": stf["kernels"]},
        "per_projection_step": {"ms_per_step": round(stp["sec"] * 1e3, 4),
                                "tflops": round(stp["flops"] / stp["sec"] / 1e12, 2),
                                "frac_bf16_peak": round(stp["flops"] / stp["sec"] / 1e12 / PEAK_BF16_TFLOPS, 4),
                                "forward": "each projection its own qlora_linear_fwd call",
                                "backward": "per projection", "step_ms_device": stp["step_ms"],
                                "roofline": stp["roofline"], "kernels": stp["kernels"]},
        "share_step": {"tokens": SHARE_TOKENS, "ms_per_step": round(sts["sec"] * 1e3, 4),
                       "tflops": round(sts["flops"] / sts["sec"] / 1e12, 2),
                       "frac_bf16_peak": round(sts["flops"] / sts["sec"] / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "what": "the headline step at one GPU's share of an 8-way data-parallel 4096-token batch",
                       "step_ms_device": sts["step_ms"], "kernels": sts["kernels"]},
        "gemv": gemv,
        "quantize": quant,
        "dtype_sweep_forward": sweep,
        "merge": merge,
        "stack_train_step": stack,
        "fused_vs_dequant_forward": paths,
        "inputs_sha256": hashes,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
