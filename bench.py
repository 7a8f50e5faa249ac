#!/usr/bin/env python3
"""Throughput of the routed 4-bit MoE expert layer on one MI355X.

A step is one pass of the layer's hot path over one batch: route -> permute
(+ gather) -> grouped expert forward (gate_up + activation, down) -> combine.
The headline workload is the Qwen3-30B-A3B-shaped NF4 layer (E=128, top-8,
H=2048, I=768) at T=4096 tokens; `value` is routed tokens/s. Weights, tokens
and router logits are seeded synthetic tensors already resident in HBM.

The dominant kernel (the gate_up grouped GEMM at this size) is timed live with
HIP events that the library records around its launch on the step's stream,
and priced against the bf16 MFMA peak. The sweep adds the decode token counts
(weight GB/s against HBM peak) and the other workloads. The CPU oracle is timed
on a bounded sample of the same workload on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
HEADLINE_T = 4096


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ HIP events

class Hip:
    """hipEvent plumbing through the HIP runtime (the library records the
    events; bench.py only creates and reads them)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            rc = self.lib.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            arr[i] = ev.value
        return arr

    def ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return out.value

    def record(self, ev, stream):
        rc = self.lib.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")


# -------------------------------------------------------------- layer set-up

def nf4_layer(moe4, inputs, spec, layer, seed, torch):
    """NF4 stack quantised on the GPU from seeded fp32 source weights."""
    E, H, I = spec.E, spec.H, spec.I
    wg, wd = inputs.device_nf4_source(spec, layer, seed)
    dev = wg.device
    gq = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    gs = torch.empty((E, 2 * I, H // 64), dtype=torch.float32, device=dev)
    dq = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    ds = torch.empty((E, H, I // 64), dtype=torch.float32, device=dev)
    moe4.moe4_quantize_nf4(wg, gq, gs)
    moe4.moe4_quantize_nf4(wd, dq, ds)
    del wg, wd
    lora = {}
    if spec.lora_r:
        lora = dict(lora_A=inputs.device_bf16((E, spec.lora_r, H), 1.0 / H ** 0.5, seed, spec,
                                              layer, 11),
                    lora_B=inputs.device_bf16((E, 2 * I, spec.lora_r), 0.01, seed, spec, layer, 12),
                    lora_scale=spec.lora_scale)
    return moe4.Experts(moe4.MOE4_FMT_NF4, gq, gs, dq, ds, gu_layout=moe4.MOE4_GU_HALVES,
                        act=moe4.MOE4_ACT_SWIGLU, E=E, H=H, I=I, **lora)


def nf4_dq_layer(moe4, inputs, spec, layer, seed, torch):
    """NF4 stack whose absmax is double-quantised on the GPU (dynamic code book)."""
    base = nf4_layer(moe4, inputs, spec, layer, seed, torch)
    gq, gs, dq, ds = base.tensors[:4]
    dev = gq.device
    book = torch.from_numpy(inputs.dq_code_book("dynamic")).to(dev)
    ws = torch.empty(moe4.MOE4_DQ_WS_BYTES, dtype=torch.uint8, device=dev)
    parts = []
    for a in (gs, ds):
        n = a.numel()
        code = torch.empty(a.shape, dtype=torch.uint8, device=dev)
        a2 = torch.empty((n + 255) // 256, dtype=torch.float32, device=dev)
        off = torch.empty(1, dtype=torch.float32, device=dev)
        moe4.moe4_compress_absmax(a.reshape(-1), book, code, a2, off, ws)
        parts.append((code, a2, off))
    (gc, ga2, goff), (dc, da2, doff) = parts
    return moe4.Experts(moe4.MOE4_FMT_NF4_DQ, gq, gc, dq, dc, gu_layout=moe4.MOE4_GU_HALVES,
                        act=moe4.MOE4_ACT_SWIGLU, E=spec.E, H=spec.H, I=spec.I, gu_s2=ga2,
                        dn_s2=da2, gu_soff=goff, dn_soff=doff, dq_book=book)


def mxfp4_layer(moe4, inputs, spec, layer, seed, torch):
    E, H, I = spec.E, spec.H, spec.I
    gb, gsc, db, dsc = inputs.device_mxfp4_stack(spec, layer, seed)
    bias = {}
    if spec.bias:
        bias = dict(gu_bias=inputs.device_bf16((E, 2 * I), spec.bias_std, seed, spec, layer, 9),
                    dn_bias=inputs.device_bf16((E, H), spec.bias_std, seed, spec, layer, 10))
    if spec.lora_r:
        bias.update(lora_A=inputs.device_bf16((E, spec.lora_r, H), 1.0 / H ** 0.5, seed, spec,
                                              layer, 11),
                    lora_B=inputs.device_bf16((E, 2 * I, spec.lora_r), 0.01, seed, spec, layer, 12),
                    lora_scale=spec.lora_scale)
    return moe4.Experts(moe4.MOE4_FMT_MXFP4, gb, gsc, db, dsc,
                        gu_layout=(moe4.MOE4_GU_INTERLEAVED if spec.layout == "interleaved"
                                   else moe4.MOE4_GU_HALVES),
                        act=(moe4.MOE4_ACT_SWIGLU_CLAMPED if spec.act == "swiglu_clamped"
                             else moe4.MOE4_ACT_SWIGLU),
                        E=E, H=H, I=I, act_alpha=spec.alpha, act_limit=spec.limit, **bias)


def expert_bytes(spec):
    """Algorithmic weight bytes of one expert: (gate_up, down), packed nibbles
    plus scales plus bias rows."""
    H, I = spec.H, spec.I
    if spec.fmt == "nf4":
        gu = 2 * I * H // 2 + 2 * I * (H // 64) * 4
        dn = H * I // 2 + H * (I // 64) * 4
    elif spec.fmt == "nf4_dq":   # 1-byte absmax codes + one fp32 per 256 of them
        gu = 2 * I * H // 2 + 2 * I * (H // 64) + 2 * I * (H // 64) * 4 / 256
        dn = H * I // 2 + H * (I // 64) + H * (I // 64) * 4 / 256
    else:
        gu = 2 * I * H // 2 + 2 * I * (H // 32)
        dn = H * I // 2 + H * (I // 32)
    if spec.bias:
        gu += 2 * I * 2
        dn += H * 2
    return gu, dn


class Step:
    """Buffers for one (workload, T) and the calls of one step."""

    def __init__(self, moe4, torch, spec, T, ex, backward=False):
        self.moe4, self.torch, self.spec, self.T = moe4, torch, spec, T
        dev = "cuda"
        k, H, E = spec.k, spec.H, spec.E
        S = T * k
        i32, f32, bf = torch.int32, torch.float32, torch.bfloat16
        self.idx = torch.empty((T, k), dtype=i32, device=dev)
        self.w = torch.empty((T, k), dtype=f32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.sor = torch.empty(S, dtype=i32, device=dev)
        self.ros = torch.empty(S, dtype=i32, device=dev)
        self.x_perm = torch.empty((S, H), dtype=bf, device=dev)
        self.y_perm = torch.empty((S, H), dtype=f32, device=dev)
        self.out = torch.empty((T, H), dtype=bf, device=dev)
        self.ws = torch.empty(moe4.moe4_workspace_size(ex, T, k), dtype=torch.uint8, device=dev)
        self.backward = backward
        if backward:
            r = ex.lora_r
            self.save_gu = torch.empty((S, 2 * spec.I), dtype=f32, device=dev)
            self.save_xa = torch.empty((S, r), dtype=f32, device=dev) if r else None
            self.dy = torch.empty((S, H), dtype=bf, device=dev)
            self.dx_perm = torch.empty((S, H), dtype=f32, device=dev)
            self.dx = torch.empty((T, H), dtype=bf, device=dev)
            self.dA = torch.empty((E, r, H), dtype=f32, device=dev) if r else None
            self.dB = torch.empty((E, 2 * spec.I, r), dtype=f32, device=dev) if r else None

    def forward(self, ex, x, logits):
        m = self.moe4
        k = self.spec.k
        if not self.backward:
            # the gate_up GEMM gathers its rows from x itself: no x_perm round
            # trip through HBM and no gather work (1-2 us a decode step, 34 us
            # at 4096 Qwen3 tokens)
            m.moe4_route_permute(logits, k, self.idx, self.w, self.offsets, self.sor, self.ros,
                                 ws=self.ws)
            m.moe4_expert_forward_gather(ex, x, k, self.sor, self.offsets, self.y_perm,
                                         ws=self.ws)
            m.moe4_combine(self.y_perm, self.ros, self.w, self.out, k)
            return
        # the backward reads x_perm again: route + permute + gather once
        m.moe4_route_permute(logits, k, self.idx, self.w, self.offsets, self.sor,
                             self.ros, x=x, x_perm=self.x_perm, ws=self.ws)
        if self.backward:
            m.moe4_expert_forward(ex, self.x_perm, self.offsets, self.y_perm, save_gu=self.save_gu,
                                  save_xa=self.save_xa, ws=self.ws)
        else:
            m.moe4_expert_forward(ex, self.x_perm, self.offsets, self.y_perm, ws=self.ws)
        m.moe4_combine(self.y_perm, self.ros, self.w, self.out, self.spec.k)

    def backward_pass(self, ex, dout):
        m = self.moe4
        # dOut gathered by the forward's permutation, scaled by the routing weights
        m.moe4_gather_rows(dout, self.spec.k, self.sor, self.dy, row_scale=self.w.reshape(-1))
        m.moe4_expert_backward(ex, self.x_perm, self.offsets, self.save_gu, self.save_xa, self.dy,
                               self.dx_perm, self.dA, self.dB, ws=self.ws)
        m.moe4_combine(self.dx_perm, self.ros, None, self.dx, self.spec.k)


def touched(torch, moe4, step, ex, x, logits):
    """Distinct experts per step for the given logits (routing is deterministic)."""
    moe4.moe4_route(logits, step.spec.k, step.idx, step.w)
    torch.cuda.synchronize()
    return int(torch.unique(step.idx).numel())


# --------------------------------------------------------------------- timing

def pct(vals, q):
    v = sorted(vals)
    if not v:
        return None
    i = min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))
    return v[i]


def spread(vals, nd=4):
    """median, p10 and p90 of a list of per-step figures."""
    return {"median": round(pct(vals, 0.5), nd), "p10": round(pct(vals, 0.1), nd),
            "p90": round(pct(vals, 0.9), nd)}


def time_steps(torch, hip, moe4, steps, warmup, run, nkern=2):
    """Run `run(i)` warmup + steps times; the timed region (steps warmup ..
    warmup + steps - 1) is bracketed by a synchronisation and an event on each
    side, with nothing recorded inside it. The same steps then run once more
    with an event at every step boundary and the library's events around each
    of the (up to two) GEMM launches of every step: the per-step spread and the
    per-launch durations. (Each event record costs the stream a few
    microseconds, about 3% of a T=4096 step, so the step time comes from the
    first pass.) Returns (region ms / steps, per-step ms of the second pass,
    [per-step ms of GEMM j])."""
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    ends = hip.events(2)
    hip.record(ends[0], stream)
    for i in range(steps):
        run(warmup + i)
    hip.record(ends[1], stream)
    torch.cuda.synchronize()
    total = hip.ms(ends[0], ends[1])
    kev = hip.events(4 * steps)
    bounds = hip.events(steps + 1)
    per_step = [(ctypes.c_void_p * 4)(*kev[4 * i:4 * i + 4]) for i in range(steps)]
    for i in range(steps):
        hip.record(bounds[i], stream)
        moe4.moe4_set_timing_events(per_step[i])
        run(warmup + i)
    moe4.moe4_set_timing_events(None)
    hip.record(bounds[steps], stream)
    torch.cuda.synchronize()
    step_ms = [hip.ms(bounds[i], bounds[i + 1]) for i in range(steps)]
    kms = [[hip.ms(kev[4 * i + 2 * j], kev[4 * i + 2 * j + 1]) for i in range(steps)]
           for j in range(nkern)]
    return total / steps, step_ms, kms


# ----------------------------------------------------------------- workloads

def bench_layer(torch, hip, moe4, inputs, spec, T, exs, steps, warmup, seed, settle=None):
    """Forward steps of one workload at T tokens. Every repetition (warm-up
    included) has its own routing draw (fresh tokens and logits), and the
    layer replicas rotate, so decode-sized steps read cold weights. settle (or
    None): called with a callable that runs one step on this step's buffers,
    before the timed region; its result is returned as the third value."""
    step = Step(moe4, torch, spec, T, exs[0])
    n = warmup + steps
    toks = [inputs.device_tokens(spec, T, layer=li % spec.layers if spec.layers > 1 else 0,
                                 seed=seed + 1000 + li)
            for li in range(n)]
    nrep = len(exs)
    counts = [touched(torch, moe4, step, exs[0], *toks[i]) for i in range(n)]
    settled = settle(lambda: step.forward(exs[0], *toks[0])) if settle else None

    def run(i):
        x, lg = toks[i]
        step.forward(exs[i % nrep], x, lg)

    ms, step_ms, (k_gu, k_dn) = time_steps(torch, hip, moe4, steps, warmup, run)
    gu_b, dn_b = expert_bytes(spec)
    ntouch = [counts[warmup + i] for i in range(steps)]
    S = T * spec.k
    flops_gu = 2.0 * S * 2 * spec.I * spec.H
    flops_dn = 2.0 * S * spec.H * spec.I
    gemm = [a + b for a, b in zip(k_gu, k_dn)]
    wbps = [nt * (gu_b + dn_b) / (g * 1e-3) / 1e9 for nt, g in zip(ntouch, gemm)]
    gubps = [nt * gu_b / (g * 1e-3) / 1e9 for nt, g in zip(ntouch, k_gu)]
    tfl = [(flops_gu + flops_dn) / (g * 1e-3) / 1e12 for g in gemm]
    gutfl = [flops_gu / (g * 1e-3) / 1e12 for g in k_gu]
    res = {
        "workload": spec.name, "T": T, "steps": steps, "replicas": nrep,
        "ms_per_step": round(ms, 5), "step_ms": spread(step_ms, 5),
        "routed_tokens_per_s": round(T / (ms / 1e3), 1),
        # the median step (robust to a host stall inside the timed region)
        "routed_tokens_per_s_median": round(T / (pct(step_ms, 0.5) / 1e3), 1),
        "kernel": moe4.moe4_last_variant() == moe4.MOE4_VARIANT_SKINNY and "skinny" or "tiled",
        "gate_up_us": spread([v * 1e3 for v in k_gu], 2),
        "down_us": spread([v * 1e3 for v in k_dn], 2),
        "touched_experts": round(sum(ntouch) / steps, 2),
        "weight_GBps": spread(wbps, 1), "gate_up_weight_GBps": spread(gubps, 1),
        "tflops": spread(tfl, 2), "gate_up_tflops": spread(gutfl, 2),
    }
    res["hbm_frac"] = round(res["weight_GBps"]["median"] / HBM_PEAK_GBS, 4)
    res["mfma_frac"] = round(res["tflops"]["median"] / BF16_PEAK_TFLOPS, 4)
    if T < 1024:
        # the same timed steps (each with its own routing draw and replica)
        # captured back to back into one HIP graph and replayed: the step time
        # a serving loop sees without host launch overhead
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(steps):
                run(warmup + i)
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream().cuda_stream
        ev = hip.events(6)
        rep = []
        for r in range(3):
            hip.record(ev[2 * r], stream)
            g.replay()
            hip.record(ev[2 * r + 1], stream)
        torch.cuda.synchronize()
        rep = sorted(hip.ms(ev[2 * r], ev[2 * r + 1]) / steps for r in range(3))
        del g
        res["graph_ms_per_step"] = round(rep[1], 5)
        res["graph_routed_tokens_per_s"] = round(T / (rep[1] / 1e3), 1)
    k_gu_mean = sum(k_gu) / steps
    return res, (k_gu_mean, flops_gu, sum(ntouch) / steps * gu_b), settled


def bench_backward(torch, hip, moe4, inputs, spec, T, ex, steps, warmup, seed):
    step = Step(moe4, torch, spec, T, ex, backward=True)
    x, lg = inputs.device_tokens(spec, T, seed=seed + 77)
    dout = inputs.device_bf16((T, spec.H), 1.0, seed, spec, 0, 13)

    def run_f(i):
        step.forward(ex, x, lg)

    def run_b(i):
        step.backward_pass(ex, dout)

    # the step's own buffers touched by the GPU before the timed regions
    for _ in range(3):
        run_f(0)
        run_b(0)
    torch.cuda.synchronize()

    f_ms, f_steps, (f_gu, f_dn) = time_steps(torch, hip, moe4, steps, warmup, run_f)
    b_ms, b_steps, (b_dn, b_gu) = time_steps(torch, hip, moe4, steps, warmup, run_b)
    med = lambda v: pct(v, 0.5)
    f_gu, f_dn, b_dn, b_gu = med(f_gu), med(f_dn), med(b_dn), med(b_gu)
    S = T * spec.k
    H, I, r = spec.H, spec.I, spec.lora_r
    f_flops = 2.0 * S * (2 * I * H + H * I)
    lora_f = 2.0 * S * (r * H + 2 * I * r)
    b_flops = 2.0 * S * (H * I + 2 * I * H)
    lora_b = 2.0 * S * (2 * I * r + r * H) + 2.0 * S * (2 * I * r + r * H)
    tot = f_flops + lora_f + b_flops + lora_b
    return {
        "workload": spec.name, "T": T, "forward_ms": round(f_ms, 4), "backward_ms": round(b_ms, 4),
        "forward_step_ms": spread(f_steps, 4), "backward_step_ms": spread(b_steps, 4),
        "fwd_bwd_ms": round(f_ms + b_ms, 4),
        "fwd_bwd_tflops_step": round(tot / ((f_ms + b_ms) * 1e-3) / 1e12, 2),
        "fwd_gemm_tflops": round(f_flops / ((f_gu + f_dn) * 1e-3) / 1e12, 2),
        "bwd_dgrad_tflops": round(b_flops / ((b_gu + b_dn) * 1e-3) / 1e12, 2),
        "gemm_us": {"fwd_gate_up": round(f_gu * 1e3, 1), "fwd_down": round(f_dn * 1e3, 1),
                    "bwd_down_dgrad": round(b_dn * 1e3, 1), "bwd_gate_up_dgrad": round(b_gu * 1e3, 1)},
        "mfma_frac_step": round(tot / ((f_ms + b_ms) * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
    }


def bench_stack(torch, hip, moe4, inputs, spec, T, exs, steps, warmup, seed):
    """36-layer stack, layers back to back with independent inputs per layer."""
    L = len(exs)
    step = Step(moe4, torch, spec, T, exs[0])
    toks = [inputs.device_tokens(spec, T, layer=l, seed=seed + 500) for l in range(L)]
    counts = [touched(torch, moe4, step, exs[l], *toks[l]) for l in range(L)]

    def run(i):
        for l in range(L):
            x, lg = toks[l]
            step.forward(exs[l], x, lg)

    # the hook times the last layer's kernels of each pass; the region is the stack
    ms, pass_ms, _ = time_steps(torch, hip, moe4, steps, warmup, run)
    # the same pass captured once in a HIP graph and replayed: the library
    # launches on the current stream and allocates or synchronises nothing, so
    # the calls of every layer capture as they are and the host launch gaps disappear
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run(0)
    for _ in range(warmup):
        graph.replay()
    stream = torch.cuda.current_stream().cuda_stream
    marks = hip.events(steps + 1)
    torch.cuda.synchronize()
    for i in range(steps):
        hip.record(marks[i], stream)
        graph.replay()
    hip.record(marks[steps], stream)
    torch.cuda.synchronize()
    ms_graph = hip.ms(marks[0], marks[steps]) / steps
    graph_ms = [hip.ms(marks[i], marks[i + 1]) for i in range(steps)]
    del graph
    gu_b, dn_b = expert_bytes(spec)
    total_bytes = sum(counts) * (gu_b + dn_b)
    return {"workload": spec.name, "T": T, "layers": L,
            "stack_ms": round(ms, 4), "stack_ms_graph": round(ms_graph, 4),
            "stack_ms_spread": spread(pass_ms, 4), "stack_ms_graph_spread": spread(graph_ms, 4),
            "stack_weight_GBps_graph": round(total_bytes / (ms_graph * 1e-3) / 1e9, 1),
            "per_layer_us": round(ms * 1e3 / L, 2),
            "touched_experts_per_layer": round(sum(counts) / L, 2),
            "stack_weight_GB": round(total_bytes / 1e9, 4),
            "stack_weight_GBps_end_to_end": round(total_bytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac_end_to_end": round(total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def bench_convert(torch, hip, moe4, inputs, spec, steps, warmup, seed, nrep=2):
    """MXFP4 -> NF4 re-quantisation of whole gate_up and down stacks (two
    launches per pass), alternating between independently seeded layers so
    that every pass reads cold bytes. Bytes = MXFP4 in + NF4 out."""
    stream = torch.cuda.current_stream().cuda_stream
    layers = []
    for li in range(nrep):
        gb, gsc, db, dsc = inputs.device_mxfp4_stack(spec, li, seed)
        outs = []
        for b, sc in ((gb, gsc), (db, dsc)):
            R, K = sc.numel() // sc.shape[-1], sc.shape[-1] * 32
            outs.append((b, sc, torch.empty((R, K // 2), dtype=torch.uint8, device=b.device),
                         torch.empty((R, K // 64), dtype=torch.float32, device=b.device)))
        layers.append(outs)

    def run(i):
        for b, sc, p, a in layers[i % nrep]:
            moe4.moe4_convert_mxfp4_nf4(b, sc, p, a)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    ev = hip.events(2 * steps)
    for i in range(steps):
        hip.record(ev[2 * i], stream)
        run(warmup + i)
        hip.record(ev[2 * i + 1], stream)
    torch.cuda.synchronize()
    ms = sorted(hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(steps))
    med = ms[len(ms) // 2]
    nbytes = sum(b.numel() + sc.numel() + p.numel() + 4 * a.numel()
                 for b, sc, p, a in layers[0])
    gbps = nbytes / (med * 1e-3) / 1e9
    return {"workload": f"{spec.name} MXFP4->NF4 conversion", "stacks": "gate_up + down",
            "weights": int(sum(p.numel() * 2 for _, _, p, _ in layers[0])),
            "bytes_in_out": int(nbytes), "ms": round(med, 4), "GBps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBS, 4)}


def bench_router(torch, hip, moe4, inputs, spec, T, steps, warmup, seed):
    """Router step at the layer's shape: logits (x W_r^T, fp32) and the routing
    backward (dw and d logits from dOut and the slots' expert outputs)."""
    stream = torch.cuda.current_stream().cuda_stream
    x, _ = inputs.device_tokens(spec, T, seed=seed + 31)
    wr, rb = inputs.device_router(spec, seed=seed)
    E, k, H = spec.E, spec.k, spec.H
    lg = torch.empty((T, E), dtype=torch.float32, device=x.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=x.device)
    sor = torch.empty(T * k, dtype=torch.int32, device=x.device)
    ros = torch.empty(T * k, dtype=torch.int32, device=x.device)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=x.device)
    moe4.moe4_router_logits(x, wr, lg)
    moe4.moe4_route(lg, k, idx, w)
    moe4.moe4_permute(idx, E, offsets, sor, ros, ws=ws)
    y = inputs.device_bf16((T * k, H), 1.0, seed, spec, 0, 16).float()
    dout = inputs.device_bf16((T, H), 1.0, seed, spec, 0, 13)
    dw = torch.empty((T, k), dtype=torch.float32, device=x.device)
    dl = torch.empty((T, E), dtype=torch.float32, device=x.device)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = hip.events(2 * steps)
        for i in range(steps):
            hip.record(ev[2 * i], stream)
            fn()
            hip.record(ev[2 * i + 1], stream)
        torch.cuda.synchronize()
        ms = sorted(hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(steps))
        return ms[len(ms) // 2]

    f_ms = timed(lambda: moe4.moe4_router_logits(x, wr, lg))
    flips = flip_floor(torch, moe4, x, wr, rb if spec.zipf else None, k)
    b_ms = timed(lambda: moe4.moe4_route_backward(idx, w, dout, y, ros, dw, dl))
    f_bytes = T * H * 2 + E * H * 2 + T * E * 4
    b_bytes = T * k * H * 4 + T * H * 2 + T * k * 12 + T * E * 4
    return {"workload": f"{spec.name} router step", "T": T,
            "logits_us": round(f_ms * 1e3, 2),
            "logits_tflops": round(2.0 * T * E * H / (f_ms * 1e-3) / 1e12, 2),
            "logits_GBps": round(f_bytes / (f_ms * 1e-3) / 1e9, 1),
            "route_backward_us": round(b_ms * 1e3, 2),
            "route_backward_GBps": round(b_bytes / (b_ms * 1e-3) / 1e9, 1),
            "route_backward_hbm_frac": round(b_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "routing_flip_floor": flips}


def flip_floor(torch, moe4, x, wr, bias, k):
    """Share of tokens whose top-k expert set on the GPU's fp32 router logits
    differs from the top-k set of the exact logits rounded to fp32 (the exact
    sums by a float64 matrix product on the host)."""
    T, E = x.shape[0], wr.shape[0]
    lg = torch.empty((T, E), dtype=torch.float32, device=x.device)
    moe4.moe4_router_logits(x, wr, lg, bias=bias)
    torch.cuda.synchronize()
    exact = x.double().cpu() @ wr.double().cpu().T
    if bias is not None:
        exact += bias.double().cpu()[None, :]
    got = lg.cpu()
    a = torch.topk(got, k, dim=1).indices.sort(dim=1).values
    b = torch.topk(exact.float(), k, dim=1).indices.sort(dim=1).values
    n = int((a != b).any(dim=1).sum())
    return {"tokens": T, "flipped": n, "fraction": round(n / T, 6),
            "exact_logits": "float64 host matmul of the same bf16 x and W_r, rounded to fp32"}


def ceilings(torch, hip):
    """Practical HBM ceiling of this part: a plain copy (torch copy_ of 2 GiB
    float32: every byte read once and written once), median of 10."""
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    a = torch.empty(1 << 29, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for name, fn, nbytes in (("copy", lambda: b.copy_(a), 2 * a.numel() * 4),):
        for _ in range(3):
            fn()
        ev = hip.events(2 * 10)
        torch.cuda.synchronize()
        for i in range(10):
            hip.record(ev[2 * i], stream)
            fn()
            hip.record(ev[2 * i + 1], stream)
        torch.cuda.synchronize()
        ms = pct([hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(10)], 0.5)
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBS, 4),
                     "bytes": nbytes}
    del a, b
    torch.cuda.empty_cache()
    out["what"] = "torch copy_ of 2 GiB fp32 (every byte read once and written once)"
    return out


def device_state(torch=None, busy=None):
    """Clocks and power as rocm-smi reports them (None where unavailable). With
    busy (a callable issuing GPU work), rocm-smi is sampled from a second thread
    while the GPU runs it for about two seconds, so the clocks are the loaded
    ones."""
    import subprocess
    import threading
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        # under rocprofv3 its preloaded library would initialise the GPU in the
        # rocm-smi child before that child starts its interpreter: the GPU runs
        # the work all the same (the traced run times what the plain run times)
        if busy is not None:
            t0 = time.time()
            while time.time() - t0 < 2.5:
                for _ in range(20):
                    busy()
                torch.cuda.synchronize()
        return {"sampled": "not sampled (run under the profiler)"}
    got = {}

    def sample():
        time.sleep(0.8)
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--showmaxpower", "--showpower",
                                "--json"], capture_output=True, text=True, timeout=30)
            if r.returncode == 0 and r.stdout.strip():
                got["rec"] = json.loads(r.stdout)
        except Exception:
            pass

    th = threading.Thread(target=sample)
    th.start()
    if busy is not None:
        t0 = time.time()
        while time.time() - t0 < 2.5 and th.is_alive():
            for _ in range(20):
                busy()
            torch.cuda.synchronize()
    th.join()
    rec = got.get("rec")
    if not rec:
        return None
    card = rec.get("card0", next(iter(rec.values()), {}))
    keep = {"sampled": "while the GPU ran the headline step" if busy else "idle"}
    for key, val in card.items():
        lk = key.lower()
        if any(w in lk for w in ("sclk", "mclk", "fclk", "power", "socclk")):
            keep[key] = val
    return keep


# -------------------------------------------------------------- CPU baseline

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_layer_phases(oracle, spec, x, lg, W):
    """The oracle's forward of one batch, step by step (the same calls its
    layer_forward makes), timed per phase: route + permute, per-expert
    dequantisation, per-expert matmuls and activation, combine."""
    import numpy as np
    t = {}
    t0 = time.perf_counter()
    ri, rw = oracle.route(lg, spec.k)
    offsets, slot_of_row, row_of_slot = oracle.permute(ri, spec.E)
    t["route_permute_s"] = time.perf_counter() - t0
    xf = oracle.bf16_bits_to_f64(x)
    y = np.zeros((x.shape[0] * spec.k, spec.H))
    deq = mm = 0.0
    for e in range(spec.E):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            continue
        t0 = time.perf_counter()
        W.expert(e)
        t1 = time.perf_counter()
        gu, _ = oracle.gate_up(xf[slot_of_row[a:b] // spec.k], W, e)
        h = oracle.bf16_round_f64(oracle.activation(gu, W))
        y[a:b] = oracle.down(h, W, e)
        t2 = time.perf_counter()
        deq += t1 - t0
        mm += t2 - t1
    t["dequantise_s"], t["matmul_activation_s"] = deq, mm
    t0 = time.perf_counter()
    oracle.combine(y, row_of_slot, rw, x.shape[0], spec.k)
    t["combine_s"] = time.perf_counter() - t0
    return t


def cpu_baseline(spec, T_batch, n_tokens, tiny, seed=0):
    """The CPU oracle, untuned, on a bounded sample of the headline workload:
    n_tokens tokens of a T_batch batch through route -> permute -> expert
    forward (dequantise + matmul per touched expert) -> combine, timed per
    phase, with numpy's BLAS threads set to the cores this process may use.
    Also the whole tiny layer (median of 3) on those cores and on one."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from bit_mixture_experts_amd import inputs
    cores = len(os.sched_getaffinity(0))

    def nf4_weights(sp, experts, phases):
        E, H, I = sp.E, sp.H, sp.I
        gq = np.zeros((E, 2 * I, H // 2), np.uint8)
        ga = np.zeros((E, 2 * I, H // 64), np.float32)
        dq = np.zeros((E, H, I // 2), np.uint8)
        da = np.zeros((E, H, I // 64), np.float32)
        t0 = time.perf_counter()
        for e in experts:
            wg, wd = inputs.host_nf4_source(sp, e, 0, seed)
            p, a = oracle.quantize_nf4(wg.reshape(-1))
            gq[e], ga[e] = p.reshape(2 * I, H // 2), a.reshape(2 * I, H // 64)
            p, a = oracle.quantize_nf4(wd.reshape(-1))
            dq[e], da[e] = p.reshape(H, I // 2), a.reshape(H, I // 64)
        phases["quantise_s"] = time.perf_counter() - t0
        return oracle.ExpertWeights.from_nf4(gq, ga, dq, da, layout=sp.layout, act=sp.act)

    with threadpool_limits(cores):
        x, lg = inputs.host_tokens(spec, T_batch, seed=seed)
        x, lg = x[:n_tokens], lg[:n_tokens]
        idx, _ = oracle.route(lg, spec.k)
        need = sorted(set(int(e) for e in idx.reshape(-1)))
        ph = {}
        W = nf4_weights(spec, need, ph)
        ph.update(oracle_layer_phases(oracle, spec, x, lg, W))
    layer_s = sum(v for k, v in ph.items() if k != "quantise_s")
    tiny_res = {}
    tx, tlg = inputs.host_tokens(tiny, tiny.tokens[0], seed=seed)
    for threads in (cores, 1):
        with threadpool_limits(threads):
            runs = []
            for _ in range(3):
                p = {}
                Wt = nf4_weights(tiny, range(tiny.E), p)
                p.update(oracle_layer_phases(oracle, tiny, tx, tlg, Wt))
                runs.append(p)
            tot = sorted(sum(v for k, v in p.items() if k != "quantise_s") for p in runs)
            tiny_res[f"{threads}_threads"] = {
                "layer_s_median": round(tot[1], 4),
                "routed_tokens_per_s": round(tiny.tokens[0] / tot[1], 1),
                "phases_s": {k: round(sorted(p[k] for p in runs)[1], 4) for k in runs[0]}}
    return {"value": round(n_tokens / layer_s, 3), "unit": "routed tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"{n_tokens} tokens of the T={T_batch} {spec.name} batch "
                       f"({len(need)} experts touched): route, permute, per-expert NF4 "
                       f"dequantise + float64 matmul, combine; {layer_s:.1f} s "
                       f"(quantising the touched experts on the host, not counted: "
                       f"{ph['quantise_s']:.1f} s)"),
            "cpu_model": cpu_model(), "blas_threads": cores,
            "phases_s": {k: round(v, 3) for k, v in ph.items()},
            "tiny_layer": {"workload": f"{tiny.name} T={tiny.tokens[0]}", **tiny_res}}


PMC_TAG = "gate_up_tiled_nf4_qwen3_T4096"
HEADLINE_KERNEL = "k_tiled<1, true, true>"   # the gate_up grouped GEMM, NF4, tiled, rows gathered
CALIB_BYTES = 256 << 20                    # the copy kernel reads and writes this much
CALIB_KERNEL = "neg"                       # torch.neg on float32: one read, one write


def traffic_from_profile(kernel_tag=PMC_TAG):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel_tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("csrc_sha256") != csrc_digest():
        return None
    return rec.get("bytes_per_launch")


def calibration_copy(torch):
    """A plain copy of known size for scaling the FETCH_SIZE / WRITE_SIZE
    counters: torch.neg over CALIB_BYTES of float32 reads and writes each byte
    once."""
    a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def pmc_summary(fetch_db, write_db, out_dir):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
    `bench.py --no-sweep --no-cpu-baseline --calibrate` into the per-launch HBM
    traffic of the headline kernel, scaled by the calibration copy."""
    import sqlite3

    def per_kernel(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute("select name, dispatch_id, counter_value from pmc_events "
                           "where counter_name = ?", (counter,)).fetchall()
        con.close()
        head = [v for n, _, v in rows if HEADLINE_KERNEL in n]
        cal = [v for n, _, v in rows if CALIB_KERNEL in n and "moe4" not in n]
        if not head or not cal:
            raise SystemExit(f"{db}: no {counter} rows for the headline or calibration kernel")
        return sum(head) / len(head), sum(cal) / len(cal), len(head), len(cal)

    f_head, f_cal, nf, ncf = per_kernel(fetch_db, "FETCH_SIZE")
    w_head, w_cal, nw, ncw = per_kernel(write_db, "WRITE_SIZE")
    f_scale = CALIB_BYTES / (f_cal * 1024.0)
    w_scale = CALIB_BYTES / (w_cal * 1024.0)
    fetch_b = f_head * 1024.0 * f_scale
    write_b = w_head * 1024.0 * w_scale
    rec = {
        "kernel": HEADLINE_KERNEL, "workload": "qwen3_30b_a3b_nf4 E=128 k=8 H=2048 I=768 T=4096",
        "fetch_kib_per_launch_raw": round(f_head, 1), "write_kib_per_launch_raw": round(w_head, 1),
        "calibration": {"kernel": "torch.neg float32", "bytes_read": CALIB_BYTES,
                        "bytes_written": CALIB_BYTES, "fetch_kib_raw": round(f_cal, 1),
                        "write_kib_raw": round(w_cal, 1), "fetch_scale": round(f_scale, 4),
                        "write_scale": round(w_scale, 4)},
        "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
        "bytes_per_launch": round(fetch_b + write_b),
        "launches": {"fetch": nf, "write": nw, "calibration": [ncf, ncw]},
        "csrc_sha256": csrc_digest(),
    }
    path = os.path.join(out_dir, f"pmc_{PMC_TAG}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def csrc_digest():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_mixture_experts_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()


# ----------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=8,
                    help="independently seeded layer replicas resident for the decode rows")
    ap.add_argument("--decode-reps", type=int, default=60,
                    help="timed repetitions of each decode-sized row (each its own routing draw)")
    ap.add_argument("--tokens", default="",
                    help="comma list of token counts to keep in the per-layer sweeps")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=128)
    ap.add_argument("--only", default="", help="comma list of sweep parts: qwen,gptoss,lora,dq,router,convert,stack")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run the copy kernel of known size (for PMC scaling)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write profiles/pmc_*.json from two rocprofv3 --pmc result databases")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], os.path.join(ROOT, "profiles"))
        return
    if args.gpus != 1:
        print("bench.py measures a single GPU: the layer runs on one device here, with no "
              "sharding or collectives; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_mixture_experts_amd import inputs, moe4
    hip = Hip()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs")

    if args.calibrate:
        calibration_copy(torch)
    spec = inputs.QWEN3_30B_NF4
    t0 = time.time()
    exs = [nf4_layer(moe4, inputs, spec, r, args.seed, torch) for r in range(args.replicas)]
    torch.cuda.synchronize()
    log(f"qwen3-shaped NF4 replicas ready ({time.time() - t0:.1f} s)")

    # clocks and power are sampled while the GPU runs the headline step on the
    # timed loop's own buffers (about 2.5 s of it, before the timed region:
    # the timed steps see the settled clock and buffers the GPU has touched;
    # from a cold start the first ~25 steps run up to 10% slower)
    head, (k_gu, flops_gu, _), state = bench_layer(
        torch, hip, moe4, inputs, spec, HEADLINE_T, exs, args.steps, args.warmup, args.seed,
        settle=lambda busy: device_state(torch, busy))
    log("device state:", json.dumps(state))
    log("headline:", json.dumps(head))
    achieved = flops_gu / (k_gu * 1e-3) / 1e12
    traffic = traffic_from_profile()
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": "gate_up grouped GEMM (tiled, NF4, rows gathered from x)",
                "avg_launch_us": round(k_gu * 1e3, 2)}

    sweep = []
    only = set(filter(None, args.only.split(",")))
    keep_t = set(int(t) for t in args.tokens.split(",") if t)
    want = lambda T: not keep_t or T in keep_t
    dreps = max(50, args.decode_reps)
    def prime(busy):
        # a prefill row's own buffers touched by the GPU before its timed region
        for _ in range(10):
            busy()
        torch.cuda.synchronize()

    if not args.no_sweep:
        reps = max(10, args.steps)
        if not only or "qwen" in only:
            for T in (1, 16, 128):
                if want(T):
                    r, _, _ = bench_layer(torch, hip, moe4, inputs, spec, T, exs, dreps,
                                          args.warmup, args.seed)
                    log("sweep:", json.dumps(r))
                    sweep.append(r)
            sweep.append(head)
        if not only or "gptoss" in only:
            g = inputs.GPT_OSS_20B_MXFP4
            gex = [mxfp4_layer(moe4, inputs, g, r, args.seed, torch) for r in range(args.replicas)]
            for T in g.tokens:
                if want(T):
                    r, _, _ = bench_layer(torch, hip, moe4, inputs, g, T, gex,
                                          dreps if T < 1024 else reps, args.warmup, args.seed,
                                          settle=prime if T >= 1024 else None)
                    log("sweep:", json.dumps(r))
                    sweep.append(r)
            del gex
        if not only or "lora" in only:
            lspec = inputs.QWEN3_30B_NF4_LORA
            lex = nf4_layer(moe4, inputs, lspec, 0, args.seed, torch)
            r = bench_backward(torch, hip, moe4, inputs, lspec, lspec.tokens[0], lex, reps,
                               args.warmup, args.seed)
            log("sweep:", json.dumps(r))
            sweep.append(r)
            del lex
            mspec = inputs.GPT_OSS_20B_MXFP4_LORA
            mex = mxfp4_layer(moe4, inputs, mspec, 0, args.seed, torch)
            r = bench_backward(torch, hip, moe4, inputs, mspec, mspec.tokens[0], mex, reps,
                               args.warmup, args.seed)
            log("sweep:", json.dumps(r))
            sweep.append(r)
            del mex
        if not only or "dq" in only:
            dspec = spec.scaled(fmt="nf4_dq", name=spec.name + "_absmax_dq")
            dex = [nf4_dq_layer(moe4, inputs, spec, r, args.seed, torch)
                   for r in range(args.replicas)]
            for T in (1, 16, 128, HEADLINE_T):
                if want(T):
                    r, _, _ = bench_layer(torch, hip, moe4, inputs, dspec, T, dex,
                                          dreps if T < HEADLINE_T else reps, args.warmup,
                                          args.seed, settle=prime if T >= 1024 else None)
                    log("sweep:", json.dumps(r))
                    sweep.append(r)
            del dex
        if not only or "router" in only:
            r = bench_router(torch, hip, moe4, inputs, spec, HEADLINE_T, reps, args.warmup,
                             args.seed)
            log("sweep:", json.dumps(r))
            sweep.append(r)
        if not only or "convert" in only:
            r = bench_convert(torch, hip, moe4, inputs, inputs.GPT_OSS_20B_MXFP4, reps,
                              args.warmup, args.seed)
            log("sweep:", json.dumps(r))
            sweep.append(r)
        if not only or "stack" in only:
            s5 = inputs.GPT_OSS_120B_STACK
            t0 = time.time()
            sex = [mxfp4_layer(moe4, inputs, s5, l, args.seed, torch) for l in range(s5.layers)]
            torch.cuda.synchronize()
            log(f"36-layer MXFP4 stack ready ({time.time() - t0:.1f} s)")
            for T in s5.tokens:
                if want(T):
                    r = bench_stack(torch, hip, moe4, inputs, s5, T, sex, max(5, reps // 2),
                                    2, args.seed)
                    log("sweep:", json.dumps(r))
                    sweep.append(r)
            del sex
            xs, _ = inputs.device_tokens(s5, 32, seed=args.seed + 31)
            wr5, rb5 = inputs.device_router(s5, seed=args.seed)
            r = {"workload": f"{s5.name} router step", "T": 32,
                 "routing_flip_floor": flip_floor(torch, moe4, xs, wr5, rb5, s5.k)}
            log("sweep:", json.dumps(r))
            sweep.append(r)
        torch.cuda.empty_cache()
    ceil = ceilings(torch, hip)
    log("ceilings:", json.dumps(ceil))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(spec, HEADLINE_T, args.cpu_tokens, inputs.TINY_NF4, args.seed)
        log("cpu_baseline:", json.dumps(cpu))

    line = {
        "metric": "routed tokens/s + effective 4-bit weight GB/s (decode) / TFLOP/s (prefill), 1 GPU",
        "value": head["routed_tokens_per_s"], "unit": "routed tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{spec.name} T={HEADLINE_T}", "T": HEADLINE_T, "E": spec.E,
                   "top_k": spec.k, "H": spec.H, "I": spec.I, "format": "nf4",
                   "replicas": args.replicas,
                   "device": f"{props.name or 'AMD GPU'} {getattr(props, 'gcnArchName', '')}".strip()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_ceilings": ceil,
        "device_state": state,
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
