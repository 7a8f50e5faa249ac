"""Shared plumbing for the GPU parity tests: moving seeded inputs to the
device, running the layer through the C ABI, and comparing with the oracle.
Nothing here computes any part of the layer."""
import sys

import numpy as np
import torch

import oracle
from bit_mixture_experts_amd import inputs as inp

DEV = "cuda"
TOL = 2e-2   # max|gpu - oracle| <= TOL * RMS(oracle), for every float output


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def bits(t):
    """bf16 device tensor -> numpy uint16 bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t):
    return oracle.bf16_bits_to_f64(bits(t))


def assert_close(got, ref, what, tol=TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    say(f"  {what}: max|err| = {err:.3e}, rms = {rms:.3e}, ratio = {err / max(rms, 1e-30):.2e}")
    assert err <= tol * rms, f"{what}: max|err| {err} > {tol} * rms {rms}"


# Where the backward takes a discrete decision on a value that the GPU carries
# in fp32 and the oracle exactly, the two may decide differently near the
# decision point, and both results are valid:
# * the clamped GLU's derivative jumps at g = limit and u = +-limit: entries
#   whose exact gu lies within CLAMP_BAND * RMS(gu) of a boundary (the test
#   first checks that the GPU's gu is that close to the exact one everywhere;
#   the forward checks measure 4.6e-6 * RMS(gu) on the clamped workloads);
# * dGU is rounded to bf16 for the MFMA: entries whose exact value lies
#   within ROUND_BAND (relative) of a rounding midpoint may take either
#   neighbouring bf16 value. Only those whose one-ulp change can move dx_perm
#   by IMPACT * RMS(dx_perm) or more are considered; the others stay far
#   below the tolerance.
CLAMP_BAND = 2e-5
ROUND_BAND = 1e-4
IMPACT = 1e-3


def backward_reference(x, ri, rw, dout, W, gu_gpu, dx_perm_gpu):
    """The oracle backward on the same inputs, with every decision that sits
    within its band of a decision point taken the way the GPU's dx_perm
    shows: for each row, candidate decisions are flipped one at a time
    (greedily, while a flip brings the GPU's row closer in the L2 norm, its
    effect predicted as the change of the dGU operand times the oracle's
    gate_up weight row), and the returned reference is the oracle run with
    the chosen flips. Only the choice uses the GPU's output; every value of
    the reference is the oracle's."""
    from oracle.layer import activation_backward, join_gate_up, split_gate_up
    ref0 = oracle.layer_backward(x, ri, rw, dout, W)
    R, I2 = ref0["dgu"].shape
    offsets = ref0["offsets"]
    expert_of = np.searchsorted(offsets, np.arange(R), side="right") - 1
    dgu, dgu_x = ref0["dgu"], ref0["dgu_exact"]
    rms_dx = float(np.sqrt(np.mean(ref0["dx_perm"] ** 2)))
    wmax = np.zeros((W.E, I2))
    for e in np.unique(expert_of):
        wmax[e] = np.max(np.abs(W.expert(int(e))[0]), axis=1)
    cand_r, cand_c, cand_kind, cand_delta = [], [], [], []
    # rounding of dGU near a midpoint
    other = oracle.bf16_other_neighbour_f64(dgu_x)
    mid = 0.5 * (dgu + other)
    near = (np.abs(dgu_x - mid) <= ROUND_BAND * np.abs(dgu_x)) & (other != dgu)
    near &= np.abs(other - dgu) * wmax[expert_of] >= IMPACT * rms_dx
    rr, cc = np.nonzero(near)
    cand_r.append(rr), cand_c.append(cc), cand_kind.append(np.zeros(rr.size, int))
    cand_delta.append(other[rr, cc] - dgu[rr, cc])
    nclamp = 0
    if W.act == "swiglu_clamped":
        gu = oracle.layer_forward(x, ri, rw, W, keep=True)["gu"]
        beta = CLAMP_BAND * float(np.sqrt(np.mean(gu ** 2)))
        dgu_err = float(np.max(np.abs(np.asarray(gu_gpu, np.float64) - gu)))
        assert dgu_err <= beta, f"GPU gu off by {dgu_err:.3e}, beyond the clamp band {beta:.3e}"
        g, u = split_gate_up(gu, W.layout, W.I)
        lim = W.limit
        nc = join_gate_up(np.abs(g - lim) <= beta,
                          (np.abs(u - lim) <= beta) | (np.abs(u + lim) <= beta), W.layout) > 0
        rr, cc = np.nonzero(nc)
        nclamp = rr.size
        if rr.size:
            fl = np.zeros((rr.size, I2), dtype=bool)
            fl[np.arange(rr.size), cc] = True
            alt = activation_backward(gu[rr], ref0["dh"][rr], W, fl)[np.arange(rr.size), cc]
            cand_r.append(rr), cand_c.append(cc), cand_kind.append(np.ones(rr.size, int))
            cand_delta.append(bf16_round(alt) - dgu[rr, cc])
    cr, cc, ck, cd = (np.concatenate(v) for v in (cand_r, cand_c, cand_kind, cand_delta))
    got = np.asarray(dx_perm_gpu, np.float64)
    clamp_flip = np.zeros((R, I2), dtype=bool)
    round_flip = np.zeros((R, I2), dtype=bool)
    for r in np.unique(cr):
        sel = np.nonzero(cr == r)[0]
        Wg = W.expert(int(expert_of[r]))[0]
        eff = cd[sel, None] * Wg[cc[sel]]                  # predicted change of row r
        res = got[r] - ref0["dx_perm"][r]
        used = np.zeros(sel.size, dtype=bool)
        while True:
            gain = np.sum(res ** 2) - np.sum((res[None, :] - eff) ** 2, axis=1)
            gain[used] = -np.inf
            j = int(np.argmax(gain))
            if gain[j] <= 0:
                break
            used[j] = True
            res = res - eff[j]
        for j in sel[used]:
            (clamp_flip if ck[j] else round_flip)[r, cc[j]] = True
    say(f"  decision points near the GPU's: {cr.size - nclamp} dGU roundings, {nclamp} clamp "
        f"entries; the GPU took the other side at {int(round_flip.sum())} roundings and "
        f"{int(clamp_flip.sum())} clamps")
    if not clamp_flip.any() and not round_flip.any():
        return ref0
    return oracle.layer_backward(x, ri, rw, dout, W, clamp_flip=clamp_flip, round_flip=round_flip)


def bf16_round(v):
    return oracle.bf16_round_f64(v)


class HostLayer:
    """Host copy of one layer's stacks plus the oracle's dense view."""

    def __init__(self, spec, layer=0, seed=0):
        self.spec, self.layer, self.seed = spec, layer, seed
        E, H, I = spec.E, spec.H, spec.I
        if spec.fmt == "nf4":
            gq, ga, dq, da = [], [], [], []
            for e in range(E):
                wg, wd = inp.host_nf4_source(spec, e, layer, seed)
                p, a = oracle.quantize_nf4(wg.reshape(-1))
                gq.append(p.reshape(2 * I, H // 2))
                ga.append(a.reshape(2 * I, H // 64))
                p, a = oracle.quantize_nf4(wd.reshape(-1))
                dq.append(p.reshape(H, I // 2))
                da.append(a.reshape(H, I // 64))
            self.gu_q, self.gu_s, self.dn_q, self.dn_s = (np.stack(v) for v in (gq, ga, dq, da))
        else:
            self.gu_q, self.gu_s, self.dn_q, self.dn_s = inp.host_stack_mxfp4(spec, layer, seed)
        self.gu_bias = self.dn_bias = self.lora_A = self.lora_B = None
        if spec.bias:
            self.gu_bias, self.dn_bias = inp.host_stack_bias(spec, layer, seed)
        if spec.lora_r:
            self.lora_A, self.lora_B = inp.host_stack_lora(spec, layer, seed)
        kw = dict(layout=spec.layout, act=spec.act, gu_bias=self.gu_bias, dn_bias=self.dn_bias,
                  lora_A=self.lora_A, lora_B=self.lora_B, lora_scale=spec.lora_scale,
                  alpha=spec.alpha, limit=spec.limit)
        if spec.fmt == "nf4":
            self.W = oracle.ExpertWeights.from_nf4(self.gu_q, self.gu_s, self.dn_q, self.dn_s, **kw)
        else:
            self.W = oracle.ExpertWeights.from_mxfp4(self.gu_q, self.gu_s, self.dn_q, self.dn_s, **kw)

    def device(self, variant=0):
        from bit_mixture_experts_amd import moe4
        s = self.spec
        t = lambda a: None if a is None else to_dev(a)
        fmt = moe4.MOE4_FMT_NF4 if s.fmt == "nf4" else moe4.MOE4_FMT_MXFP4
        return moe4.Experts(
            fmt, t(self.gu_q), t(self.gu_s), t(self.dn_q), t(self.dn_s),
            gu_layout=moe4.MOE4_GU_HALVES if s.layout == "halves" else moe4.MOE4_GU_INTERLEAVED,
            act=moe4.MOE4_ACT_SWIGLU if s.act == "swiglu" else moe4.MOE4_ACT_SWIGLU_CLAMPED,
            E=s.E, H=s.H, I=s.I, gu_bias=t(self.gu_bias), dn_bias=t(self.dn_bias),
            lora_A=t(self.lora_A), lora_B=t(self.lora_B), lora_scale=s.lora_scale,
            act_alpha=s.alpha, act_limit=s.limit, variant=variant)


def run_layer(ex, x_dev, logits_dev, k, keep=True, save=False):
    """route -> permute -> expert forward -> combine on the GPU. Returns a dict
    of device tensors."""
    from bit_mixture_experts_amd import moe4
    T, E = logits_dev.shape
    H = x_dev.shape[1]
    S = T * k
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    sor = torch.empty(S, dtype=torch.int32, device=DEV)
    ros = torch.empty(S, dtype=torch.int32, device=DEV)
    x_perm = torch.empty((S, H), dtype=torch.bfloat16, device=DEV)
    y_perm = torch.empty((S, H), dtype=torch.float32, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    out32 = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = torch.empty(moe4.moe4_workspace_size(ex, T, k), dtype=torch.uint8, device=DEV)
    save_gu = torch.empty((S, 2 * ex.I), dtype=torch.float32, device=DEV) if save else None
    save_xa = (torch.empty((S, ex.lora_r), dtype=torch.float32, device=DEV)
               if save and ex.lora_r else None)
    moe4.moe4_route(logits_dev, k, idx, w)
    moe4.moe4_permute(idx, E, offsets, sor, ros, x=x_dev, x_perm=x_perm, ws=ws)
    moe4.moe4_expert_forward(ex, x_perm, offsets, y_perm, save_gu=save_gu, save_xa=save_xa, ws=ws)
    variant = moe4.moe4_last_variant()
    moe4.moe4_combine(y_perm, ros, w, out, k)
    moe4.moe4_combine(y_perm, ros, w, out32, k)
    torch.cuda.synchronize()
    return dict(idx=idx, w=w, offsets=offsets, slot_of_row=sor, row_of_slot=ros, x_perm=x_perm,
                y_perm=y_perm, out=out, out32=out32, save_gu=save_gu, save_xa=save_xa, ws=ws,
                variant=variant)


def check_bf16_output(out_bf16, out_f32, ref, what):
    """The bf16 output is the fp32 output rounded once (torch's cast), and it
    stays within the bound plus half a bf16 ulp of the exact value."""
    assert torch.equal(out_bf16.view(torch.int16), out_f32.to(torch.bfloat16).view(torch.int16)), \
        f"{what}: bf16 output is not the rounded fp32 output"
    got = f64(out_bf16)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    half_ulp = np.abs(ref) * 2.0 ** -8
    assert np.all(np.abs(got - ref) <= TOL * rms + half_ulp), f"{what}: bf16 output off"

