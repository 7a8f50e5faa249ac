"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic kernel choice). The whole batch's routing,
permutation and gathered rows are checked bit-exactly; layer outputs are
checked on sampled tokens, which the oracle computes one by one from its own
quantisation of the experts those tokens use (the GPU-quantised codes of those
experts are compared bit-exactly first)."""
import numpy as np
import pytest
import torch

import oracle
from bit_mixture_experts_amd import inputs as inp
from tests.gpu_helpers import DEV, assert_close, bits, run_layer, say, to_dev

pytestmark = pytest.mark.gpu

moe4 = pytest.importorskip("bit_mixture_experts_amd.moe4")


class BigNF4Layer:
    """NF4 stack quantised on the GPU from the seeded fp32 source; the oracle
    re-quantises single experts on demand from the same source."""

    def __init__(self, spec, layer=0, seed=0):
        self.spec, self.layer, self.seed = spec, layer, seed
        E, H, I = spec.E, spec.H, spec.I
        wg = torch.empty((E, 2 * I, H), dtype=torch.float32, device=DEV)
        wd = torch.empty((E, H, I), dtype=torch.float32, device=DEV)
        for e in range(E):
            g, d = inp.host_nf4_source(spec, e, layer, seed)
            wg[e].copy_(torch.from_numpy(g))
            wd[e].copy_(torch.from_numpy(d))
        self.gq = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=DEV)
        self.gs = torch.empty((E, 2 * I, H // 64), dtype=torch.float32, device=DEV)
        self.dq = torch.empty((E, H, I // 2), dtype=torch.uint8, device=DEV)
        self.ds = torch.empty((E, H, I // 64), dtype=torch.float32, device=DEV)
        moe4.moe4_quantize_nf4(wg, self.gq, self.gs)
        moe4.moe4_quantize_nf4(wd, self.dq, self.ds)
        torch.cuda.synchronize()
        del wg, wd
        torch.cuda.empty_cache()
        self.A = self.B = None
        if spec.lora_r:
            self.A, self.B = inp.host_stack_lora(spec, layer, seed)
        self._q = {}

    def oracle_expert(self, e):
        if e not in self._q:
            g, d = inp.host_nf4_source(self.spec, e, self.layer, self.seed)
            q = oracle.quantize_nf4(g.reshape(-1)) + oracle.quantize_nf4(d.reshape(-1))
            # the GPU quantiser's output for this expert is bit-exact
            assert np.array_equal(self.gq[e].cpu().numpy().reshape(-1), q[0])
            assert np.array_equal(self.gs[e].cpu().numpy().reshape(-1), q[1])
            assert np.array_equal(self.dq[e].cpu().numpy().reshape(-1), q[2])
            assert np.array_equal(self.ds[e].cpu().numpy().reshape(-1), q[3])
            if len(self._q) > 16:
                self._q.clear()
            self._q[e] = q
        return self._q[e]

    def W(self):
        s = self.spec
        I, H = s.I, s.H
        return oracle.ExpertWeights(
            E=s.E, H=H, I=I, layout=s.layout, act=s.act,
            gu=lambda e: oracle.dequantize_nf4_bf16(*self.oracle_expert(e)[:2]).reshape(2 * I, H),
            dn=lambda e: oracle.dequantize_nf4_bf16(*self.oracle_expert(e)[2:]).reshape(H, I),
            lora_A=None if self.A is None else (lambda e: oracle.bf16_bits_to_f64(self.A[e])),
            lora_B=None if self.B is None else (lambda e: oracle.bf16_bits_to_f64(self.B[e])),
            lora_scale=s.lora_scale)

    def device(self):
        s = self.spec
        lora = {}
        if self.A is not None:
            lora = dict(lora_A=to_dev(self.A), lora_B=to_dev(self.B), lora_scale=s.lora_scale)
        return moe4.Experts(moe4.MOE4_FMT_NF4, self.gq, self.gs, self.dq, self.ds,
                            gu_layout=moe4.MOE4_GU_HALVES, act=moe4.MOE4_ACT_SWIGLU,
                            E=s.E, H=s.H, I=s.I, **lora)


class BigMXFP4Layer:
    def __init__(self, spec, layer=0, seed=0):
        self.spec = spec
        self.q = inp.host_stack_mxfp4(spec, layer, seed)
        self.bias = inp.host_stack_bias(spec, layer, seed) if spec.bias else (None, None)
        self.A = self.B = None
        if spec.lora_r:
            self.A, self.B = inp.host_stack_lora(spec, layer, seed)
        self.W = oracle.ExpertWeights.from_mxfp4(*self.q, layout=spec.layout, act=spec.act,
                                                 gu_bias=self.bias[0], dn_bias=self.bias[1],
                                                 lora_A=self.A, lora_B=self.B,
                                                 lora_scale=spec.lora_scale,
                                                 alpha=spec.alpha, limit=spec.limit)

    def device(self):
        s = self.spec
        t = lambda a: None if a is None else to_dev(a)
        lora = {}
        if self.A is not None:
            lora = dict(lora_A=to_dev(self.A), lora_B=to_dev(self.B), lora_scale=s.lora_scale)
        return moe4.Experts(moe4.MOE4_FMT_MXFP4, *[to_dev(a) for a in self.q],
                            gu_layout=moe4.MOE4_GU_INTERLEAVED, act=moe4.MOE4_ACT_SWIGLU_CLAMPED,
                            E=s.E, H=s.H, I=s.I, gu_bias=t(self.bias[0]), dn_bias=t(self.bias[1]),
                            act_alpha=s.alpha, act_limit=s.limit, **lora)


def _check_layer(spec, W, ex, T, n_sample, layer=0, seed=0):
    x, lg = inp.host_tokens(spec, T, layer, seed)
    say(f"  T={T}: running the layer")
    res = run_layer(ex, to_dev(x), to_dev(lg), spec.k)
    say(f"  kernel family {res['variant']}; checking routing and permutation")
    ri, rw = oracle.route(lg, spec.k)
    assert np.array_equal(res["idx"].cpu().numpy(), ri)
    assert np.allclose(res["w"].cpu().numpy(), rw, rtol=1e-5, atol=0)
    ro, rs, rr = oracle.permute(ri, spec.E)
    assert np.array_equal(res["offsets"].cpu().numpy(), ro)
    assert np.array_equal(res["slot_of_row"].cpu().numpy(), rs)
    assert np.array_equal(res["row_of_slot"].cpu().numpy(), rr)
    assert np.array_equal(bits(res["x_perm"]), oracle.gather_rows(x, rs, spec.k))
    rng = np.random.default_rng(T)
    tokens = np.sort(rng.choice(T, min(T, n_sample), replace=False))
    say(f"  oracle on {len(tokens)} sampled tokens")
    ref = np.stack([oracle.token_forward(x[t], ri[t], rw[t], W) for t in tokens])
    got = res["out32"].cpu().numpy()[tokens]
    assert_close(got, ref, f"out (T={T}, sampled)")
    return res


@pytest.mark.parametrize("T", [1, 16, 128, 4096])
def test_qwen3_30b_a3b_nf4_full(T, qwen_layer):
    say(f"Qwen3-30B-A3B-shaped NF4 layer, T={T}")
    _check_layer(inp.QWEN3_30B_NF4, qwen_layer.W(), qwen_layer.device(), T, 6)


@pytest.fixture(scope="module")
def qwen_layer():
    say("building the Qwen3-30B-A3B-shaped NF4 stack (GPU quantisation)")
    return BigNF4Layer(inp.QWEN3_30B_NF4)


def test_qwen3_30b_a3b_nf4_double_quant_full(qwen_layer):
    """The full Qwen3-shaped stack with double-quantised absmax: the GPU's
    compression of its (bit-exact) absmax is bit-exact with the oracle's
    compression of the oracle's own absmax; the layer runs at a decode and a
    prefill token count on the nested form."""
    spec = inp.QWEN3_30B_NF4
    L = qwen_layer
    book = inp.dq_code_book("dynamic")
    say("  oracle absmax of every expert (host quantisation of the seeded source)")
    ga, da = [], []
    for e in range(spec.E):
        g, d = inp.host_nf4_source(spec, e, L.layer, L.seed)
        ga.append(oracle.quantize_nf4(g.reshape(-1))[1])
        da.append(oracle.quantize_nf4(d.reshape(-1))[1])
    ref = {"gu": oracle.compress_absmax(np.concatenate(ga), book),
           "dn": oracle.compress_absmax(np.concatenate(da), book)}
    dev = {}
    ws = torch.empty(moe4.MOE4_DQ_WS_BYTES, dtype=torch.uint8, device=DEV)
    for name, a in (("gu", L.gs), ("dn", L.ds)):
        n = a.numel()
        code = torch.empty(a.shape, dtype=torch.uint8, device=DEV)
        a2 = torch.empty((n + 255) // 256, dtype=torch.float32, device=DEV)
        off = torch.empty(1, dtype=torch.float32, device=DEV)
        moe4.moe4_compress_absmax(a.reshape(-1), to_dev(book), code, a2, off, ws)
        torch.cuda.synchronize()
        rc, ra2, roff = ref[name]
        assert off.cpu().numpy()[0] == roff
        assert np.array_equal(code.cpu().numpy().reshape(-1), rc)
        assert np.array_equal(a2.cpu().numpy().view(np.uint32), ra2.view(np.uint32))
        dev[name] = (code, a2, off)
    exp = {k: oracle.expand_absmax(*ref[k], book) for k in ref}
    I, H = spec.I, spec.H
    ng, nd = 2 * I * H // 64, H * I // 64

    def expert(e):
        q = L.oracle_expert(e)
        return (q[0], exp["gu"][e * ng:(e + 1) * ng], q[2], exp["dn"][e * nd:(e + 1) * nd])

    W = oracle.ExpertWeights(
        E=spec.E, H=H, I=I, layout=spec.layout, act=spec.act,
        gu=lambda e: oracle.dequantize_nf4_bf16(*expert(e)[:2]).reshape(2 * I, H),
        dn=lambda e: oracle.dequantize_nf4_bf16(*expert(e)[2:]).reshape(H, I))
    (gc, ga2, goff), (dc, da2, doff) = dev["gu"], dev["dn"]
    ex = moe4.Experts(moe4.MOE4_FMT_NF4_DQ, L.gq, gc, L.dq, dc, gu_layout=moe4.MOE4_GU_HALVES,
                      act=moe4.MOE4_ACT_SWIGLU, E=spec.E, H=H, I=I, gu_s2=ga2, dn_s2=da2,
                      gu_soff=goff, dn_soff=doff, dq_book=to_dev(book))
    for T in (16, 4096):
        say(f"  T={T}")
        _check_layer(spec, W, ex, T, 6)


@pytest.fixture(scope="module")
def gptoss_layer():
    say("building the gpt-oss-20b-shaped MXFP4 stack")
    return BigMXFP4Layer(inp.GPT_OSS_20B_MXFP4)


@pytest.mark.parametrize("T", [1, 64, 2048])
def test_gpt_oss_20b_mxfp4_full(T, gptoss_layer):
    say(f"gpt-oss-20b-shaped MXFP4 layer, T={T}")
    _check_layer(inp.GPT_OSS_20B_MXFP4, gptoss_layer.W, gptoss_layer.device(), T, 8)


def test_gpt_oss_20b_decode_stack_bit_exact(gptoss_layer):
    say("MXFP4 decode of the full gpt-oss-20b-shaped gate_up stack")
    q, s = gptoss_layer.q[0], gptoss_layer.q[1]
    out = torch.empty(s.shape[:-1] + (s.shape[-1] * 32,), dtype=torch.bfloat16, device=DEV)
    moe4.moe4_decode_mxfp4(to_dev(q), to_dev(s), out)
    torch.cuda.synchronize()
    for e in (0, 17, 31):   # whole experts
        assert np.array_equal(bits(out[e]), oracle.decode_mxfp4_bf16(q[e], s[e]))
    rows = np.random.default_rng(3).choice(s.shape[1], 64, replace=False)
    for e in range(s.shape[0]):   # sampled rows of every expert
        assert np.array_equal(bits(out[e][rows]), oracle.decode_mxfp4_bf16(q[e][rows], s[e][rows]))


def test_gpt_oss_20b_convert_to_nf4_bit_exact(gptoss_layer):
    say("MXFP4 -> NF4 conversion of the full gpt-oss-20b-shaped gate_up and down stacks")
    for q, s in ((gptoss_layer.q[0], gptoss_layer.q[1]), (gptoss_layer.q[2], gptoss_layer.q[3])):
        E, R, nb = s.shape
        packed = torch.empty((E, R, nb * 16), dtype=torch.uint8, device=DEV)
        absmax = torch.empty((E, R, nb // 2), dtype=torch.float32, device=DEV)
        moe4.moe4_convert_mxfp4_nf4(to_dev(q), to_dev(s), packed, absmax)
        torch.cuda.synchronize()
        rows = np.random.default_rng(4).choice(R, 96, replace=False)
        for e in range(E):   # sampled rows of every expert, one whole expert
            sel = slice(None) if e == 5 else rows
            rp, ra = oracle.convert_mxfp4_to_nf4(q[e][sel], s[e][sel])
            assert np.array_equal(packed[e][sel].cpu().numpy(), rp)
            assert np.array_equal(absmax[e][sel].cpu().numpy().view(np.uint32), ra.view(np.uint32))


@pytest.mark.parametrize("spec,T,layer", [(inp.QWEN3_30B_NF4, 4096, 0),
                                           (inp.GPT_OSS_120B_STACK, 32, 7)],
                         ids=["qwen3_T4096", "gpt_oss_120b_T32"])
def test_router_step_full(spec, T, layer):
    """Router logits at the layer's real shape (with the Zipf router bias of
    the 120b stack), the routing-flip floor against the exact logits, and the
    routing backward on the same tokens."""
    say(f"router step: {spec.name}, T={T}")
    x, _ = inp.host_tokens(spec, T, layer)
    wr, rb = inp.host_router(spec, layer)
    bias = rb if spec.zipf else None
    lg = torch.empty((T, spec.E), dtype=torch.float32, device=DEV)
    moe4.moe4_router_logits(to_dev(x), to_dev(wr), lg, bias=None if bias is None else to_dev(bias))
    torch.cuda.synchronize()
    got = lg.cpu().numpy()
    exact = oracle.router_logits(x, wr, bias)
    bound = oracle.router_logits_error_bound(x, wr, bias)
    err = np.abs(got.astype(np.float64) - exact)
    say(f"  logits: max|err| = {err.max():.3e}, max err/bound = {(err / bound).max():.3e}")
    assert np.all(err <= bound)
    k = spec.k
    gi, gw = oracle.route(got, k)
    ei, _ = oracle.route(exact.astype(np.float32), k)
    flips = np.array([set(gi[t]) != set(ei[t]) for t in range(T)])
    srt = -np.sort(-exact, axis=1)
    gap = srt[:, k - 1] - srt[:, k]
    say(f"  routing-flip floor (GPU fp32 logits vs exact): {int(flips.sum())} of {T} tokens "
        f"({flips.mean():.2e}); smallest top-k gap {gap.min():.2e}")
    assert np.all(gap[flips] <= 2 * bound.max())
    # backward on stand-in expert outputs, routed by the GPU's own logits
    _, _, row_of_slot = oracle.permute(gi, spec.E)
    y = inp.host_slot_outputs(spec, T, layer)
    dout = inp.host_upstream_grad(spec, T, layer)
    dw = torch.empty((T, k), dtype=torch.float32, device=DEV)
    dl = torch.empty((T, spec.E), dtype=torch.float32, device=DEV)
    moe4.moe4_route_backward(to_dev(gi), to_dev(gw.astype(np.float32)), to_dev(dout), to_dev(y),
                             to_dev(row_of_slot), dw, dl)
    torch.cuda.synchronize()
    dw_ref = oracle.routing_weight_grad(dout, y, row_of_slot, k)
    dl_ref = oracle.routing_logit_grad(gi, gw, dw_ref, spec.E)
    assert_close(dw.cpu().numpy(), dw_ref, "dw")
    assert_close(dl.cpu().numpy(), dl_ref, "dlogits")


@pytest.mark.parametrize("T", [1, 8, 32])
def test_gpt_oss_120b_stack_layer_full(T):
    spec = inp.GPT_OSS_120B_STACK
    layer = 7   # one of the 36 independently seeded layers, with its Zipf skew
    say(f"gpt-oss-120b-shaped MXFP4 stack, layer {layer}, T={T}")
    L = _stack_layer(spec, layer)
    _check_layer(spec, L.W, L.device(), T, 8, layer=layer)


_STACK = {}


def _stack_layer(spec, layer):
    if layer not in _STACK:
        _STACK.clear()
        _STACK[layer] = BigMXFP4Layer(spec, layer)
    return _STACK[layer]


def test_lora_backward_full(qwen_lora_layer):
    say("per-expert LoRA on the Qwen3-shaped NF4 stack: forward + backward")
    L = qwen_lora_layer
    _check_lora_backward(inp.QWEN3_30B_NF4_LORA, L.device(), L.W())


def test_mxfp4_lora_backward_full():
    spec = inp.GPT_OSS_20B_MXFP4_LORA
    say("per-expert LoRA on the gpt-oss-20b-shaped MXFP4 stack (bias, clamped GLU): "
        "forward + backward")
    L = BigMXFP4Layer(spec)
    _check_lora_backward(spec, L.device(), L.W)


def _check_lora_backward(spec, ex, W):
    T = spec.tokens[0]
    x, lg = inp.host_tokens(spec, T)
    dout = inp.host_upstream_grad(spec, T)
    res = run_layer(ex, to_dev(x), to_dev(lg), spec.k, save=True)
    S = T * spec.k
    dy = torch.empty((S, spec.H), dtype=torch.bfloat16, device=DEV)
    sc = torch.empty(S, dtype=torch.int32, device=DEV)
    moe4.moe4_permute(res["idx"], spec.E, torch.empty_like(res["offsets"]), sc,
                      torch.empty_like(sc), x=to_dev(dout), row_scale=res["w"].reshape(-1),
                      x_perm=dy, ws=res["ws"])
    dx_perm = torch.empty((S, spec.H), dtype=torch.float32, device=DEV)
    dA = torch.empty((spec.E, spec.lora_r, spec.H), dtype=torch.float32, device=DEV)
    dB = torch.empty((spec.E, 2 * spec.I, spec.lora_r), dtype=torch.float32, device=DEV)
    moe4.moe4_expert_backward(ex, res["x_perm"], res["offsets"], res["save_gu"], res["save_xa"],
                              dy, dx_perm, dA, dB, ws=res["ws"])
    dx = torch.empty((T, spec.H), dtype=torch.float32, device=DEV)
    moe4.moe4_combine(dx_perm, res["row_of_slot"], None, dx, spec.k)
    torch.cuda.synchronize()
    ri, rw = oracle.route(lg, spec.k)
    assert np.array_equal(res["idx"].cpu().numpy(), ri)
    # dX of sampled tokens: the oracle backward of those tokens alone
    tokens = np.sort(np.random.default_rng(5).choice(T, 4, replace=False))
    say("  oracle dX on sampled tokens")
    refb = oracle.layer_backward(x[tokens], ri[tokens], rw[tokens], dout[tokens], W)
    assert_close(dx.cpu().numpy()[tokens], refb["dx"], "dx (sampled)")
    # dA, dB of one expert: the oracle backward over exactly the tokens routed to it
    e = int(ri[0, 0])
    toks = np.nonzero((ri == e).any(axis=1))[0]
    say(f"  oracle dA/dB of expert {e} ({len(toks)} tokens)")
    refe = oracle.layer_backward(x[toks], ri[toks], rw[toks], dout[toks], W)
    assert_close(dA.cpu().numpy()[e], refe["dA"][e], f"dA[{e}]")
    assert_close(dB.cpu().numpy()[e], refe["dB"][e], f"dB[{e}]")
    # experts without rows have exact-zero adapter gradients
    counts = np.bincount(ri.reshape(-1), minlength=spec.E)
    for ee in np.nonzero(counts == 0)[0]:
        assert torch.all(dA[ee] == 0) and torch.all(dB[ee] == 0)


@pytest.fixture(scope="module")
def qwen_lora_layer():
    say("building the LoRA NF4 stack")
    return BigNF4Layer(inp.QWEN3_30B_NF4_LORA)
