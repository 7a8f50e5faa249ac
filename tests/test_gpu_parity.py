"""GPU parity against the oracle, element by element, at sizes the oracle
finishes in seconds that still span several tiles and ragged tails. Every call
goes through the C ABI (bit_mixture_experts_amd.moe4).

Bars: bit-exact for the MXFP4 decode, NF4 codes/absmax, top-k indices, the
permutation and x_perm; routing weights to 1e-5 relative; every other float
output within max|err| <= 2e-2 * RMS(oracle)."""
import numpy as np
import pytest
import torch

import oracle
from bit_mixture_experts_amd import inputs as inp
from tests.gpu_helpers import (DEV, HostLayer, assert_close, backward_reference, bits,
                               check_bf16_output, f64, run_layer, say, to_dev)

pytestmark = pytest.mark.gpu

moe4 = pytest.importorskip("bit_mixture_experts_amd.moe4")

# both kernel families of the expert forward
VARIANTS = [moe4.MOE4_VARIANT_SKINNY, moe4.MOE4_VARIANT_TILED]

# scaled-down shapes of the workloads (same formats, layouts, epilogues)
QWEN_SMALL = inp.QWEN3_30B_NF4.scaled(name="qwen3_shaped_small", seed_id=102, E=16, H=512,
                                      I=192, tokens=(5, 100))
GPTOSS_SMALL = inp.GPT_OSS_20B_MXFP4.scaled(name="gpt_oss_shaped_small", seed_id=103, E=8,
                                            H=352, I=352, tokens=(3, 200))
LORA_SMALL = inp.QWEN3_30B_NF4_LORA.scaled(name="lora_small", seed_id=104, E=8, k=2, H=256,
                                           I=128, tokens=(150,))
MXFP4_LORA_SMALL = inp.GPT_OSS_20B_MXFP4.scaled(name="mxfp4_lora_small", seed_id=105, E=8, k=2,
                                                H=320, I=192, tokens=(40,), lora_r=4,
                                                lora_alpha=8.0)
# rows longer than one staged chunk of scales in the decode kernel (8192 k for
# NF4, 16384 k for MXFP4): the gate_up GEMM's K runs over two chunks
LONGK_NF4 = inp.QWEN3_30B_NF4.scaled(name="long_k_nf4", seed_id=107, E=4, k=2, H=8256, I=64,
                                     tokens=(6,))
LONGK_MXFP4 = inp.GPT_OSS_20B_MXFP4.scaled(name="long_k_mxfp4", seed_id=108, E=4, k=2,
                                           H=16416, I=32, tokens=(5,))
# degenerate shapes of the method: one expert at top-1 (a dense 4-bit MLP),
# every expert chosen (k = E), and the smallest MXFP4 rows (H = I = 32: one
# partial iteration / k-tile everywhere)
DENSE_NF4 = inp.TINY_NF4.scaled(name="dense_nf4_E1_k1", seed_id=109, E=1, k=1, H=256, I=128,
                                tokens=(40,))
ALLEXP_NF4 = inp.TINY_NF4.scaled(name="all_experts_nf4_E4_k4", seed_id=110, E=4, k=4, H=128,
                                 I=64, tokens=(33,))
MIN_MXFP4 = inp.GPT_OSS_20B_MXFP4.scaled(name="min_mxfp4_H32_I32", seed_id=111, E=4, k=2, H=32,
                                         I=32, tokens=(9,))
# more experts than one 64-lane pass over the offsets covers twice (E > 128),
# up to the largest E the interface takes
WIDE_NF4 = inp.TINY_NF4.scaled(name="wide_nf4_E160_k2", seed_id=115, E=160, k=2, H=128, I=64,
                               tokens=(40,))
WIDEST_MXFP4 = inp.GPT_OSS_20B_MXFP4.scaled(name="widest_mxfp4_E1024_k4", seed_id=116, E=1024,
                                            k=4, H=64, I=64, tokens=(20,))
# 257..512 experts (eight experts per lane in the tile locator), routing
# skewed so that some experts fill several row tiles
WIDE8_NF4 = inp.TINY_NF4.scaled(name="wide_nf4_E400_k4_zipf", seed_id=143, E=400, k=4, H=128,
                                I=64, tokens=(300,), zipf=1.1)
# top-16 routing: the combine's rows past the eighth and permute's k > 8
TOPK16_NF4 = inp.TINY_NF4.scaled(name="top16_nf4_E64_k16", seed_id=118, E=64, k=16, H=128,
                                 I=64, tokens=(30,))
# adapter ranks other than the workloads' 8, with lora_scale = alpha / r not
# always a power of two: ranks that are not a multiple of four (the adapter
# gradient reductions then read the ranks a dword at a time), ranks past one
# 16-wide MFMA rank step (r > 16) and past one 32-wide tile of the rank
# projection (r > 32), up to the largest rank the interface takes
RANKS = [(1, 2.0), (3, 5.0), (6, 12.0), (12, 16.0), (33, 66.0), (64, 16.0), (4, 3.0)]
RANK_NF4 = [LORA_SMALL.scaled(name=f"lora_nf4_r{r}_a{a:g}", seed_id=120 + i, lora_r=r,
                              lora_alpha=a, tokens=(60,)) for i, (r, a) in enumerate(RANKS)]
RANK_MXFP4 = [MXFP4_LORA_SMALL.scaled(name="lora_mxfp4_r3_a5", seed_id=130, lora_r=3,
                                      lora_alpha=5.0, tokens=(36,)),
              MXFP4_LORA_SMALL.scaled(name="lora_mxfp4_r33_a40", seed_id=131, lora_r=33,
                                      lora_alpha=40.0, tokens=(36,))]
_LAYERS = {}


def layer_of(spec):
    if spec.name not in _LAYERS:
        _LAYERS[spec.name] = HostLayer(spec)
    return _LAYERS[spec.name]


# ------------------------------------------------------------------- codecs

def test_decode_mxfp4_exhaustive():
    say("decode_mxfp4: all 256 bytes x 256 scales")
    byte = np.repeat(np.arange(256, dtype=np.uint8), 256)
    scale = np.tile(np.arange(256, dtype=np.uint8), 256)
    blocks = np.repeat(byte[:, None], 16, axis=1).reshape(-1, 1, 16)
    scales = scale.reshape(-1, 1)
    out = torch.empty((blocks.shape[0], 32), dtype=torch.bfloat16, device=DEV)
    moe4.moe4_decode_mxfp4(to_dev(blocks), to_dev(scales), out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), oracle.decode_mxfp4_bf16(blocks, scales).reshape(-1, 32))


def test_decode_mxfp4_stack_rows_ragged():
    say("decode_mxfp4: gpt-oss-shaped small stack")
    L = layer_of(GPTOSS_SMALL)
    for q, s in ((L.gu_q, L.gu_s), (L.dn_q[:, :37], L.dn_s[:, :37])):
        q = np.ascontiguousarray(q)
        s = np.ascontiguousarray(s)
        out = torch.empty(s.shape[:-1] + (s.shape[-1] * 32,), dtype=torch.bfloat16, device=DEV)
        moe4.moe4_decode_mxfp4(to_dev(q), to_dev(s), out)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), oracle.decode_mxfp4_bf16(q, s))


def test_quantize_nf4_bit_exact():
    say("quantize_nf4: random, midpoint ties, zero and constant blocks")
    rng = np.random.default_rng(20)
    parts = [(rng.standard_normal(64 * 5000) * 0.02).astype(np.float32),
             (rng.standard_normal(64 * 100) * 1e3).astype(np.float32),
             np.zeros(64 * 3, np.float32),
             np.full(64, -0.5, np.float32)]
    # blocks whose elements sit exactly on the fp32 midpoints (absmax = 1)
    mids = oracle.nf4_midpoints()
    tie = np.zeros(64, np.float32)
    tie[0] = 1.0
    tie[1:16] = mids
    tie[16:31] = -mids
    parts.append(tie)
    w = np.concatenate(parts)
    packed = torch.empty(w.size // 2, dtype=torch.uint8, device=DEV)
    absmax = torch.empty(w.size // 64, dtype=torch.float32, device=DEV)
    moe4.moe4_quantize_nf4(to_dev(w), packed, absmax)
    torch.cuda.synchronize()
    rp, ra = oracle.quantize_nf4(w)
    assert np.array_equal(packed.cpu().numpy(), rp)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), ra.view(np.uint32))


def test_quantize_nf4_tiny_stack_matches_oracle_stack():
    spec = inp.TINY_NF4
    L = layer_of(spec)
    for e in (0, spec.E - 1):
        wg, wd = inp.host_nf4_source(spec, e)
        for src, q, s in ((wg, L.gu_q[e], L.gu_s[e]), (wd, L.dn_q[e], L.dn_s[e])):
            packed = torch.empty(src.size // 2, dtype=torch.uint8, device=DEV)
            absmax = torch.empty(src.size // 64, dtype=torch.float32, device=DEV)
            moe4.moe4_quantize_nf4(to_dev(src.reshape(-1)), packed, absmax)
            torch.cuda.synchronize()
            assert np.array_equal(packed.cpu().numpy(), q.reshape(-1))
            assert np.array_equal(absmax.cpu().numpy(), s.reshape(-1))


def _convert(blocks, scales):
    R, nb = scales.shape
    packed = torch.empty((R, nb * 16), dtype=torch.uint8, device=DEV)
    absmax = torch.empty((R, nb // 2), dtype=torch.float32, device=DEV)
    moe4.moe4_convert_mxfp4_nf4(to_dev(blocks), to_dev(scales), packed, absmax)
    torch.cuda.synchronize()
    return packed.cpu().numpy(), absmax.cpu().numpy()


def test_convert_mxfp4_nf4_bit_exact():
    say("convert_mxfp4_nf4: gpt-oss-shaped small stack, wide scale spreads, zero blocks")
    L = layer_of(GPTOSS_SMALL)
    # K = 352 there: take 10 of the 11 blocks per row (K % 64 == 0)
    cases = [(L.gu_q[:, :, :10], L.gu_s[:, :, :10]), (L.dn_q[:, :37, 3:], L.dn_s[:, :37, 3:]),
             (L.dn_q[:, :, :2], L.dn_s[:, :, :2])]
    rng = np.random.default_rng(21)
    R, nb = 300, 90
    blocks = rng.integers(0, 256, (R, nb, 16), dtype=np.uint8)
    blocks[::7] &= rng.choice(np.array([0, 0x0F, 0xF0, 0x88, 0x11], np.uint8), (43, nb, 16))
    blocks[5, 10:12] = 0
    blocks[6, 20:22] = 0x88
    scales = rng.integers(0, 253, (R, nb), dtype=np.uint8)
    scales[100:200, 1::2] = np.clip(scales[100:200, 0::2].astype(int)
                                    - rng.integers(0, 12, (100, nb // 2)), 0, 252)
    scales[200:220] = rng.integers(0, 3, (20, nb), dtype=np.uint8)   # subnormal decodes
    cases.append((blocks, scales))
    for q, s in cases:
        q = np.ascontiguousarray(q).reshape(-1, q.shape[-2], 16)
        s = np.ascontiguousarray(s).reshape(-1, s.shape[-1])
        gp, ga = _convert(q, s)
        rp, ra = oracle.convert_mxfp4_to_nf4(q, s)
        assert np.array_equal(ga.view(np.uint32), ra.view(np.uint32))
        assert np.array_equal(gp, rp)
    # R = 0 is a no-op
    moe4.moe4_convert_mxfp4_nf4(torch.empty((0, 2, 16), dtype=torch.uint8, device=DEV),
                                torch.empty((0, 2), dtype=torch.uint8, device=DEV),
                                torch.empty((0, 32), dtype=torch.uint8, device=DEV),
                                torch.empty((0, 1), dtype=torch.float32, device=DEV))


# ------------------------------------------------ double-quantised absmax

def _gpu_compress(a, book):
    n = a.size
    code = torch.empty(n, dtype=torch.uint8, device=DEV)
    a2 = torch.empty((n + 255) // 256, dtype=torch.float32, device=DEV)
    off = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(moe4.MOE4_DQ_WS_BYTES, dtype=torch.uint8, device=DEV)
    moe4.moe4_compress_absmax(to_dev(a.reshape(-1)), to_dev(book), code, a2, off, ws)
    torch.cuda.synchronize()
    return code, a2, off


def test_compress_expand_absmax_bit_exact():
    say("compress/expand absmax: small stacks, ragged, large, constant; two code books")
    L = layer_of(QWEN_SMALL)
    rng = np.random.default_rng(22)
    arrays = [L.gu_s, np.ascontiguousarray(L.dn_s[:, :37]),
              (np.abs(rng.standard_normal(256 * 3000 + 13)) * 0.05).astype(np.float32),
              np.full(700, 0.03125, np.float32)]
    for kind in ("dynamic", "linear"):
        book = inp.dq_code_book(kind)
        for a in arrays:
            code, a2, off = _gpu_compress(a, book)
            rc, ra2, roff = oracle.compress_absmax(a, book)
            assert off.cpu().numpy()[0] == roff
            assert np.array_equal(a2.cpu().numpy().view(np.uint32), ra2.view(np.uint32))
            assert np.array_equal(code.cpu().numpy(), rc)
            out = torch.empty(a.size, dtype=torch.float32, device=DEV)
            moe4.moe4_expand_absmax(code, a2, off, to_dev(book), out)
            torch.cuda.synchronize()
            want = oracle.expand_absmax(rc, ra2, roff, book)
            assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))


class DQLayer:
    """An NF4 layer whose absmax is double-quantised on the GPU (bit-exact with
    the oracle's), and the oracle's weights built on the decoded absmax."""

    def __init__(self, spec, kind="dynamic"):
        L = layer_of(spec)
        self.L, self.spec = L, spec
        self.book = inp.dq_code_book(kind)
        self.dev = {}
        expanded = []
        for name, a in (("gu", L.gu_s), ("dn", L.dn_s)):
            code, a2, off = _gpu_compress(a, self.book)
            rc, ra2, roff = oracle.compress_absmax(a, self.book)
            assert np.array_equal(code.cpu().numpy(), rc) and off.cpu().numpy()[0] == roff
            self.dev[name] = (code.view(a.shape), a2, off)
            expanded.append(oracle.expand_absmax(rc, ra2, roff, self.book).reshape(a.shape))
        kw = dict(layout=spec.layout, act=spec.act, lora_A=L.lora_A, lora_B=L.lora_B,
                  lora_scale=spec.lora_scale)
        self.W = oracle.ExpertWeights.from_nf4(L.gu_q, expanded[0], L.dn_q, expanded[1], **kw)

    def device(self, variant=0):
        L, s = self.L, self.spec
        t = lambda a: None if a is None else to_dev(a)
        (gc, ga2, goff), (dc, da2, doff) = self.dev["gu"], self.dev["dn"]
        return moe4.Experts(moe4.MOE4_FMT_NF4_DQ, t(L.gu_q), gc, t(L.dn_q), dc,
                            gu_layout=moe4.MOE4_GU_HALVES, act=moe4.MOE4_ACT_SWIGLU,
                            E=s.E, H=s.H, I=s.I, lora_A=t(L.lora_A), lora_B=t(L.lora_B),
                            lora_scale=s.lora_scale, variant=variant, gu_s2=ga2, dn_s2=da2,
                            gu_soff=goff, dn_soff=doff, dq_book=to_dev(self.book))


DQ_CASES = [(QWEN_SMALL, 5, "dynamic"), (QWEN_SMALL, 100, "linear"), (LORA_SMALL, 150, "dynamic"),
            (DENSE_NF4, 40, "dynamic")]


@pytest.mark.parametrize("variant", [moe4.MOE4_VARIANT_SKINNY, moe4.MOE4_VARIANT_TILED])
@pytest.mark.parametrize("spec,T,kind", DQ_CASES, ids=[f"{s.name}-T{t}-{k}" for s, t, k in DQ_CASES])
def test_layer_forward_double_quant(spec, T, kind, variant):
    say(f"forward, double-quantised absmax: {spec.name} T={T} book={kind} variant={variant}")
    D = DQLayer(spec, kind)
    x, lg = inp.host_tokens(spec, T)
    res = run_layer(D.device(variant), to_dev(x), to_dev(lg), spec.k, save=True)
    assert res["variant"] == variant
    ri, rw = oracle.route(lg, spec.k)
    ref = oracle.layer_forward(x, ri, rw, D.W, keep=True)
    assert_close(res["save_gu"].cpu().numpy(), ref["gu"], "gu")
    assert_close(res["y_perm"].cpu().numpy(), ref["y"], "y_perm")
    assert_close(res["out32"].cpu().numpy(), ref["out"], "out")


# rows of 5 and 3 absmax: the 256-absmax groups of the second level begin
# inside weight rows and inside dgrad k-tiles
DQ_LORA_ODD = inp.QWEN3_30B_NF4_LORA.scaled(name="lora_dq_odd_rows", seed_id=142, E=8, k=2, H=320,
                                            I=192, tokens=(90,))


@pytest.mark.parametrize("spec,T", [(LORA_SMALL, 150), (DQ_LORA_ODD, 90)],
                         ids=["lora_small-T150", "lora_dq_odd_rows-T90"])
def test_layer_backward_double_quant(spec, T):
    say(f"backward, double-quantised absmax: {spec.name} T={T}")
    D = DQLayer(spec)
    ex = D.device()
    x, lg = inp.host_tokens(spec, T)
    dout = inp.host_upstream_grad(spec, T)
    res = run_layer(ex, to_dev(x), to_dev(lg), spec.k, save=True)
    S = T * spec.k
    dy = torch.empty((S, spec.H), dtype=torch.bfloat16, device=DEV)
    e0 = torch.empty(S, dtype=torch.int32, device=DEV)
    moe4.moe4_permute(res["idx"], spec.E, torch.empty_like(res["offsets"]), e0,
                      torch.empty_like(e0), x=to_dev(dout), row_scale=res["w"].reshape(-1),
                      x_perm=dy, ws=res["ws"])
    dx_perm = torch.empty((S, spec.H), dtype=torch.float32, device=DEV)
    dA = torch.empty((spec.E, spec.lora_r, spec.H), device=DEV)
    dB = torch.empty((spec.E, 2 * spec.I, spec.lora_r), device=DEV)
    moe4.moe4_expert_backward(ex, res["x_perm"], res["offsets"], res["save_gu"], res["save_xa"],
                              dy, dx_perm, dA, dB, ws=res["ws"])
    torch.cuda.synchronize()
    ri, rw = oracle.route(lg, spec.k)
    ref = oracle.layer_backward(x, ri, rw, dout, D.W)
    assert_close(dx_perm.cpu().numpy(), ref["dx_perm"], "dx_perm")
    assert_close(dA.cpu().numpy(), ref["dA"], "dA")
    assert_close(dB.cpu().numpy(), ref["dB"], "dB")


# --------------------------------------------------------------- router step

def router_case(T, E, H, seed, bias=True):
    rng = np.random.default_rng(seed)
    xb = inp.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = inp.to_bf16_bits((rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32))
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    return xb, wb, b


def gpu_router_logits(xb, wb, b):
    T, E = xb.shape[0], wb.shape[0]
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    moe4.moe4_router_logits(to_dev(xb), to_dev(wb), lg, bias=None if b is None else to_dev(b))
    torch.cuda.synchronize()
    return lg.cpu().numpy()


def check_router_logits(xb, wb, b):
    """GPU logits within the fp32 dot-product bound of the exact sums; routing
    on them equal to routing on the rounded exact logits except where the
    exact gap at the top-k boundary is within the bound. Returns the flip
    fraction."""
    got = gpu_router_logits(xb, wb, b)
    exact = oracle.router_logits(xb, wb, b)
    bound = oracle.router_logits_error_bound(xb, wb, b)
    err = np.abs(got.astype(np.float64) - exact)
    say(f"  logits: max|err| = {err.max():.3e}, max err/bound = {(err / bound).max():.3e}")
    assert np.all(err <= bound)
    return got, exact, bound


@pytest.mark.parametrize("T,E,H", [(100, 40, 264), (37, 8, 256), (300, 128, 2048), (5, 1024, 64)])
def test_router_logits_within_fp32_bound(T, E, H):
    say(f"router_logits T={T} E={E} H={H}")
    xb, wb, b = router_case(T, E, H, seed=T + E + H)
    check_router_logits(xb, wb, b)
    check_router_logits(xb, wb, None)


def test_router_route_flip_floor_small():
    say("router -> route: flips only where the exact top-k gap is within the bound")
    T, E, H, k = 512, 128, 2048, 8
    xb, wb, b = router_case(T, E, H, seed=77, bias=False)
    got, exact, bound = check_router_logits(xb, wb, b)
    gi, _ = oracle.route(got, k)
    ei, _ = oracle.route(exact.astype(np.float32), k)
    srt = -np.sort(-exact, axis=1)
    gap = srt[:, k - 1] - srt[:, k]
    flips = np.array([set(gi[t]) != set(ei[t]) for t in range(T)])
    say(f"  flipped tokens: {int(flips.sum())} of {T}")
    assert np.all(gap[flips] <= 2 * bound.max())
    # the GPU's own route of its logits is bit-exact with the oracle's route of
    # the same logits (the rule is exact on given fp32 logits)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe4.moe4_route(to_dev(got), k, idx, w)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), gi)


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("T,E,k,H", [(64, 8, 2, 256), (150, 128, 8, 2048), (9, 32, 4, 2880),
                                     (3, 1024, 70, 64)])
def test_route_backward(T, E, k, H, renorm):
    say(f"route_backward T={T} E={E} k={k} H={H} renorm={renorm}")
    spec = inp.QWEN3_30B_NF4.scaled(name="route_bwd", seed_id=106, E=E, k=k, H=H)
    _, lg = inp.host_tokens(spec, T)
    ri, rw = oracle.route(lg, k, renormalize=renorm)
    _, slot_of_row, row_of_slot = oracle.permute(ri, E)
    y = inp.host_slot_outputs(spec, T)          # expert outputs in permuted-row order
    dout = inp.host_upstream_grad(spec, T)
    dw_ref = oracle.routing_weight_grad(dout, y, row_of_slot, k)
    dl_ref = oracle.routing_logit_grad(ri, rw, dw_ref, E, renormalize=renorm, logits=lg)
    dw = torch.empty((T, k), dtype=torch.float32, device=DEV)
    dl = torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV)
    moe4.moe4_route_backward(to_dev(ri.astype(np.int32)), to_dev(rw.astype(np.float32)),
                             to_dev(dout), to_dev(y), to_dev(row_of_slot), dw, dl,
                             logits=to_dev(lg), renormalize=renorm)
    torch.cuda.synchronize()
    gdw, gdl = dw.cpu().numpy(), dl.cpu().numpy()
    # dw: fp32 sums of H fp32 products, each product rounded once
    d = np.abs(oracle.bf16_bits_to_f64(dout))
    mag = np.einsum("th,tjh->tj", d, np.abs(y.astype(np.float64))[row_of_slot.reshape(T, k)])
    n = H + 1
    bound = (n * 2.0 ** -24 / (1 - n * 2.0 ** -24) + 2.0 ** -24) * mag
    assert np.all(np.abs(gdw - dw_ref) <= bound)
    assert_close(gdw, dw_ref, "dw")
    assert_close(gdl, dl_ref, "dlogits")
    assert np.max(np.abs(gdl - dl_ref)) <= 1e-4 * np.sqrt(np.mean(dl_ref ** 2))
    if renorm:   # experts that were not chosen get exactly zero
        mask = np.ones((T, E), bool)
        np.put_along_axis(mask, ri.astype(np.int64), False, 1)
        assert np.all(gdl[mask] == 0)


# ------------------------------------------------------------------ routing

def _route(lg, k, renorm=True):
    T, E = lg.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe4.moe4_route(to_dev(lg), k, idx, w, renormalize=renorm)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("T,E,k,kind", [(64, 8, 2, "normal"), (300, 128, 8, "normal"),
                                        (77, 32, 4, "normal"), (50, 128, 4, "zipf"),
                                        (40, 1024, 16, "normal"), (33, 16, 16, "normal"),
                                        (129, 64, 6, "ties"), (17, 1, 1, "normal"),
                                        (65, 256, 64, "special"), (9, 1000, 100, "normal"),
                                        (31, 96, 20, "special")])
def test_route_bit_exact(T, E, k, kind):
    """Top-k indices equal to the oracle's; weights within 1e-5 relative.
    'special' rows mix -inf, +-0, subnormals and values near the fp32 limits
    into the logits (each row keeps a finite maximum)."""
    say(f"route T={T} E={E} k={k} {kind}")
    rng = np.random.default_rng(T * 1000 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        lg = rng.integers(-3, 3, (T, E)).astype(np.float32)
        lg[lg == 0] = np.where(rng.random((lg == 0).sum()) < 0.5, 0.0, -0.0)
    if kind == "zipf":
        lg += -1.1 * np.log(1 + rng.permutation(E)).astype(np.float32)
    if kind == "special":
        pool = np.array([-np.inf, 0.0, -0.0, 1e-45, -1e-45, 1e-40, -3.0e38, 3.0e38, -1.0],
                        dtype=np.float32)
        hit = rng.random((T, E)) < 0.4
        lg[hit] = pool[rng.integers(0, len(pool), hit.sum())]
        lg[:, 0] = np.maximum(lg[:, 0], 0.0)   # a finite maximum in every row
    for renorm in (True, False):
        gi, gw = _route(lg, k, renorm)
        ri, rw = oracle.route(lg, k, renormalize=renorm)
        assert np.array_equal(gi, ri)
        assert np.allclose(gw, rw, rtol=1e-5, atol=0)


def _perm_ws_bytes(S, E):
    """A descriptor-free workspace size for the permutation: per-chunk expert
    counts, chunks of 512 slots up to 64K slots and of 2048 beyond."""
    chunk = 512 if S <= 65536 else 2048
    return max(256, 4 * -(-S // chunk) * E + 256)


def _permute(idx, E, x=None, scale=None):
    T, k = idx.shape
    S = T * k
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    sor = torch.empty(max(S, 1), dtype=torch.int32, device=DEV)
    ros = torch.empty(max(S, 1), dtype=torch.int32, device=DEV)
    xd = None if x is None else to_dev(x)
    x_perm = None if x is None else torch.empty((max(S, 1), x.shape[1]), dtype=torch.bfloat16,
                                                device=DEV)
    # a descriptor-free workspace size: the permutation part only needs E, T, k
    ws = torch.empty(_perm_ws_bytes(S, E), dtype=torch.uint8, device=DEV)
    moe4.moe4_permute(to_dev(idx), E, offsets, sor, ros, x=xd,
                      row_scale=None if scale is None else to_dev(scale), x_perm=x_perm, ws=ws)
    torch.cuda.synchronize()
    return offsets, sor, ros, x_perm


# (8192, 128, 8) and (9000, 128, 8): 65536 and 72000 slots, both sides of the
# switch from 512-slot to 2048-slot chunks
@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (1, 128, 8), (128, 128, 8), (200, 32, 4),
                                   (3000, 128, 8), (300, 1024, 7), (1500, 4, 4), (100, 64, 16),
                                   (700, 32, 16), (40, 1024, 32), (50, 64, 16), (8192, 128, 8),
                                   (9000, 128, 8)])
def test_permute_bit_exact(T, E, k):
    say(f"permute T={T} E={E} k={k}")
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    H = 40
    x = inp.to_bf16_bits(rng.standard_normal((T, H)))
    scale = rng.random(T * k).astype(np.float32)
    for sc in (None, scale):
        off, sor, ros, xp = _permute(idx, E, x, sc)
        ro, rs, rr = oracle.permute(idx, E)
        assert np.array_equal(off.cpu().numpy(), ro)
        assert np.array_equal(sor.cpu().numpy(), rs)
        assert np.array_equal(ros.cpu().numpy(), rr)
        assert np.array_equal(bits(xp), oracle.gather_rows(x, rs, k, row_scale=sc))


@pytest.mark.parametrize("T,E,k,H", [(100, 40, 2, 264), (300, 128, 8, 2048), (1, 8, 2, 8),
                                     (0, 8, 2, 64)])
def test_gather_rows_bit_exact(T, E, k, H):
    """moe4_gather_rows on moe4_permute's slot_of_row gives moe4_permute's
    x_perm bit for bit, with and without a row scale, and the oracle's rows;
    a slot outside [0, T*k) gives a zero row (the other rows unchanged)."""
    say(f"gather rows T={T} E={E} k={k} H={H}")
    rng = np.random.default_rng(900 + T + E + k + H)
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)],
                   dtype=np.int32).reshape(T, k)
    x = inp.to_bf16_bits(rng.standard_normal((T, H)))
    scale = rng.random(T * k).astype(np.float32)
    for sc in (None, scale):
        _, sor, _, xp = _permute(idx, E, x, sc) if T else (None, None, None, None)
        S = T * k
        sor_d = sor if T else torch.empty(0, dtype=torch.int32, device=DEV)
        out = torch.full((S, H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        xd = to_dev(x) if T else torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
        moe4.moe4_gather_rows(xd, k, sor_d, out,
                              row_scale=None if sc is None else to_dev(sc))
        torch.cuda.synchronize()
        if T == 0:
            continue
        assert np.array_equal(bits(out), bits(xp))
        _, rs, _ = oracle.permute(idx, E)
        assert np.array_equal(bits(out), oracle.gather_rows(x, rs, k, row_scale=sc))
    if T:
        bad = sor.clone()
        bad[0] = S
        bad[-1] = -1
        out = torch.full((S, H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        moe4.moe4_gather_rows(to_dev(x), k, bad, out)
        torch.cuda.synchronize()
        ob, ref = bits(out), oracle.gather_rows(x, rs, k)
        assert np.all(ob[0] == 0) and np.all(ob[-1] == 0)
        assert np.array_equal(ob[1:-1], ref[1:-1])


# fused routing + permutation: batches of up to 4 tokens in one launch, the rest
# through the two separate calls; ties, one expert, E up to 1024
ROUTE_PERMUTE_CASES = [(1, 128, 8, "normal"), (4, 1024, 16, "ties"), (3, 1, 1, "normal"),
                       (2, 300, 3, "zipf"), (4, 32, 32, "normal"), (5, 128, 8, "normal"),
                       (16, 128, 8, "normal"), (64, 32, 4, "zipf"), (200, 64, 6, "ties"),
                       (1, 256, 64, "ties"), (4, 64, 16, "zipf"), (2, 1000, 2, "normal")]


@pytest.mark.parametrize("T,E,k,kind", ROUTE_PERMUTE_CASES)
def test_route_permute_bit_exact(T, E, k, kind):
    """moe4_route_permute gives every output of moe4_route + moe4_permute bit
    for bit, and the oracle's indices, permutation and gathered rows; also
    without the row gather (x = None), which for up to 64 slots of up to 4
    tokens runs in a kernel of its own."""
    say(f"route + permute T={T} E={E} k={k} {kind}")
    rng = np.random.default_rng(7000 + T * 31 + E + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        lg = rng.integers(-3, 3, (T, E)).astype(np.float32)
    if kind == "zipf":
        lg += -1.1 * np.log(1 + rng.permutation(E)).astype(np.float32)
    H = 72
    x = inp.to_bf16_bits(rng.standard_normal((T, H)))
    S = T * k
    for renorm, gather in ((True, True), (False, True), (True, False), (False, False)):
        gi, gw = _route(lg, k, renorm)
        off, sor, ros, xp = _permute(gi, E, x)
        fi = torch.empty((T, k), dtype=torch.int32, device=DEV)
        fw = torch.empty((T, k), dtype=torch.float32, device=DEV)
        foff = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        fsor = torch.empty(S, dtype=torch.int32, device=DEV)
        fros = torch.empty(S, dtype=torch.int32, device=DEV)
        fxp = torch.empty((S, H), dtype=torch.bfloat16, device=DEV)
        ws = torch.empty(_perm_ws_bytes(S, E), dtype=torch.uint8,
                         device=DEV)
        if gather:
            moe4.moe4_route_permute(to_dev(lg), k, fi, fw, foff, fsor, fros, x=to_dev(x),
                                    x_perm=fxp, ws=ws, renormalize=renorm)
        else:
            # stale contents must not leak into the outputs
            for t_ in (fi, foff, fsor, fros):
                t_.fill_(-7)
            fw.fill_(float("nan"))
            moe4.moe4_route_permute(to_dev(lg), k, fi, fw, foff, fsor, fros, ws=ws,
                                    renormalize=renorm)
        torch.cuda.synchronize()
        assert np.array_equal(fi.cpu().numpy(), gi)
        assert np.array_equal(fw.cpu().numpy().view(np.uint32), gw.view(np.uint32))
        for a_, b_ in ((foff, off), (fsor, sor), (fros, ros)):
            assert torch.equal(a_, b_)
        if gather:
            assert np.array_equal(bits(fxp), bits(xp))
        ri, _ = oracle.route(lg, k, renormalize=renorm)
        ro, rs, _ = oracle.permute(ri, E)
        assert np.array_equal(fi.cpu().numpy(), ri)
        assert np.array_equal(foff.cpu().numpy(), ro) and np.array_equal(fsor.cpu().numpy(), rs)
        if gather:
            assert np.array_equal(bits(fxp), oracle.gather_rows(x, rs, k))


def test_permute_skewed_one_expert():
    say("permute: every slot on one expert")
    T, E, k = 2500, 64, 1
    idx = np.full((T, k), 17, np.int32)
    off, sor, ros, _ = _permute(idx, E)
    ro, rs, rr = oracle.permute(idx, E)
    assert np.array_equal(off.cpu().numpy(), ro) and np.array_equal(sor.cpu().numpy(), rs)


# k = 8 is the last count whose rows are all loaded together; k > 8 takes the
# one-row-at-a-time tail; H = 8 leaves most lanes of the wave idle
COMBINE_CASES = [(70, 4, 264), (33, 1, 64), (50, 8, 136), (19, 9, 72), (23, 16, 2056),
                 (5, 32, 8)]


@pytest.mark.parametrize("T,k,H", COMBINE_CASES)
def test_combine_against_oracle(T, k, H):
    say(f"combine T={T} k={k} H={H}")
    rng = np.random.default_rng(21 + T * k + H)
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    ros = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    out32 = torch.empty((T, H), dtype=torch.float32, device=DEV)
    for ww in (w, None):
        wd = None if ww is None else to_dev(ww)
        moe4.moe4_combine(to_dev(y), to_dev(ros), wd, out, k)
        moe4.moe4_combine(to_dev(y), to_dev(ros), wd, out32, k)
        torch.cuda.synchronize()
        ref = oracle.combine(y.astype(np.float64), ros, ww, T, k)
        assert_close(out32.cpu().numpy(), ref, "combine out fp32")
        # fp32 sum of k terms: relative error of a few fp32 ulps
        assert np.all(np.abs(out32.cpu().numpy() - ref) <= 1e-6 * (np.abs(ref) + 1))
        check_bf16_output(out, out32, ref, "combine out")


# ------------------------------------------------------------ layer forward

FWD_CASES = [(inp.TINY_NF4, 64), (QWEN_SMALL, 5), (QWEN_SMALL, 100), (GPTOSS_SMALL, 3),
             (GPTOSS_SMALL, 200), (LORA_SMALL, 150), (MXFP4_LORA_SMALL, 40), (LONGK_NF4, 6),
             (LONGK_MXFP4, 5), (DENSE_NF4, 40), (ALLEXP_NF4, 33), (MIN_MXFP4, 9), (QWEN_SMALL, 1),
             (GPTOSS_SMALL, 1), (WIDE_NF4, 40), (WIDEST_MXFP4, 20), (TOPK16_NF4, 30),
             (WIDE8_NF4, 300)]


@pytest.mark.parametrize("variant", [moe4.MOE4_VARIANT_SKINNY, moe4.MOE4_VARIANT_TILED])
@pytest.mark.parametrize("spec,T", FWD_CASES, ids=[f"{s.name}-T{t}" for s, t in FWD_CASES])
def test_layer_forward(spec, T, variant):
    say(f"forward {spec.name} T={T} variant={variant}")
    L = layer_of(spec)
    x, lg = inp.host_tokens(spec, T)
    res = run_layer(L.device(variant), to_dev(x), to_dev(lg), spec.k, save=True)
    assert res["variant"] == variant
    ri, rw = oracle.route(lg, spec.k)
    assert np.array_equal(res["idx"].cpu().numpy(), ri)
    ref = oracle.layer_forward(x, ri, rw, L.W, keep=True)
    assert np.array_equal(res["offsets"].cpu().numpy(), ref["offsets"])
    assert_close(res["save_gu"].cpu().numpy(), ref["gu"], "gu")
    assert_close(res["y_perm"].cpu().numpy(), ref["y"], "y_perm")
    assert_close(res["out32"].cpu().numpy(), ref["out"], "out")
    check_bf16_output(res["out"], res["out32"], ref["out"], "out")
    if spec.lora_r:
        assert_close(res["save_xa"].cpu().numpy(), ref["xa"], "xa")
        # the adapter's own contribution, isolated: the GPU's gu minus the oracle's
        # adapter-free gu, against the oracle's delta (relative L2, 5%)
        base = oracle.layer_forward(x, ri, rw, _without_lora(L), keep=True)
        got = res["save_gu"].cpu().numpy() - base["gu"]
        want = ref["gu"] - base["gu"]
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        say(f"  lora delta relative L2 error {rel:.2e}")
        assert rel < 0.05


RANK_FWD = [(s, s.tokens[0]) for s in RANK_NF4 + RANK_MXFP4]


@pytest.mark.parametrize("variant", [moe4.MOE4_VARIANT_SKINNY, moe4.MOE4_VARIANT_TILED])
@pytest.mark.parametrize("spec,T", RANK_FWD, ids=[s.name for s, _ in RANK_FWD])
def test_layer_forward_lora_ranks(spec, T, variant):
    """Both kernel families apply lora_scale in fp32 to the rank sum, for any
    rank the interface takes."""
    say(f"forward {spec.name} (scale {spec.lora_scale:g}) T={T} variant={variant}")
    L = layer_of(spec)
    x, lg = inp.host_tokens(spec, T)
    res = run_layer(L.device(variant), to_dev(x), to_dev(lg), spec.k, save=True)
    assert res["variant"] == variant
    ri, rw = oracle.route(lg, spec.k)
    ref = oracle.layer_forward(x, ri, rw, L.W, keep=True)
    assert_close(res["save_xa"].cpu().numpy(), ref["xa"], "xa")
    assert_close(res["save_gu"].cpu().numpy(), ref["gu"], "gu")
    assert_close(res["y_perm"].cpu().numpy(), ref["y"], "y_perm")
    assert_close(res["out32"].cpu().numpy(), ref["out"], "out")
    base = oracle.layer_forward(x, ri, rw, _without_lora(L), keep=True)
    got = res["save_gu"].cpu().numpy() - base["gu"]
    want = ref["gu"] - base["gu"]
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    say(f"  lora delta relative L2 error {rel:.2e}")
    assert rel < 0.05


# the row gather fused into gate_up: shapes that reach both kernel families,
# ragged tiles, E = 1, one row per expert, double-quantised stacks, skewed rows
GATHER_CASES = [(QWEN_SMALL, 5), (QWEN_SMALL, 100), (GPTOSS_SMALL, 3), (GPTOSS_SMALL, 200),
                (DENSE_NF4, 40), (ALLEXP_NF4, 33), (WIDE_NF4, 40), (TOPK16_NF4, 30),
                (LONGK_MXFP4, 5), (WIDE8_NF4, 300)]


def _gather_forward(ex, x_dev, res, k, save):
    S, H = res["x_perm"].shape
    y = torch.full((S, H), float("nan"), dtype=torch.float32, device=DEV)
    gu = torch.full((S, 2 * ex.I), float("nan"), dtype=torch.float32, device=DEV) if save else None
    moe4.moe4_expert_forward_gather(ex, x_dev, k, res["slot_of_row"], res["offsets"], y,
                                    save_gu=gu, ws=res["ws"])
    torch.cuda.synchronize()
    return y, gu, moe4.moe4_last_variant()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("spec,T", GATHER_CASES, ids=[f"{s.name}-T{t}" for s, t in GATHER_CASES])
def test_forward_gather_matches_x_perm_forward(spec, T, variant):
    """Gathering the rows inside the gate_up GEMM gives the x_perm forward's
    y_perm and gu bit for bit (the same operands reach the same MFMAs), and
    the oracle's layer."""
    say(f"forward with the gather fused: {spec.name} T={T} variant={variant}")
    L = layer_of(spec)
    ex = L.device(variant)
    x, lg = inp.host_tokens(spec, T)
    xd = to_dev(x)
    res = run_layer(ex, xd, to_dev(lg), spec.k, save=True)
    y, gu, v = _gather_forward(ex, xd, res, spec.k, True)
    assert v == variant
    assert torch.equal(y, res["y_perm"]) and torch.equal(gu, res["save_gu"])
    ri, rw = oracle.route(lg, spec.k)
    ref = oracle.layer_forward(x, ri, rw, L.W)
    assert_close(y.cpu().numpy(), ref["y"], "y_perm (gathered)")


@pytest.mark.parametrize("variant", VARIANTS)
def test_forward_gather_double_quant(variant):
    spec, T = QWEN_SMALL, 100
    say(f"forward with the gather fused, double-quantised: T={T} variant={variant}")
    D = DQLayer(spec)
    ex = D.device(variant)
    x, lg = inp.host_tokens(spec, T)
    xd = to_dev(x)
    res = run_layer(ex, xd, to_dev(lg), spec.k, save=True)
    y, gu, _ = _gather_forward(ex, xd, res, spec.k, True)
    assert torch.equal(y, res["y_perm"]) and torch.equal(gu, res["save_gu"])


def test_forward_gather_skewed_rows():
    """Two hot experts with hundreds of rows: several skinny chunks and several
    equal tiles per expert, each gathering its own rows."""
    spec, T = inp.TINY_NF4, 700
    L = layer_of(spec)
    x, _ = inp.host_tokens(spec, T)
    lg = np.full((T, spec.E), -5.0, np.float32)
    lg[:, 3] = 5.0
    lg[:, 6] = 4.0
    xd = to_dev(x)
    for variant in VARIANTS:
        res = run_layer(L.device(variant), xd, to_dev(lg), spec.k)
        y, _, _ = _gather_forward(L.device(variant), xd, res, spec.k, False)
        assert torch.equal(y, res["y_perm"]), f"variant {variant}"


def _without_lora(L):
    import copy
    W = copy.copy(L.W)
    W.lora_A = W.lora_B = None
    W._cache = {}
    return W


def test_auto_variant_choice():
    # decode-sized rows per expert pick the skinny kernel, prefill-sized the tiled one
    L = layer_of(QWEN_SMALL)
    for T, want in ((5, moe4.MOE4_VARIANT_SKINNY), (100, moe4.MOE4_VARIANT_TILED)):
        x, lg = inp.host_tokens(QWEN_SMALL, T)
        res = run_layer(L.device(), to_dev(x), to_dev(lg), QWEN_SMALL.k)
        assert res["variant"] == want


@pytest.mark.parametrize("T", [300, 320, 321, 700])
def test_forward_single_expert_overflow_rows(T):
    """All tokens on two experts: the skinny kernel loops over row chunks; the
    tiled kernel takes 320 rows in one tile and cuts 321 rows into two (161 +
    160), and at T=700 each expert into three equal tiles (of up to 320 rows),
    which the largest-first order deals with the other experts' empty ones."""
    spec = inp.TINY_NF4
    L = layer_of(spec)
    x, _ = inp.host_tokens(spec, T)
    lg = np.full((T, spec.E), -5.0, np.float32)
    lg[:, 3] = 5.0
    lg[:, 6] = 4.0
    ri, rw = oracle.route(lg, spec.k)
    ref = oracle.layer_forward(x, ri, rw, L.W)
    for variant in (moe4.MOE4_VARIANT_SKINNY, moe4.MOE4_VARIANT_TILED):
        say(f"forward skewed T={T} variant={variant}")
        res = run_layer(L.device(variant), to_dev(x), to_dev(lg), spec.k)
        assert_close(res["out32"].cpu().numpy(), ref["out"], f"out skewed T={T} v{variant}")


def test_forward_deterministic():
    spec = GPTOSS_SMALL
    L = layer_of(spec)
    x, lg = inp.host_tokens(spec, 200)
    ex = L.device()
    a = run_layer(ex, to_dev(x), to_dev(lg), spec.k)
    b = run_layer(ex, to_dev(x), to_dev(lg), spec.k)
    for key in ("idx", "offsets", "slot_of_row", "x_perm", "y_perm", "out"):
        assert torch.equal(a[key].view(torch.int16) if a[key].dtype == torch.bfloat16 else a[key],
                           b[key].view(torch.int16) if b[key].dtype == torch.bfloat16 else b[key]), key


def test_empty_inputs():
    say("empty: T = 0")
    spec = inp.TINY_NF4
    L = layer_of(spec)
    ex = L.device()
    e = torch.empty(0, dtype=torch.int32, device=DEV)
    lg = torch.empty((0, spec.E), dtype=torch.float32, device=DEV)
    idx = torch.empty((0, spec.k), dtype=torch.int32, device=DEV)
    w = torch.empty((0, spec.k), dtype=torch.float32, device=DEV)
    moe4.moe4_route(lg, spec.k, idx, w)
    offsets = torch.full((spec.E + 1,), 7, dtype=torch.int32, device=DEV)
    ws = torch.empty(moe4.moe4_workspace_size(ex, 0, spec.k), dtype=torch.uint8, device=DEV)
    moe4.moe4_permute(idx, spec.E, offsets, e, e, ws=ws)
    xp = torch.empty((0, spec.H), dtype=torch.bfloat16, device=DEV)
    yp = torch.empty((0, spec.H), dtype=torch.float32, device=DEV)
    moe4.moe4_expert_forward(ex, xp, offsets, yp, ws=ws)
    out = torch.empty((0, spec.H), dtype=torch.bfloat16, device=DEV)
    moe4.moe4_combine(yp, e, w, out, spec.k)
    torch.cuda.synchronize()
    assert torch.all(offsets == 0)


# ----------------------------------------------------------------- backward

# one expert at top-1 with an adapter: the backward of a dense 4-bit QLoRA MLP
DENSE_LORA = inp.QWEN3_30B_NF4_LORA.scaled(name="dense_lora_E1_k1", seed_id=112, E=1, k=1,
                                           H=128, I=64, tokens=(50,), lora_r=4,
                                           lora_alpha=8.0)
# and its MXFP4 counterpart (biases, interleaved rows, clamped GLU), and every
# expert chosen with an adapter (k = E = 2)
DENSE_MXFP4_LORA = inp.GPT_OSS_20B_MXFP4.scaled(name="dense_mxfp4_lora_E1_k1", seed_id=113, E=1,
                                                k=1, H=96, I=64, tokens=(30,), lora_r=4,
                                                lora_alpha=8.0)
ALLEXP_LORA = inp.QWEN3_30B_NF4_LORA.scaled(name="all_experts_lora_E2_k2", seed_id=114, E=2,
                                            k=2, H=128, I=64, tokens=(45,), lora_r=8,
                                            lora_alpha=16.0)
WIDE_LORA = inp.QWEN3_30B_NF4_LORA.scaled(name="wide_lora_E160_k2", seed_id=117, E=160, k=2,
                                          H=128, I=64, tokens=(40,), lora_r=4, lora_alpha=8.0)
# the dgrad kernels' column groups of 512 and row tiles of 160: a second
# column group of 64 (NF4) or 32 (MXFP4) columns, where whole waves have no
# column and one wave (MXFP4) only half its lanes; an output width of 96
# (MXFP4 gate_up dgrad: one and a half waves); a reduction of 96 (MXFP4 down
# dgrad: one and a half k-tiles); Zipf-skewed rows, so that hot experts take
# two row tiles
COLGROUP_NF4_LORA = inp.QWEN3_30B_NF4_LORA.scaled(name="lora_nf4_H128_I576_zipf", seed_id=150,
                                                  E=4, k=2, H=128, I=576, tokens=(200,),
                                                  zipf=1.1)
COLGROUP_MXFP4_LORA = inp.GPT_OSS_20B_MXFP4.scaled(name="lora_mxfp4_H96_I544_zipf", seed_id=151,
                                                   E=4, k=2, H=96, I=544, tokens=(200,),
                                                   lora_r=4, lora_alpha=8.0, zipf=1.1)
BWD_CASES = [(LORA_SMALL, 150), (MXFP4_LORA_SMALL, 40), (DENSE_LORA, 50), (DENSE_MXFP4_LORA, 30),
             (ALLEXP_LORA, 45), (WIDE_LORA, 40), (COLGROUP_NF4_LORA, 200),
             (COLGROUP_MXFP4_LORA, 200)]


@pytest.mark.parametrize("T", [256, 257, 300])
def test_layer_backward_skewed(T):
    """All tokens on two experts (T rows each): the dgrad kernels (tiles of at
    most 160 rows) cut 256 rows into two of 128, 257 into 160 + 97 and 300
    into 160 + 140, and the adapter reductions run over long row ranges."""
    spec = LORA_SMALL
    say(f"backward skewed {spec.name} T={T}")
    L = layer_of(spec)
    ex = L.device()
    x, _ = inp.host_tokens(spec, T)
    lg = np.full((T, spec.E), -5.0, np.float32)
    lg[:, 2] = 5.0
    lg[:, 5] = 4.0
    dout = inp.host_upstream_grad(spec, T)
    res = run_layer(ex, to_dev(x), to_dev(lg), spec.k, save=True)
    S = T * spec.k
    dy = torch.empty((S, spec.H), dtype=torch.bfloat16, device=DEV)
    e0 = torch.empty(S, dtype=torch.int32, device=DEV)
    moe4.moe4_permute(res["idx"], spec.E, torch.empty_like(res["offsets"]), e0,
                      torch.empty_like(e0), x=to_dev(dout), row_scale=res["w"].reshape(-1),
                      x_perm=dy, ws=res["ws"])
    dx_perm = torch.empty((S, spec.H), dtype=torch.float32, device=DEV)
    dA = torch.full((spec.E, spec.lora_r, spec.H), float("nan"), device=DEV)
    dB = torch.full((spec.E, 2 * spec.I, spec.lora_r), float("nan"), device=DEV)
    moe4.moe4_expert_backward(ex, res["x_perm"], res["offsets"], res["save_gu"], res["save_xa"],
                              dy, dx_perm, dA, dB, ws=res["ws"])
    torch.cuda.synchronize()
    ri, rw = oracle.route(lg, spec.k)
    ref = oracle.layer_backward(x, ri, rw, dout, L.W)
    assert_close(dx_perm.cpu().numpy(), ref["dx_perm"], "dx_perm")
    dA_h, dB_h = dA.cpu().numpy(), dB.cpu().numpy()
    for e in range(spec.E):
        if e not in (2, 5):
            assert np.all(dA_h[e] == 0) and np.all(dB_h[e] == 0)
    assert_close(dA_h, ref["dA"], "dA")
    assert_close(dB_h, ref["dB"], "dB")


def gpu_backward(spec, ex, x, lg, dout):
    """Forward (saving gu and xa), the row-scaled gather of dOut, the expert
    backward and the dX combine, on the GPU."""
    T = x.shape[0]
    res = run_layer(ex, to_dev(x), to_dev(lg), spec.k, save=True)
    S = T * spec.k
    dy = torch.empty((S, spec.H), dtype=torch.bfloat16, device=DEV)
    e0 = torch.empty(S, dtype=torch.int32, device=DEV)
    moe4.moe4_permute(res["idx"], spec.E, torch.empty_like(res["offsets"]), e0,
                      torch.empty_like(e0), x=to_dev(dout), row_scale=res["w"].reshape(-1),
                      x_perm=dy, ws=res["ws"])
    dx_perm = torch.empty((S, spec.H), dtype=torch.float32, device=DEV)
    dA = torch.full((spec.E, spec.lora_r, spec.H), float("nan"), device=DEV)
    dB = torch.full((spec.E, 2 * spec.I, spec.lora_r), float("nan"), device=DEV)
    moe4.moe4_expert_backward(ex, res["x_perm"], res["offsets"], res["save_gu"], res["save_xa"],
                              dy, dx_perm, dA, dB, ws=res["ws"])
    dx = torch.empty((T, spec.H), dtype=torch.float32, device=DEV)
    moe4.moe4_combine(dx_perm, res["row_of_slot"], None, dx, spec.k)
    torch.cuda.synchronize()
    return dict(res=res, dy=dy, dx_perm=dx_perm, dA=dA, dB=dB, dx=dx)


def check_backward(spec, L, T):
    ex = L.device()
    x, lg = inp.host_tokens(spec, T)
    dout = inp.host_upstream_grad(spec, T)
    g = gpu_backward(spec, ex, x, lg, dout)
    ri, rw = oracle.route(lg, spec.k)
    # the row-scaled gather is bit-exact with the oracle's definition
    _, rs, _ = oracle.permute(ri, spec.E)
    assert np.array_equal(bits(g["dy"]), oracle.gather_rows(
        dout, rs, spec.k, row_scale=g["res"]["w"].cpu().numpy().reshape(-1)))
    ref = backward_reference(x, ri, rw, dout, L.W, g["res"]["save_gu"].cpu().numpy(),
                             g["dx_perm"].cpu().numpy())
    assert_close(g["dx_perm"].cpu().numpy(), ref["dx_perm"], "dx_perm")
    assert_close(g["dx"].cpu().numpy(), ref["dx"], "dx")
    dA_h, dB_h = g["dA"].cpu().numpy(), g["dB"].cpu().numpy()
    counts = np.bincount(ri.reshape(-1), minlength=spec.E)
    for e in range(spec.E):
        if counts[e] == 0:
            assert np.all(dA_h[e] == 0) and np.all(dB_h[e] == 0)
    assert_close(dA_h, ref["dA"], "dA")
    assert_close(dB_h, ref["dB"], "dB")


@pytest.mark.parametrize("spec,T", BWD_CASES, ids=[s.name for s, _ in BWD_CASES])
def test_layer_backward(spec, T):
    say(f"backward {spec.name} T={T}")
    check_backward(spec, layer_of(spec), T)


@pytest.mark.parametrize("spec", RANK_NF4 + RANK_MXFP4, ids=[s.name for s in RANK_NF4 + RANK_MXFP4])
def test_layer_backward_lora_ranks(spec):
    say(f"backward {spec.name} (r={spec.lora_r}, scale {spec.lora_scale:g}) T={spec.tokens[0]}")
    check_backward(spec, layer_of(spec), spec.tokens[0])


@pytest.mark.parametrize("spec,T", [(LORA_SMALL, 150), (MXFP4_LORA_SMALL, 40)],
                         ids=["nf4", "mxfp4"])
def test_backward_deterministic(spec, T):
    """Two backward passes of one batch agree bit for bit: the dgrad kernels,
    the rank projection and the adapter-gradient reductions sum in a fixed
    order (no atomics)."""
    say(f"backward run twice, bitwise: {spec.name} T={T}")
    L = layer_of(spec)
    ex = L.device()
    x, lg = inp.host_tokens(spec, T)
    dout = inp.host_upstream_grad(spec, T)
    a = gpu_backward(spec, ex, x, lg, dout)
    b = gpu_backward(spec, ex, x, lg, dout)
    for key in ("dy", "dx_perm", "dA", "dB", "dx"):
        ta, tb = a[key], b[key]
        if ta.dtype == torch.bfloat16:
            ta, tb = ta.view(torch.int16), tb.view(torch.int16)
        assert torch.equal(ta, tb), key
    for key in ("save_gu", "save_xa", "y_perm"):
        assert torch.equal(a["res"][key], b["res"][key]), key


def test_route_backward_deterministic():
    say("route_backward run twice, bitwise")
    T, E, k, H = 300, 128, 8, 2048
    spec = inp.QWEN3_30B_NF4.scaled(name="route_bwd_det", seed_id=119, E=E, k=k, H=H)
    _, lg = inp.host_tokens(spec, T)
    ri, rw = oracle.route(lg, k)
    _, _, row_of_slot = oracle.permute(ri, E)
    args = [to_dev(ri.astype(np.int32)), to_dev(rw.astype(np.float32)),
            to_dev(inp.host_upstream_grad(spec, T)), to_dev(inp.host_slot_outputs(spec, T)),
            to_dev(row_of_slot)]
    outs = []
    for _ in range(2):
        dw = torch.empty((T, k), dtype=torch.float32, device=DEV)
        dl = torch.empty((T, E), dtype=torch.float32, device=DEV)
        moe4.moe4_route_backward(*args, dw, dl)
        torch.cuda.synchronize()
        outs.append((dw, dl))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
