"""Pins for the oracle's expert layer.

* brute force on tiny inputs: an independent loop implementation that decodes
  every weight from the raw packed bytes (NF4 and MXFP4), with its own nibble,
  absmax/scale indexing, gate/up split, activation and combine;
* a special case that reduces to a library routine: one expert, k=1, plain
  SwiGLU, HALVES is a dense SwiGLU MLP written with torch.nn.functional.silu;
* closed forms of the activations at special points;
* LoRA-only special case (zero base) against a torch matmul;
* the backward against float64 central finite differences of the forward and
  against torch float64 autograd.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (ExpertWeights, layer_forward, layer_backward, token_forward,
                    route, quantize_nf4, activation, combine, bf16_round_f64)
from oracle.layer import HALVES, INTERLEAVED, SWIGLU, SWIGLU_CLAMPED, activation_backward
from tests.conftest import read_golden

NF4_GOLD = [float(r[0]) for r in read_golden("nf4_levels.txt")]
E2M1_GOLD = {int(n): float(v) for n, v in read_golden("e2m1_values.txt")}


def _bits_to_float(b):
    return float(np.array([b], np.uint16).astype(np.uint32).__lshift__(16).view(np.float32)[0])


def _bf16(a, rng=None):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z)) if z >= 0 else math.exp(z) / (1.0 + math.exp(z))


# ---------------------------------------------------------- brute force loops

def _torch_bf16(v):
    """fp32 value -> nearest bf16 (torch's CPU cast, an independent library)."""
    return float(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).float()[0])


def _nf4_w(packed, absmax, e, n, kk):
    byte = int(packed[e, n, kk // 2])
    nib = byte & 15 if kk % 2 == 0 else byte >> 4
    # the bf16 GEMM operand: one fp32 product, one rounding
    return _torch_bf16(np.float32(NF4_GOLD[nib]) * np.float32(absmax[e, n, kk // 64]))


def _mx_w(blocks, scales, e, n, kk):
    byte = int(blocks[e, n, kk // 32, (kk % 32) // 2])
    nib = byte & 15 if kk % 2 == 0 else byte >> 4
    return E2M1_GOLD[nib] * 2.0 ** (int(scales[e, n, kk // 32]) - 127)


def _brute_layer(x_bits, idx, w, wfun_gu, wfun_dn, H, I, layout, act, b_gu=None, b_dn=None,
                 A=None, B=None, scale=0.0, alpha=1.702, limit=7.0):
    T, k = idx.shape
    out = [[0.0] * H for _ in range(T)]
    for t in range(T):
        x = [_bits_to_float(x_bits[t, c]) for c in range(H)]
        for j in range(k):
            e = int(idx[t, j])
            gu = []
            for n in range(2 * I):
                acc = sum(x[c] * wfun_gu(e, n, c) for c in range(H))
                if b_gu is not None:
                    acc += _bits_to_float(b_gu[e, n])
                gu.append(acc)
            if A is not None:
                r = A.shape[1]
                xa = [sum(x[c] * _bits_to_float(A[e, q, c]) for c in range(H)) for q in range(r)]
                xa = [float(bf16_round_f64(v)) for v in xa]
                for n in range(2 * I):
                    gu[n] += scale * sum(xa[q] * _bits_to_float(B[e, n, q]) for q in range(r))
            h = []
            for i in range(I):
                g, u = (gu[i], gu[I + i]) if layout == HALVES else (gu[2 * i], gu[2 * i + 1])
                if act == SWIGLU:
                    h.append(g * _sig(g) * u)
                else:
                    gc, uc = min(g, limit), max(-limit, min(u, limit))
                    h.append((uc + 1.0) * gc * _sig(alpha * gc))
                h[-1] = float(bf16_round_f64(h[-1]))
            for c in range(H):
                y = sum(h[i] * wfun_dn(e, c, i) for i in range(I))
                if b_dn is not None:
                    y += _bits_to_float(b_dn[e, c])
                out[t][c] += float(w[t, j]) * y
    return np.array(out)


def _tiny_nf4(rng, E, H, I, lora_r=0):
    gq, ga, dq, da = [], [], [], []
    for e in range(E):
        p, a = quantize_nf4((rng.standard_normal(2 * I * H) * 0.05).astype(np.float32))
        gq.append(p.reshape(2 * I, H // 2))
        ga.append(a.reshape(2 * I, H // 64))
        p, a = quantize_nf4((rng.standard_normal(H * I) * 0.05).astype(np.float32))
        dq.append(p.reshape(H, I // 2))
        da.append(a.reshape(H, I // 64))
    out = [np.stack(v) for v in (gq, ga, dq, da)]
    if lora_r:
        out.append(_bf16(rng.standard_normal((E, lora_r, H)) / math.sqrt(H)))
        out.append(_bf16(rng.standard_normal((E, 2 * I, lora_r)) * 0.05))
    return out


def test_forward_brute_force_nf4_halves_lora():
    rng = np.random.default_rng(10)
    E, H, I, T, k, r = 3, 64, 64, 4, 2, 3
    gq, ga, dq, da, A, B = _tiny_nf4(rng, E, H, I, lora_r=r)
    x = _bf16(rng.standard_normal((T, H)))
    idx, w = route(rng.standard_normal((T, E)).astype(np.float32), k)
    W = ExpertWeights.from_nf4(gq, ga, dq, da, layout=HALVES, act=SWIGLU, lora_A=A, lora_B=B,
                               lora_scale=2.0)
    got = layer_forward(x, idx, w, W)["out"]
    ref = _brute_layer(x, idx, w, lambda e, n, c: _nf4_w(gq, ga, e, n, c),
                       lambda e, n, c: _nf4_w(dq, da, e, n, c), H, I, HALVES, SWIGLU,
                       A=A, B=B, scale=2.0)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)
    # the per-token path agrees with the whole-layer path
    for t in range(T):
        assert np.allclose(token_forward(x[t], idx[t], w[t], W), got[t], rtol=1e-12, atol=1e-14)


def test_forward_brute_force_mxfp4_interleaved_clamped_bias():
    rng = np.random.default_rng(11)
    E, H, I, T, k = 3, 64, 32, 3, 2
    gb = rng.integers(0, 256, (E, 2 * I, H // 32, 16), dtype=np.uint8)
    gs = rng.integers(118, 124, (E, 2 * I, H // 32), dtype=np.uint8)
    db = rng.integers(0, 256, (E, H, I // 32, 16), dtype=np.uint8)
    ds = rng.integers(118, 124, (E, H, I // 32), dtype=np.uint8)
    bg = _bf16(rng.standard_normal((E, 2 * I)) * 0.5)
    bd = _bf16(rng.standard_normal((E, H)) * 0.5)
    x = _bf16(rng.standard_normal((T, H)) * 4)
    idx, w = route(rng.standard_normal((T, E)).astype(np.float32), k)
    W = ExpertWeights.from_mxfp4(gb, gs, db, ds, layout=INTERLEAVED, act=SWIGLU_CLAMPED,
                                 gu_bias=bg, dn_bias=bd, alpha=1.702, limit=7.0)
    res = layer_forward(x, idx, w, W, keep=True)
    # the clamp is exercised on both sides
    g, u = res["gu"][:, 0::2], res["gu"][:, 1::2]
    assert (g > 7).any() and (u > 7).any() and (u < -7).any()
    ref = _brute_layer(x, idx, w, lambda e, n, c: _mx_w(gb, gs, e, n, c),
                       lambda e, n, c: _mx_w(db, ds, e, n, c), H, I, INTERLEAVED,
                       SWIGLU_CLAMPED, b_gu=bg, b_dn=bd)
    assert np.allclose(res["out"], ref, rtol=1e-10, atol=1e-12)


def test_single_expert_reduces_to_library_swiglu_mlp():
    rng = np.random.default_rng(12)
    H, I, T = 128, 64, 5
    gq, ga, dq, da = _tiny_nf4(rng, 1, H, I)
    W = ExpertWeights.from_nf4(gq, ga, dq, da, layout=HALVES, act=SWIGLU, bf16_weights=False)
    x = _bf16(rng.standard_normal((T, H)))
    idx = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1))
    got = layer_forward(x, idx, w, W, exact=True)["out"]
    Wgu, Wd = (torch.from_numpy(a) for a in W.expert(0))
    xt = torch.from_numpy(x.astype(np.uint32) << 16).view(torch.float32).double()
    ref = (torch.nn.functional.silu(xt @ Wgu[:I].T) * (xt @ Wgu[I:].T)) @ Wd.T
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-14)


# ------------------------------------------------------- activation closed forms

def _act(gs, us, layout=HALVES, act=SWIGLU, alpha=1.702, limit=7.0):
    I = len(gs)
    W = ExpertWeights(E=1, H=1, I=I, layout=layout, act=act, gu=None, dn=None,
                      alpha=alpha, limit=limit)
    gu = np.array([list(gs) + list(us)]) if layout == HALVES else \
        np.array([[v for p in zip(gs, us) for v in p]])
    return activation(gu, W)[0]


def test_swiglu_special_points():
    ln3 = math.log(3.0)   # sigmoid(ln 3) = 3/4
    h = _act([0.0, 40.0, -40.0, ln3, 1.0], [5.0, 3.0, 3.0, 2.0, 0.0])
    assert h[0] == 0.0
    assert abs(h[1] - 120.0) < 1e-12          # sigmoid -> 1: h -> g*u
    assert abs(h[2]) < 1e-15                   # sigmoid -> 0
    assert abs(h[3] - ln3 * 0.75 * 2.0) < 1e-15
    assert h[4] == 0.0                         # up = 0
    # interleaved: even entries are gate
    hi = _act([ln3], [2.0], layout=INTERLEAVED)
    assert abs(hi[0] - ln3 * 0.75 * 2.0) < 1e-15


def test_clamped_glu_special_points():
    a, L = 1.702, 7.0
    sig7 = 1.0 / (1.0 + math.exp(-a * 7.0))
    h = _act([100.0, 100.0, 100.0, 0.0, 2.0, 7.0], [0.0, 100.0, -100.0, 5.0, -1.0, 7.0],
             act=SWIGLU_CLAMPED)
    assert abs(h[0] - 7.0 * sig7) < 1e-12            # g clamped to 7, (0 + 1) factor
    assert abs(h[1] - 8.0 * 7.0 * sig7) < 1e-12      # u clamped to +7
    assert abs(h[2] + 6.0 * 7.0 * sig7) < 1e-12      # u clamped to -7
    assert h[3] == 0.0                               # g = 0
    assert h[4] == 0.0                               # u = -1 cancels the +1 term
    assert abs(h[5] - 8.0 * 7.0 * sig7) < 1e-12      # at the limit the clamp is idle
    # the gate is clamped from above only
    h = _act([-30.0], [0.0], act=SWIGLU_CLAMPED)
    assert h[0] < 0 and abs(h[0] + 30.0 / (1.0 + math.exp(a * 30.0))) < 1e-20


def test_combine_k1_unit_weight_is_identity_and_plain_sum():
    rng = np.random.default_rng(13)
    y = rng.standard_normal((6, 8))
    row_of_slot = rng.permutation(6).astype(np.int32)
    out = combine(y, row_of_slot, np.ones((6, 1)), 6, 1)
    assert np.array_equal(out, y[row_of_slot])
    out = combine(y, row_of_slot, None, 3, 2)
    assert np.array_equal(out, y[row_of_slot[0::2]] + y[row_of_slot[1::2]])


def test_lora_only_special_case():
    rng = np.random.default_rng(14)
    E, H, I, T, r = 2, 64, 64, 3, 4
    zq = np.full((E, 2 * I, H // 2), 0x77, np.uint8)     # every code 7 (level 0)
    za = np.zeros((E, 2 * I, H // 64), np.float32)
    dq = np.full((E, H, I // 2), 0x77, np.uint8)
    dA = np.zeros((E, H, I // 64), np.float32)
    A = _bf16(rng.standard_normal((E, r, H)))
    B = _bf16(rng.standard_normal((E, 2 * I, r)))
    W = ExpertWeights.from_nf4(zq, za, dq, dA, layout=HALVES, act=SWIGLU,
                               lora_A=A, lora_B=B, lora_scale=2.0)
    x = _bf16(rng.standard_normal((T, H)))
    idx = np.array([[1], [0], [1]], np.int32)
    res = layer_forward(x, idx, np.ones((T, 1)), W, keep=True, exact=True)
    xt = torch.from_numpy(x.astype(np.uint32) << 16).view(torch.float32).double()
    At = torch.from_numpy(A.astype(np.uint32) << 16).view(torch.float32).double()
    Bt = torch.from_numpy(B.astype(np.uint32) << 16).view(torch.float32).double()
    for row in range(T):
        s = int(res["slot_of_row"][row])
        e = int(idx[s, 0])
        ref = 2.0 * torch.linalg.multi_dot([xt[s:s + 1], At[e].T, Bt[e].T])
        assert np.allclose(res["gu"][row], ref.numpy()[0], rtol=1e-12, atol=1e-14)
    assert np.all(res["out"] == 0)   # zero down projection


# ---------------------------------------------------------------- backward

def _dense_layer(rng, E, H, I, r, layout, act, limit=7.0):
    Wg = rng.standard_normal((E, 2 * I, H)) * 0.6
    Wd = rng.standard_normal((E, H, I)) * 0.6
    A = rng.standard_normal((E, r, H)) * 0.5
    B = rng.standard_normal((E, 2 * I, r)) * 0.5
    bg = rng.standard_normal((E, 2 * I)) * 0.3
    W = ExpertWeights(E=E, H=H, I=I, layout=layout, act=act,
                      gu=lambda e: Wg[e], dn=lambda e: Wd[e],
                      b_gu=lambda e: bg[e], b_dn=None,
                      lora_A=lambda e: A[e], lora_B=lambda e: B[e], lora_scale=2.0,
                      alpha=1.702, limit=limit)
    return W, Wg, Wd, A, B, bg


@pytest.mark.parametrize("layout,act,limit", [(HALVES, SWIGLU, 7.0),
                                              (INTERLEAVED, SWIGLU_CLAMPED, 0.7)])
def test_backward_matches_finite_differences(layout, act, limit):
    rng = np.random.default_rng(15)
    E, H, I, r, T, k = 4, 6, 5, 3, 5, 2
    W, Wg, Wd, A, B, bg = _dense_layer(rng, E, H, I, r, layout, act, limit)
    x = rng.standard_normal((T, H))
    dout = rng.standard_normal((T, H))
    idx = np.array([[0, 1], [1, 2], [0, 2], [2, 0], [1, 0]], np.int32)   # expert 3 idle
    w = rng.random((T, k)) + 0.2
    gr = layer_backward(x, idx, w, dout, W, exact=True)
    if act == SWIGLU_CLAMPED:
        gu = layer_forward(x, idx, w, W, keep=True, exact=True)["gu"]
        assert (gu[:, 0::2] > limit).any() and (np.abs(gu[:, 1::2]) > limit).any()

    def loss():
        W._cache.clear()
        return float(np.sum(dout * layer_forward(x, idx, w, W, exact=True)["out"]))

    eps = 1e-6

    def fd(arr, pos):
        old = arr[pos]
        arr[pos] = old + eps
        lp = loss()
        arr[pos] = old - eps
        lm = loss()
        arr[pos] = old
        return (lp - lm) / (2 * eps)

    for pos in np.ndindex(x.shape):
        assert abs(fd(x, pos) - gr["dx"][pos]) < 1e-6 * (1 + abs(gr["dx"][pos]))
    for pos in list(np.ndindex(A.shape))[::3]:
        assert abs(fd(A, pos) - gr["dA"][pos]) < 1e-6 * (1 + abs(gr["dA"][pos]))
    for pos in list(np.ndindex(B.shape))[::3]:
        assert abs(fd(B, pos) - gr["dB"][pos]) < 1e-6 * (1 + abs(gr["dB"][pos]))
    assert np.all(gr["dA"][3] == 0) and np.all(gr["dB"][3] == 0)


def test_clamp_flip_takes_the_neighbouring_side():
    """A flipped clamp entry sitting exactly on a boundary gets the derivative
    of the point one float64 ulp across that boundary (the clamped function
    is continuous there, so only the indicator changes); unflipped entries,
    and every entry of the plain SwiGLU, are untouched."""
    a, L = 1.702, 7.0
    W = ExpertWeights(E=1, H=1, I=4, layout=INTERLEAVED, act=SWIGLU_CLAMPED, gu=None, dn=None,
                      alpha=a, limit=L)
    # pairs (g, u): g on its boundary, u on +limit, u on -limit, an interior point
    g = np.array([[L, 0.5, -2.0, 1.0]])
    u = np.array([[3.0, L, -L, 2.0]])
    gu = np.empty((1, 8))
    gu[:, 0::2], gu[:, 1::2] = g, u
    dh = np.array([[1.5, -0.75, 2.0, 1.25]])
    base = activation_backward(gu, dh, W)
    flip = np.zeros_like(gu, dtype=bool)
    flip[0, 0] = flip[0, 3] = flip[0, 5] = True   # g of pair 0, u of pairs 1 and 2
    got = activation_backward(gu, dh, W, flip)
    across = gu.copy()
    across[0, 0] = np.nextafter(L, np.inf)
    across[0, 3] = np.nextafter(L, np.inf)
    across[0, 5] = np.nextafter(-L, -np.inf)
    want = activation_backward(across, dh, W)
    assert np.allclose(got, want, rtol=1e-13, atol=0)
    assert got[0, 0] == 0 and got[0, 3] == 0 and got[0, 5] == 0 and base[0, 0] != 0
    keep = ~flip
    assert np.array_equal(got[keep], base[keep])
    assert np.array_equal(activation_backward(gu, dh, W, np.zeros_like(flip)), base)
    # and the other direction: a value just outside, flipped, passes like the boundary
    out = across.copy()
    assert np.allclose(activation_backward(out, dh, W, flip), base, rtol=1e-13, atol=0)
    Ws = ExpertWeights(E=1, H=1, I=4, layout=INTERLEAVED, act=SWIGLU, gu=None, dn=None)
    assert np.array_equal(activation_backward(gu, dh, Ws, flip), activation_backward(gu, dh, Ws))


def test_round_flip_takes_the_other_neighbour_of_dgu():
    """round_flip changes exactly the flagged dGU operands, each to the other
    bf16 neighbour of its exact value, and the rest of the backward follows
    from the changed operand: dx_perm moves by the change times the gate_up
    weight row (plus the adapter path)."""
    from oracle import bf16_other_neighbour_f64
    rng = np.random.default_rng(19)
    E, H, I, r, T, k = 2, 64, 32, 4, 6, 2
    W, Wg, *_ = _dense_layer(rng, E, H, I, r, HALVES, SWIGLU)
    W.lora_A = W.lora_B = None
    x = _bf16(rng.standard_normal((T, H)))
    dout = _bf16(rng.standard_normal((T, H)))
    idx, w = route(rng.standard_normal((T, E)).astype(np.float32), k)
    base = layer_backward(x, idx, w, dout, W)
    flip = np.zeros_like(base["dgu"], dtype=bool)
    flip[1, 3] = flip[4, 40] = True
    got = layer_backward(x, idx, w, dout, W, round_flip=flip)
    assert np.array_equal(got["dgu"][~flip], base["dgu"][~flip])
    want = bf16_other_neighbour_f64(base["dgu_exact"][flip])
    assert np.array_equal(got["dgu"][flip], want) and np.all(want != base["dgu"][flip])
    e_of = np.searchsorted(base["offsets"], np.arange(T * k), side="right") - 1
    for (row, col) in ((1, 3), (4, 40)):
        delta = got["dgu"][row, col] - base["dgu"][row, col]
        pred = base["dx_perm"][row] + delta * Wg[e_of[row]][col]
        assert np.allclose(got["dx_perm"][row], pred, rtol=1e-12, atol=1e-12)


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(16)
    E, H, I, r, T, k = 3, 16, 8, 2, 6, 2
    W, Wg, Wd, A, B, bg = _dense_layer(rng, E, H, I, r, HALVES, SWIGLU)
    x = rng.standard_normal((T, H))
    dout = rng.standard_normal((T, H))
    idx, w = route(rng.standard_normal((T, E)).astype(np.float32), k)
    gr = layer_backward(x, idx, w, dout, W, exact=True)
    xt = torch.tensor(x, requires_grad=True)
    At = torch.tensor(A, requires_grad=True)
    Bt = torch.tensor(B, requires_grad=True)
    out = torch.zeros(T, H, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            gu = xt[t] @ torch.from_numpy(Wg[e]).T + torch.from_numpy(bg[e]) \
                + 2.0 * (xt[t] @ At[e].T) @ Bt[e].T
            h = torch.nn.functional.silu(gu[:I]) * gu[I:]
            out[t] = out[t] + float(w[t, j]) * (h @ torch.from_numpy(Wd[e]).T)
    (out * torch.from_numpy(dout)).sum().backward()
    assert np.allclose(gr["dx"], xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(gr["dA"], At.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(gr["dB"], Bt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_rounded_backward_stays_near_exact_backward():
    """The bf16 operand roundings of the backward (dY, dGU, t) move the result
    by bf16-sized amounts only; the exact mode is pinned by finite differences."""
    rng = np.random.default_rng(17)
    E, H, I, r, T, k = 3, 64, 32, 4, 12, 2
    W, *_ = _dense_layer(rng, E, H, I, r, HALVES, SWIGLU)
    x = _bf16(rng.standard_normal((T, H)))
    dout = _bf16(rng.standard_normal((T, H)))
    idx, w = route(rng.standard_normal((T, E)).astype(np.float32), k)
    ex = layer_backward(x, idx, w, dout, W, exact=True)
    rd = layer_backward(x, idx, w, dout, W)
    for key in ("dx", "dA", "dB"):
        rel = np.linalg.norm(rd[key] - ex[key]) / np.linalg.norm(ex[key])
        assert 0 < rel < 2e-2, (key, rel)


def test_bf16_round_f64_is_the_nearest_bf16_value():
    rng = np.random.default_rng(18)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        np.ldexp(rng.random(2000), -130),            # subnormal range
                        np.ldexp(2 * rng.integers(128, 256, 2000) + 1.0, -20)])  # 9-bit odd: exact ties
    r = bf16_round_f64(x)
    # r is a bf16 value
    r32 = r.astype(np.float32)
    assert np.array_equal(r32.astype(np.float64), r)
    bits = r32.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    # no bf16 value is nearer: compare with the neighbours one bf16 ulp away
    # (stepping the magnitude up and down; zero's neighbours are +-2^-133)
    sign = np.where(bits >> 31, -1.0, 1.0)
    mag = (bits & 0x7FFFFFFF).astype(np.int64)
    up = sign * (mag + 0x10000).astype(np.uint32).view(np.float32).astype(np.float64)
    dn = np.where(mag == 0, -np.sign(x) * 2.0 ** -133,
                  sign * np.maximum(mag - 0x10000, 0).astype(np.uint32).view(np.float32))
    d = np.abs(x - r)
    assert np.all(d <= np.abs(x - up)) and np.all(d <= np.abs(x - dn))
    # ties go to the even mantissa
    tie = (d == np.abs(x - up)) | (d == np.abs(x - dn))
    assert tie.any() and np.all(((bits[tie] >> 16) & 1) == 0)
