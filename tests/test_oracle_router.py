"""Pins for the oracle's router step: exact brute-force dot products (Python's
math.fsum over library bf16 decodes), fp32 summations in several orders
against the error bound, torch float64 autograd through the routing softmax,
and central finite differences."""
import math

import numpy as np
import pytest
import torch

from oracle import (route, router_logits, router_logits_error_bound, routing_weight_grad,
                    routing_logit_grad, permute)


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _bf16_vals(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(
        torch.bfloat16).double().numpy()


def test_router_logits_brute_force():
    rng = np.random.default_rng(30)
    T, E, H = 3, 5, 24
    xb = _bf16_bits(rng.standard_normal((T, H)))
    wb = _bf16_bits(rng.standard_normal((E, H)) / np.sqrt(H))
    b = rng.standard_normal(E).astype(np.float32)
    x, w = _bf16_vals(xb), _bf16_vals(wb)
    got = router_logits(xb, wb, b)
    for t in range(T):
        for e in range(E):
            ref = math.fsum([x[t, h] * w[e, h] for h in range(H)] + [float(b[e])])
            assert abs(got[t, e] - ref) <= 1e-15 * max(1.0, abs(ref))
    assert np.array_equal(router_logits(xb, wb), router_logits(xb, wb, np.zeros(E, np.float32)))


def test_router_logits_bound_holds_for_fp32_orders():
    rng = np.random.default_rng(31)
    T, E, H = 8, 16, 2048
    xb = _bf16_bits(rng.standard_normal((T, H)))
    wb = _bf16_bits(rng.standard_normal((E, H)) / np.sqrt(H))
    exact = router_logits(xb, wb)
    bound = router_logits_error_bound(xb, wb)
    prods = (_bf16_vals(xb)[:, None, :] * _bf16_vals(wb)[None, :, :]).astype(np.float32)
    assert np.array_equal(prods.astype(np.float64),
                          _bf16_vals(xb)[:, None, :] * _bf16_vals(wb)[None, :, :])
    orders = [np.arange(H), np.arange(H)[::-1], rng.permutation(H)]
    worst = 0.0
    for o in orders:
        acc = np.zeros((T, E), np.float32)
        for h in o:                       # sequential fp32 accumulation
            acc = (acc + prods[:, :, h]).astype(np.float32)
        err = np.abs(acc.astype(np.float64) - exact)
        assert np.all(err <= bound)
        worst = max(worst, float(np.max(err / bound)))
    # pairwise (tree) fp32 summation
    v = prods.copy()
    while v.shape[-1] > 1:
        v = (v[..., 0::2] + v[..., 1::2]).astype(np.float32)
    assert np.all(np.abs(v[..., 0].astype(np.float64) - exact) <= bound)
    # the bound is a worst case: real errors sit far inside it (by orders of
    # magnitude), and it stays small against the logits' unit spread
    assert worst < 0.05
    assert np.max(bound) < 5e-3


def _torch_chain(lg, idx, y, dout, renormalize):
    """float64 autograd: logits -> softmax -> top-k weights -> out -> <dOut, out>."""
    L = torch.tensor(lg, dtype=torch.float64, requires_grad=True)
    p = torch.softmax(L, dim=1)
    w = torch.gather(p, 1, torch.from_numpy(idx.astype(np.int64)))
    if renormalize:
        w = w / w.sum(dim=1, keepdim=True)
    w.retain_grad()
    out = (w[:, :, None] * torch.from_numpy(y)).sum(dim=1)
    loss = (out * torch.from_numpy(dout)).sum()
    loss.backward()
    return L.grad.numpy(), w.grad.numpy(), w.detach().numpy()


@pytest.mark.parametrize("renormalize", [True, False])
def test_routing_gradients_match_torch_autograd(renormalize):
    rng = np.random.default_rng(32)
    T, E, k, H = 6, 10, 3, 16
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = route(lg, k, renormalize=renormalize)
    dout_bits = _bf16_bits(rng.standard_normal((T, H)))
    y_slots = rng.standard_normal((T, k, H))       # expert output of slot (t, j)
    # lay the slot outputs out in permuted-row order, as the layer stores them
    _, slot_of_row, row_of_slot = permute(idx, E)
    y_perm = y_slots.reshape(T * k, H)[slot_of_row]
    dw = routing_weight_grad(dout_bits, y_perm, row_of_slot, k)
    dl = routing_logit_grad(idx, w, dw, E, renormalize=renormalize, logits=lg)
    gl, gw, wt = _torch_chain(lg, idx, y_slots, _bf16_vals(dout_bits), renormalize)
    assert np.allclose(wt, w, rtol=1e-12, atol=0)
    assert np.allclose(dw, gw, rtol=1e-12, atol=1e-12)
    assert np.allclose(dl, gl, rtol=1e-10, atol=1e-12)
    if renormalize:
        assert np.allclose(dl.sum(axis=1), 0.0, atol=1e-12)
        mask = np.ones((T, E), bool)
        np.put_along_axis(mask, idx.astype(np.int64), False, 1)
        assert np.all(dl[mask] == 0)


def test_routing_logit_grad_finite_differences():
    rng = np.random.default_rng(33)
    T, E, k = 4, 8, 3
    lg = rng.standard_normal((T, E))
    idx, _ = route(lg.astype(np.float32), k)
    c = rng.standard_normal((T, k))

    def f(L, renorm):
        out = 0.0
        for t in range(T):
            z = np.exp(L[t] - L[t].max())
            p = z / z.sum()
            ws = p[idx[t]]
            if renorm:
                ws = ws / ws.sum()
            out += float(np.dot(ws, c[t]))
        return out

    for renorm in (True, False):
        _, w = route(lg.astype(np.float32), k, renormalize=renorm)
        # the weights of float64 logits: recompute at the fp64 point itself
        z = np.exp(lg - lg.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, idx.astype(np.int64), 1)
        if renorm:
            w = w / w.sum(axis=1, keepdims=True)
        dl = routing_logit_grad(idx, w, c, E, renormalize=renorm, logits=lg.astype(np.float32))
        eps = 1e-6
        num = np.zeros((T, E))
        for t in range(T):
            for e in range(E):
                Lp, Lm = lg.copy(), lg.copy()
                Lp[t, e] += eps
                Lm[t, e] -= eps
                num[t, e] = (f(Lp, renorm) - f(Lm, renorm)) / (2 * eps)
        if not renorm:
            # the closed form uses p from the fp32-rounded logits: compare at
            # that precision
            assert np.allclose(dl, num, rtol=1e-5, atol=1e-7)
        else:
            assert np.allclose(dl, num, rtol=1e-6, atol=1e-9)
