"""Pins for the oracle's routing and permutation: exhaustive subset search,
a library softmax, Python's stable sort, and a library bf16 cast."""
import itertools

import numpy as np
import pytest
import torch
from scipy.special import softmax

from oracle import route, permute, gather_rows


def _beats(a, ia, b, ib):
    """Total order of the selection: larger logit first, then lower index."""
    return a > b or (a == b and ia < ib)


def test_route_is_the_unique_dominating_subset():
    rng = np.random.default_rng(6)
    for trial in range(60):
        E = int(rng.integers(1, 8))
        k = int(rng.integers(1, E + 1))
        T = 4
        lg = rng.standard_normal((T, E)).astype(np.float32)
        if trial % 3 == 0:   # force ties and signed zeros
            lg = rng.integers(-2, 3, (T, E)).astype(np.float32)
            lg[lg == 0] = np.where(rng.random((lg == 0).sum()) < 0.5, 0.0, -0.0)
        idx, w = route(lg, k)
        for t in range(T):
            good = [S for S in itertools.combinations(range(E), k)
                    if all(_beats(lg[t, i], i, lg[t, j], j)
                           for i in S for j in range(E) if j not in S)]
            assert len(good) == 1
            assert sorted(idx[t].tolist()) == list(good[0])
            # selection order: each slot beats the next
            for j in range(k - 1):
                assert _beats(lg[t, idx[t, j]], idx[t, j], lg[t, idx[t, j + 1]], idx[t, j + 1])


def test_route_weights_match_library_softmax():
    rng = np.random.default_rng(7)
    lg = rng.standard_normal((16, 32)).astype(np.float32)
    # k = E without renormalisation is the full softmax, in selection order
    idx, w = route(lg, 32, renormalize=False)
    ref = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(ref, idx.astype(np.int64), 1), rtol=1e-13, atol=0)
    # renormalised top-k equals the softmax of the selected logits alone
    idx, w = route(lg, 4)
    sel = np.take_along_axis(lg.astype(np.float64), idx.astype(np.int64), 1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=1e-13, atol=0)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_route_rejects_bad_k_and_nan():
    with pytest.raises(ValueError):
        route(np.zeros((2, 4), np.float32), 5)
    lg = np.zeros((1, 4), np.float32)
    lg[0, 1] = np.nan
    with pytest.raises(ValueError):
        route(lg, 2)


def test_permute_matches_python_sorted():
    rng = np.random.default_rng(8)
    for E, T, k in [(1, 5, 1), (8, 64, 2), (13, 37, 4), (128, 50, 8)]:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
        offsets, slot_of_row, row_of_slot = permute(idx, E)
        keys = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k))
        assert slot_of_row.tolist() == [t * k + j for _, t, j in keys]
        assert np.array_equal(row_of_slot[slot_of_row], np.arange(T * k))
        assert offsets[0] == 0 and offsets[E] == T * k
        for e in range(E):
            rows = slot_of_row[offsets[e]:offsets[e + 1]]
            assert np.all(idx.reshape(-1)[rows] == e)


def test_gather_rows_plain_and_scaled():
    rng = np.random.default_rng(9)
    T, k, H = 6, 3, 16
    x32 = rng.standard_normal((T, H)).astype(np.float32)
    xb = torch.from_numpy(x32).to(torch.bfloat16)
    x_bits = xb.view(torch.int16).numpy().view(np.uint16)
    idx = rng.integers(0, 4, (T, k)).astype(np.int32)
    _, slot_of_row, _ = permute(idx, 4)
    got = gather_rows(x_bits, slot_of_row, k)
    assert np.array_equal(got, x_bits[slot_of_row // k])
    scale = rng.random(T * k).astype(np.float32)
    got = gather_rows(x_bits, slot_of_row, k, row_scale=scale)
    # library path: fp32 product (torch, IEEE) then torch's bf16 cast
    prod = torch.from_numpy(scale[slot_of_row])[:, None] * xb.float()[torch.from_numpy(slot_of_row // k)]
    ref = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
