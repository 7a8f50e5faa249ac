"""Pins for the oracle's bf16 conversion: torch's CPU float32 -> bfloat16 cast
(round to nearest even) is an independent library routine."""
import numpy as np
import torch

from oracle import bf16_bits_from_f32, bf16_bits_to_f32


def _torch_bits(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_on_random_bits():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    assert np.array_equal(bf16_bits_from_f32(x), _torch_bits(x))


def test_bf16_matches_torch_on_gaussians_and_ties():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(1 << 18).astype(np.float32) * np.float32(3.0)
    # exact halfway cases: low 16 bits = 0x8000, both even and odd kept bits
    hw = ((rng.integers(0, 2**15, 4096, dtype=np.uint32) << 16) | 0x8000).astype(np.uint32)
    x = np.concatenate([x, hw.view(np.float32)])
    x = x[~np.isnan(x)]   # NaN payloads: the oracle emits 0x7FC0 (checked below)
    assert np.array_equal(bf16_bits_from_f32(x), _torch_bits(x))


def test_bf16_specials():
    sp = np.array([0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max,
                   -np.finfo(np.float32).max, 1e-45, -1e-45, 1.0, -2.5], dtype=np.float32)
    assert np.array_equal(bf16_bits_from_f32(sp), _torch_bits(sp))
    assert bf16_bits_from_f32(np.array([np.nan], np.float32))[0] == 0x7FC0
    # round trip of representable values is exact
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f32(b)
    keep = ~np.isnan(v)
    assert np.array_equal(bf16_bits_from_f32(v[keep]), b[keep])


def _bf16_grid():
    """Every finite bf16 value, sorted: all 65536 bit patterns through torch's
    bfloat16 -> float32 conversion (NaNs dropped, the two zeros merged)."""
    b = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    with np.errstate(invalid="ignore"):
        v = b.numpy().astype(np.float64)
    return np.unique(v[np.isfinite(v)])


def test_bf16_other_neighbour_brackets_and_is_adjacent():
    from oracle import bf16_other_neighbour_f64, bf16_round_f64
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-30, 30, 300),
                        np.ldexp(rng.random(40), -130), [1.0 + 2.0 ** -9, -3.0 - 2.0 ** -8]])
    r = bf16_round_f64(x)
    o = bf16_other_neighbour_f64(x)
    grid = _bf16_grid()
    # both are bf16 values, they bracket x, and no bf16 value lies between them:
    # o is the next value of the grid beyond r on x's side
    i = np.searchsorted(grid, r)
    assert np.array_equal(grid[i], r)
    nxt = np.where(x > r, grid[np.minimum(i + 1, grid.size - 1)], grid[np.maximum(i - 1, 0)])
    assert np.array_equal(o, nxt)
    assert np.all((np.minimum(r, o) <= x) & (x <= np.maximum(r, o)))
    # exact ties (9 significant bits, odd): the rounding is even, the other neighbour odd
    t = np.ldexp(2 * rng.integers(128, 256, 50) + 1.0, rng.integers(-20, 20, 50))
    ob = bf16_other_neighbour_f64(t).astype(np.float32).view(np.uint32)
    rb = bf16_round_f64(t).astype(np.float32).view(np.uint32)
    assert np.all((rb >> 16) & 1 == 0) and np.all((ob >> 16) & 1 == 1)
    # a bf16 value has no other neighbour; zero's is +-2^-133 on its side
    b = bf16_round_f64(rng.standard_normal(100))
    assert np.array_equal(bf16_other_neighbour_f64(b), b)
    tiny = np.array([2.0 ** -140, -2.0 ** -140])
    assert np.array_equal(bf16_other_neighbour_f64(tiny), [2.0 ** -133, -2.0 ** -133])
