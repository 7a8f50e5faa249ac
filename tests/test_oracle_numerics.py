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
