"""Pins for the oracle's NF4 and MXFP4 codecs.

NF4: the published table (golden fixture) and its construction from normal
quantiles; brute-force nearest-level search; round-trip invariants; a
hand-packed byte. MXFP4: exhaustive enumeration of all 256 bytes x 256 scales
against the OCP bit-field formula (rounded by torch, a library routine), and
hand-worked cases.
"""
import math

import numpy as np
import pytest
import torch
from scipy.stats import norm

from oracle import (NF4_LEVELS, nf4_midpoints, quantize_nf4, dequantize_nf4,
                    mxfp4_values, decode_mxfp4_bf16, convert_mxfp4_to_nf4, compress_absmax,
                    expand_absmax, dq_midpoints)
from bit_mixture_experts_amd.inputs import dq_code_book
from oracle.formats import nf4_codes
from tests.conftest import read_golden


# ------------------------------------------------------------------ NF4 table

def test_nf4_table_matches_published_values():
    gold = np.array([float(r[0]) for r in read_golden("nf4_levels.txt")])
    assert gold.shape == (16,)
    assert np.array_equal(NF4_LEVELS.astype(np.float64), gold)


def test_nf4_table_shape_and_construction():
    lv = NF4_LEVELS.astype(np.float64)
    assert lv[0] == -1.0 and lv[7] == 0.0 and lv[15] == 1.0
    assert np.all(np.diff(lv) > 0)
    # QLoRA construction: 8 positive quantiles of linspace(d, 1/2, 9)[:-1], 7
    # negative ones of linspace(d, 1/2, 8)[:-1], plus zero, normalised by the
    # maximum, with d = 1 - (1/30 + 1/32)/2.
    d = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    pos = norm.ppf(np.linspace(d, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(d, 0.5, 8)[:-1])
    built = np.sort(np.concatenate([pos, [0.0], neg]))
    built /= built.max()
    # the published values came from a float32 construction: a few ulp apart
    assert np.max(np.abs(built - lv)) < 3e-7


def test_nf4_midpoints_lie_between_levels():
    mids = nf4_midpoints().astype(np.float64)
    lv = NF4_LEVELS.astype(np.float64)
    assert mids.shape == (15,)
    assert np.all(lv[:-1] < mids) and np.all(mids < lv[1:])
    assert np.all(np.abs(mids - (lv[:-1] + lv[1:]) / 2) <= np.spacing(np.float32(1.0)))


# ------------------------------------------------------------- NF4 quantise

def _brute_codes(w):
    """Nearest level by exhaustive search on fp32 x = w/absmax (float64 distance);
    returns codes and a mask of exact ties between two levels."""
    blocks = w.reshape(-1, 64).astype(np.float32)
    am = np.abs(blocks).max(axis=1)
    x = np.where(am[:, None] == 0, 0, blocks / np.where(am == 0, 1, am)[:, None]).astype(np.float32)
    dist = np.abs(x.astype(np.float64)[..., None] - NF4_LEVELS.astype(np.float64))
    codes = np.argmin(dist, axis=-1)
    srt = np.sort(dist, axis=-1)
    tie = srt[..., 0] == srt[..., 1]
    return codes.reshape(-1), tie.reshape(-1), am


def test_quantize_nf4_matches_brute_force_nearest_level():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(64 * 4096) * 0.02).astype(np.float32)
    packed, absmax = quantize_nf4(w)
    codes = nf4_codes(packed)
    bc, tie, am = _brute_codes(w)
    assert np.array_equal(absmax, am)
    assert not tie.any()
    assert np.array_equal(codes, bc)


def test_quantize_nf4_near_thresholds():
    # elements within +-16 fp32 ulps of every midpoint, absmax fixed at 1.0
    mids = nf4_midpoints()
    offs = np.arange(-16, 17, dtype=np.int64)
    bits = mids.view(np.uint32).astype(np.int64)
    # negative floats: a larger bit pattern is a more negative value; either
    # way the set {bits + d} is the 33 nearest floats around each midpoint
    vals = (bits[:, None] + offs[None, :]).astype(np.uint32).view(np.float32).reshape(-1)
    pad = (-len(vals)) % 63
    vals = np.concatenate([vals, np.zeros(pad, np.float32)])
    blocks = vals.reshape(-1, 63)
    w = np.concatenate([np.ones((blocks.shape[0], 1), np.float32), blocks], axis=1).reshape(-1)
    codes = nf4_codes(quantize_nf4(w)[0])
    bc, tie, _ = _brute_codes(w)
    on_mid = np.isin(w, mids)
    # away from the thresholds themselves, the rule is the nearest level
    keep = ~tie & ~on_mid
    assert np.array_equal(codes[keep], bc[keep])
    # a value exactly on a (fp32) midpoint takes the lower code; there the
    # float64 nearest level may be either neighbour, since the fp32 midpoint
    # is within half an ulp of the exact one
    for i, m in enumerate(mids):
        hit = w == m
        assert hit.sum() == 1 and np.all(codes[hit] == i)
        assert np.all(np.isin(bc[hit], [i, i + 1]))


def test_quantize_nf4_round_trip_invariants():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal(64 * 2048) * 0.05).astype(np.float32)
    packed, absmax = quantize_nf4(w)
    codes = nf4_codes(packed).reshape(-1, 64)
    blocks = w.reshape(-1, 64)
    deq = dequantize_nf4(packed, absmax).reshape(-1, 64)
    # the largest-magnitude element of each block decodes exactly to +-absmax
    arg = np.argmax(np.abs(blocks), axis=1)
    rows = np.arange(blocks.shape[0])
    assert np.all(np.isin(codes[rows, arg], [0, 15]))
    assert np.array_equal(np.abs(deq[rows, arg]), absmax.astype(np.float64))
    # error bound: half the largest gap between adjacent levels, times absmax
    half_gap = np.max(np.diff(NF4_LEVELS.astype(np.float64))) / 2
    assert half_gap < 0.1520
    assert np.all(np.abs(deq - blocks) <= half_gap * absmax[:, None] + 1e-12)
    # quantising the decoded values reproduces the codes bit for bit
    p2, a2 = quantize_nf4(deq.reshape(-1).astype(np.float32))
    assert np.array_equal(p2, packed) and np.array_equal(a2, absmax)


def test_quantize_nf4_zero_block_and_packing_order():
    w = np.zeros(128, np.float32)
    w[64] = -1.0   # second block: element 0 = -1 (code 0), element 1 = +1 (code 15)
    w[65] = 1.0
    packed, absmax = quantize_nf4(w)
    assert absmax[0] == 0 and np.all(packed[:32] == 0x77)
    assert absmax[1] == 1.0
    assert packed[32] == 0xF0          # low nibble = even element
    assert np.all(packed[33:] == 0x77)


def test_quantize_nf4_rejects_bad_sizes():
    with pytest.raises(ValueError):
        quantize_nf4(np.zeros(65, np.float32))
    with pytest.raises(ValueError):
        quantize_nf4(np.zeros(64, np.float32), blocksize=32)


# ------------------------------------------------------------------- MXFP4

def _ocp_e2m1(n):
    """E2M1 from its bit fields (OCP MX v1.0): sign, 2-bit exponent with bias 1,
    1-bit mantissa; exponent 0 is subnormal."""
    s, e, m = (n >> 3) & 1, (n >> 1) & 3, n & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


def test_e2m1_golden_table():
    for nib, val in read_golden("e2m1_values.txt"):
        n, v = int(nib), float(val)
        assert _ocp_e2m1(n) == v and math.copysign(1, _ocp_e2m1(n)) == math.copysign(1, v)


def test_mxfp4_decode_exhaustive_bytes_and_scales():
    byte = np.repeat(np.arange(256, dtype=np.uint8), 256)
    scale = np.tile(np.arange(256, dtype=np.uint8), 256)
    # one block of 32 per (byte, scale) pair: the byte repeated 16 times
    blocks = np.repeat(byte[:, None], 16, axis=1).reshape(-1, 1, 16)
    scales = scale.reshape(-1, 1)
    got = decode_mxfp4_bf16(blocks, scales).reshape(-1, 32)
    lo = np.array([_ocp_e2m1(int(b) & 15) for b in range(256)])
    hi = np.array([_ocp_e2m1(int(b) >> 4) for b in range(256)])
    p2 = np.ldexp(1.0, scale.astype(np.int64) - 127)
    exp_lo = torch.from_numpy(lo[byte] * p2).to(torch.bfloat16)
    exp_hi = torch.from_numpy(hi[byte] * p2).to(torch.bfloat16)
    exp_lo = exp_lo.view(torch.int16).numpy().view(np.uint16).copy()
    exp_hi = exp_hi.view(torch.int16).numpy().view(np.uint16).copy()
    nan = scale == 255
    exp_lo[nan] = 0x7FC0
    exp_hi[nan] = 0x7FC0
    assert np.array_equal(got[:, 0], exp_lo)
    assert np.array_equal(got[:, 1], exp_hi)
    assert np.all(got[:, 0::2] == got[:, [0]]) and np.all(got[:, 1::2] == got[:, [1]])


def test_mxfp4_decode_hand_cases():
    for b, s, lo, hi in read_golden("mxfp4_decode_cases.txt"):
        blk = np.full((1, 1, 16), int(b, 16), np.uint8)
        scl = np.full((1, 1), int(s), np.uint8)
        got = decode_mxfp4_bf16(blk, scl).reshape(-1)
        assert got[0] == int(lo, 16) and got[1] == int(hi, 16), (b, s)


def test_mxfp4_values_layout():
    # element k of a row comes from block k//32, byte (k%32)//2, nibble k%2
    rng = np.random.default_rng(5)
    blocks = rng.integers(0, 256, (3, 4, 16), dtype=np.uint8)
    scales = rng.integers(120, 130, (3, 4), dtype=np.uint8)
    v = mxfp4_values(blocks, scales)
    assert v.shape == (3, 128)
    for r in range(3):
        for k in range(128):
            byte = int(blocks[r, k // 32, (k % 32) // 2])
            nib = byte & 15 if k % 2 == 0 else byte >> 4
            assert v[r, k] == _ocp_e2m1(nib) * 2.0 ** (int(scales[r, k // 32]) - 127)


# -------------------------------------------------------- MXFP4 -> NF4

def _ocp_values(blocks, scales):
    """Element values of [R, K/32, 16] blocks from the OCP bit fields, one by one
    (float64; exact)."""
    R, nb, _ = blocks.shape
    v = np.empty((R, nb * 32))
    for r in range(R):
        for k in range(nb * 32):
            byte = int(blocks[r, k // 32, (k % 32) // 2])
            nib = byte & 15 if k % 2 == 0 else byte >> 4
            v[r, k] = math.ldexp(_ocp_e2m1(nib), int(scales[r, k // 32]) - 127)
    return v


def test_convert_mxfp4_nf4_matches_brute_force():
    # scale pairs inside one NF4 block range from equal to far apart, down to
    # the fp32-subnormal decodes of scale bytes 0 and 1
    rng = np.random.default_rng(11)
    R, K = 24, 192
    blocks = rng.integers(0, 256, (R, K // 32, 16), dtype=np.uint8)
    scales = rng.integers(118, 131, (R, K // 32), dtype=np.uint8)
    scales[:8] = rng.integers(0, 253, (8, K // 32), dtype=np.uint8)
    scales[8:12, 1::2] = scales[8:12, 0::2] - rng.integers(0, 9, (4, K // 64), dtype=np.uint8)
    scales[12, :] = [0, 1, 1, 0, 2, 0]
    blocks[13, 2:4] = 0x88            # a block of negative zeros
    blocks[14, 4:6] = 0               # an all-zero block
    packed, absmax = convert_mxfp4_to_nf4(blocks, scales)
    assert packed.shape == (R, K // 2) and absmax.shape == (R, K // 64)
    v = _ocp_values(blocks, scales).astype(np.float32)   # exact: <= 2 significant bits
    assert np.array_equal(v.astype(np.float64), _ocp_values(blocks, scales))
    bc, tie, am = _brute_codes(v.reshape(-1))
    assert not tie.any()
    assert np.array_equal(absmax.reshape(-1), am)
    assert np.array_equal(nf4_codes(packed.reshape(-1)), bc)
    assert absmax[14, 2] == 0 and np.all(packed[14, 64:96] == 0x77)
    assert np.all(packed[13, 32:64] == 0x77)


def test_convert_mxfp4_nf4_no_ratio_on_a_threshold():
    # every x = v / absmax the conversion can form: e2m1 magnitude ratios times
    # powers of two; none lies on an NF4 decision threshold, so the
    # nearest-level rule has no ties to break on this path
    mags = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    xs = set()
    for a in mags:
        for m in mags:
            for d in range(-12, 13):
                x = np.float32(math.ldexp(a, d)) / np.float32(m)
                if x <= 1:
                    xs.update([float(x), -float(x)])
    mids = set(float(m) for m in nf4_midpoints())
    assert not (xs & mids)


def test_convert_mxfp4_nf4_closed_forms():
    # uniform blocks: every element equal -> absmax = |value|, codes 15 / 0
    for nib, code in ((7, 15), (0xF, 0), (3, 15), (0xB, 0), (1, 15)):
        byte = nib | (nib << 4)
        blocks = np.full((1, 2, 16), byte, np.uint8)
        scales = np.array([[125, 125]], np.uint8)
        packed, absmax = convert_mxfp4_to_nf4(blocks, scales)
        assert absmax[0, 0] == abs(_ocp_e2m1(nib)) * 2.0 ** -2
        assert np.all(nf4_codes(packed.reshape(-1)) == code)
    # hand case: 6 * 2^0 in element 0 (first block), 6 * 2^-2 = 1.5 in element
    # 32 (second block, scale 125), 0.5 * 2^0 in element 1: x = 1, 0.25, 1/12
    blocks = np.zeros((1, 2, 16), np.uint8)
    blocks[0, 0, 0] = 0x17     # element 0 = nibble 7 (6.0), element 1 = nibble 1 (0.5)
    blocks[0, 1, 0] = 0x07     # element 32 = nibble 7
    scales = np.array([[127, 125]], np.uint8)
    packed, absmax = convert_mxfp4_to_nf4(blocks, scales)
    codes = nf4_codes(packed.reshape(-1))
    assert absmax[0, 0] == 6.0
    # 0.25 is nearest to level 10 (0.2461); 1/12 = 0.0833 to level 8 (0.0796)
    assert codes[0] == 15 and codes[32] == 10 and codes[1] == 8
    assert np.all(np.delete(codes, [0, 1, 32]) == 7)


def test_convert_mxfp4_nf4_round_trip_bound_and_refusals():
    rng = np.random.default_rng(12)
    blocks = rng.integers(0, 256, (16, 6, 16), dtype=np.uint8)
    scales = rng.integers(118, 131, (16, 6), dtype=np.uint8)
    packed, absmax = convert_mxfp4_to_nf4(blocks, scales)
    v = _ocp_values(blocks, scales).reshape(-1, 64)
    deq = dequantize_nf4(packed.reshape(-1), absmax.reshape(-1)).reshape(-1, 64)
    half_gap = np.max(np.diff(NF4_LEVELS.astype(np.float64))) / 2
    assert np.all(np.abs(deq - v) <= half_gap * absmax.reshape(-1, 1))
    with pytest.raises(ValueError):      # K = 32 is not a whole NF4 block
        convert_mxfp4_to_nf4(blocks[:, :1], scales[:, :1])
    bad = scales.copy()
    bad[0, 0] = 255                       # e8m0 NaN
    with pytest.raises(ValueError):
        convert_mxfp4_to_nf4(blocks, bad)


# ------------------------------------------------ double-quantised absmax

def _absmax_sample(rng, n):
    # absmax of NF4 blocks of N(0, 0.02^2) weights: positive, clustered
    w = rng.standard_normal((n, 64)).astype(np.float32) * np.float32(0.02)
    return np.abs(w).max(axis=1).astype(np.float32)


@pytest.mark.parametrize("kind", ["dynamic", "linear"])
def test_compress_absmax_brute_force(kind):
    rng = np.random.default_rng(40)
    book = dq_code_book(kind)
    a = _absmax_sample(rng, 256 * 9 + 77)          # ragged last group
    code, a2, off = compress_absmax(a, book)
    assert code.shape == a.shape and a2.shape == (10,)
    # offset: fp32 rounding of the exactly summed mean
    assert off == np.float32(math.fsum(a.astype(np.float64)) / a.size)
    d = (a - off).astype(np.float32)
    for g in range(10):
        blk = d[256 * g:256 * (g + 1)]
        assert a2[g] == np.max(np.abs(blk))
        x = (blk / a2[g]).astype(np.float32)
        dist = np.abs(x.astype(np.float64)[:, None] - book.astype(np.float64)[None, :])
        srt = np.sort(dist, axis=1)
        assert np.all(srt[:, 0] < srt[:, 1])       # no exact ties in this sample
        assert np.array_equal(code[256 * g:256 * (g + 1)], np.argmin(dist, axis=1))
    if kind == "linear":
        # closed form for evenly spaced entries: the nearest index
        x = (d / a2[np.arange(a.size) // 256]).astype(np.float64)
        assert np.array_equal(code, np.clip(np.floor((x + 1.0) * 127.5 + 0.5), 0, 255))


def test_expand_absmax_round_trip_and_special_cases():
    rng = np.random.default_rng(41)
    book = dq_code_book("dynamic")
    a = _absmax_sample(rng, 256 * 6)
    code, a2, off = compress_absmax(a, book)
    got = expand_absmax(code, a2, off, book)
    gaps = np.diff(book.astype(np.float64))
    err = np.abs(got.astype(np.float64) - a)
    lim = (np.max(gaps) / 2) * np.repeat(a2, 256).astype(np.float64) + 4 * np.spacing(a)
    assert np.all(err <= lim)
    # each group's largest |d| sits on an end entry (+-1) and decodes to
    # fp32(+-absmax2 + offset)
    d = (a - off).astype(np.float32).reshape(6, 256)
    arg = np.argmax(np.abs(d), axis=1)
    for g in range(6):
        c = code[256 * g + arg[g]]
        assert c in (0, 255)
        assert got[256 * g + arg[g]] == np.float32(np.float32(book[c] * a2[g]) + off)
    # a stack of equal absmax: offset is that value, every group's scale 0,
    # codes point at the zero entry, the decode is exact
    code, a2, off = compress_absmax(np.full(300, 0.0375, np.float32), book)
    assert off == np.float32(0.0375) and np.all(a2 == 0)
    assert np.all(book[code] == 0) and np.all(expand_absmax(code, a2, off, book) == np.float32(0.0375))
    # hand case: book[code] * absmax2 rounded to fp32, then + offset rounded
    c = np.array([255, 0, 128], np.uint8)
    got = expand_absmax(c, np.array([0.5], np.float32), np.float32(0.25), book)
    assert np.array_equal(got, np.array([0.75, -0.25, 0.25 + 0.5 * float(book[128])], np.float32))


def test_dq_book_and_midpoints():
    book = dq_code_book("dynamic")
    assert book[0] == -1 and book[255] == 1 and 0.0 in book
    m = dq_midpoints(book)
    assert m.shape == (255,) and np.all(book[:-1] < m) and np.all(m < book[1:])
    with pytest.raises(ValueError):
        dq_midpoints(np.sort(book)[::-1])
