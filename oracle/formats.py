"""4-bit expert storage formats: NF4 blockwise-absmax and MXFP4 (test oracle).

NF4 ([experts4bit-qlora page], "Limitations -- qlora-fused-moe-experts", the
double-quantised absmax item: an NF4 expert stack keeps one fp32 absmax per 64
weights; [MXFP4 page], "Two fidelity paths": the fused stack is quantised to
NF4 by the stack constructor). The 16 levels are the NormalFloat4 data type of
the QLoRA paper (Dettmers et al. 2023, appendix E); the pages name the type but
print no table. Two codes share a byte, the even element in the low nibble.

MXFP4 ([MXFP4 page], "Why it happens"): OCP microscaling FP4 -- two e2m1 nibbles
per byte, 32 values per block, one e8m0 power-of-two scale per block. The
decode must be bit-identical to the reference decode ([MXFP4 page], "Two
fidelity paths").

Readings where the pages are silent (each also listed in the design notes):
* NF4 code = nearest level, decided by fp32 midpoint thresholds; a value
  exactly on a midpoint takes the lower code.
* x = w / absmax is an IEEE fp32 division (not a reciprocal multiply).
* An all-zero block has absmax 0 and every code 7 (the level 0.0).
* MXFP4 nibble order: the even element sits in the low nibble.
* E8M0 byte 0xFF is NaN (the OCP encoding); the decode emits bf16 0x7FC0.
"""

import numpy as np

from .numerics import bf16_bits_from_f32, bf16_bits_to_f64

# NormalFloat4 levels, exact float32 numbers (QLoRA paper, appendix E).
NF4_LEVELS = np.array([
    -1.0, -0.6961928009986877, -0.5250730514526367, -0.39491748809814453,
    -0.28444138169288635, -0.18477343022823334, -0.09105003625154495, 0.0,
    0.07958029955625534, 0.16093020141124725, 0.24611230194568634,
    0.33791524171829224, 0.44070982933044434, 0.5626170039176941,
    0.7229568362236023, 1.0,
], dtype=np.float32)

NF4_BLOCK = 64

# Magnitudes of the e2m1 code points for mantissa/exponent bits 0..7
# (OCP Microscaling Formats v1.0, FP4 E2M1: 1 sign, 2 exponent bits with bias 1,
# 1 mantissa bit; exponent field 0 is subnormal).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

MX_BLOCK = 32


def nf4_midpoints():
    """The 15 decision thresholds: fp32 rounding of the float64 midpoint of
    adjacent levels."""
    lv = NF4_LEVELS.astype(np.float64)
    return ((lv[:-1] + lv[1:]) / 2.0).astype(np.float32)


def quantize_nf4(w, blocksize=NF4_BLOCK):
    """Quantise a flat float32 array to NF4.

    Returns (packed uint8 [n/2], absmax float32 [n/64]). Per block of 64:
    absmax = max |w| (exact); x = fp32(w / absmax); code = number of thresholds
    strictly below x; two codes per byte, even element in the low nibble.
    """
    if blocksize != NF4_BLOCK:
        raise ValueError("NF4 blocksize must be 64")
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32)).reshape(-1)
    if w.size % NF4_BLOCK:
        raise ValueError("element count must be a multiple of 64")
    if not np.all(np.isfinite(w)):
        raise ValueError("NF4 quantisation is defined for finite inputs only")
    blocks = w.reshape(-1, NF4_BLOCK)
    absmax = np.max(np.abs(blocks), axis=1).astype(np.float32)
    safe = np.where(absmax == 0, np.float32(1), absmax).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)   # IEEE fp32 division
    x[absmax == 0] = np.float32(0)
    mids = nf4_midpoints()
    codes = np.zeros(blocks.shape, dtype=np.uint8)
    for m in mids:
        codes += (x > m).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8).reshape(-1)
    return packed, absmax


def nf4_codes(packed):
    """Unpack NF4 bytes to one code per element (even element = low nibble)."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    codes = np.empty(p.size * 2, dtype=np.uint8)
    codes[0::2] = p & 0x0F
    codes[1::2] = p >> 4
    return codes


def dequantize_nf4(packed, absmax):
    """Exact float64 value of each NF4 weight: level[code] * absmax.

    The product of two fp32 numbers is exact in float64, so nothing is rounded.
    """
    codes = nf4_codes(packed).reshape(-1, NF4_BLOCK)
    am = np.asarray(absmax, dtype=np.float32).astype(np.float64).reshape(-1)
    if am.size != codes.shape[0]:
        raise ValueError("absmax length does not match the packed data")
    return (NF4_LEVELS.astype(np.float64)[codes] * am[:, None]).reshape(-1)


def dequantize_nf4_bf16(packed, absmax):
    """The bf16 operand value of each NF4 weight: level[code] * absmax formed
    as one IEEE fp32 product, then rounded once to bf16 (float64 result).

    Reading: the pages fix fp32 accumulation over bf16 operands but not how the
    decoded weight is rounded; one fp32 product and one rounding is the plain
    way to form a bf16 operand from an fp32 level and an fp32 absmax.
    """
    codes = nf4_codes(packed).reshape(-1, NF4_BLOCK)
    am = np.asarray(absmax, dtype=np.float32).reshape(-1)
    if am.size != codes.shape[0]:
        raise ValueError("absmax length does not match the packed data")
    prod = (NF4_LEVELS[codes] * am[:, None]).astype(np.float32)   # fp32 product
    return bf16_bits_to_f64(bf16_bits_from_f32(prod)).reshape(-1)


def mxfp4_values(blocks, scales):
    """Exact float64 values of an MXFP4 tensor.

    blocks: uint8 [..., K/32, 16], scales: uint8 [..., K/32]. Returns float64
    [..., K]. Element k of a block is nibble k%2 of byte k//2 (even = low).
    value = (-1)^sign * E2M1_MAGNITUDES[n & 7] * 2^(scale - 127); scale byte
    255 gives NaN.
    """
    b = np.asarray(blocks, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8)
    if b.shape[-1] != 16 or b.shape[:-1] != s.shape:
        raise ValueError("blocks must be [..., K/32, 16] and scales [..., K/32]")
    nib = np.empty(b.shape[:-1] + (32,), dtype=np.uint8)
    nib[..., 0::2] = b & 0x0F
    nib[..., 1::2] = b >> 4
    mag = E2M1_MAGNITUDES[nib & 7]
    sign = np.where(nib & 8, -1.0, 1.0)
    scale = np.ldexp(1.0, s.astype(np.int64) - 127)[..., None]
    val = sign * mag * scale
    val = np.where((s == 255)[..., None], np.nan, val)
    return val.reshape(b.shape[:-2] + (b.shape[-2] * 32,))


def decode_mxfp4_bf16(blocks, scales):
    """bf16 bit patterns of the MXFP4 decode (what ``moe4_decode_mxfp4`` must
    produce bit for bit).

    Every finite decoded value with a scale byte <= 254 is either exactly
    representable in bf16 (normal or subnormal) or overflows; the float32
    intermediate is therefore exact and the bf16 rounding is the only rounding.
    The sign of zero is kept (nibble 8 -> 0x8000).
    """
    v = mxfp4_values(blocks, scales)
    with np.errstate(over="ignore", invalid="ignore"):
        v32 = v.astype(np.float32)
    return bf16_bits_from_f32(v32)


def convert_mxfp4_to_nf4(blocks, scales):
    """Re-quantise an MXFP4 stack to NF4 ([MXFP4 page], "Two fidelity paths",
    the convenient QLoRA path: an exact decode of the released blocks, then the
    NF4 quantiser applied to the decoded stack).

    blocks uint8 [R, K/32, 16], scales uint8 [R, K/32], K % 64 == 0. The decode
    is the bf16 one (``decode_mxfp4_bf16``); its values, read as fp32, go
    through ``quantize_nf4`` row-major, so each NF4 block of 64 covers two
    consecutive MXFP4 blocks of one row. Returns (packed uint8 [R, K/2],
    absmax float32 [R, K/64]). Scale bytes up to 252 always decode to finite
    values; a block that decodes to inf or NaN is refused, like any non-finite
    input of the quantiser.

    Reading: the page says the decoded stack is quantised but not in which
    dtype it is held in between; bf16, the decode's own output, is the plain
    one (for scale bytes up to 252 it holds every decoded value exactly, so
    the choice changes nothing there).
    """
    b = np.asarray(blocks, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8)
    if b.ndim != 3 or b.shape[-1] != 16 or s.shape != b.shape[:2]:
        raise ValueError("blocks must be [R, K/32, 16] and scales [R, K/32]")
    R, nb = s.shape
    if nb % 2:
        raise ValueError("K must be a multiple of 64")
    dec = bf16_bits_to_f64(decode_mxfp4_bf16(b, s)).astype(np.float32)
    packed, absmax = quantize_nf4(dec.reshape(-1))
    return packed.reshape(R, nb * 16), absmax.reshape(R, nb // 2)


# ------------------------------------------- double-quantised NF4 absmax
#
# [experts4bit-qlora page], "Limitations -- qlora-fused-moe-experts", the
# double-quantised absmax item: a resident NF4 stack may keep its fp32 absmax
# (one per 64 weights) in a nested form -- one offset, an 8-bit code per
# absmax and one fp32 scale per 256 absmax values -- at about a quarter of the
# bytes; the absmax values change (lossy against fp32). Readings, where the
# page is silent:
# * offset = the fp32 rounding of the float64 mean of the stack's absmax;
# * per 256 consecutive absmax values (the last group may be shorter):
#   d = fp32(absmax - offset), absmax2 = max |d|, x = fp32(d / absmax2)
#   (x = 0 when absmax2 = 0), code = nearest entry of a 256-entry code book,
#   decided by the fp32 midpoints of adjacent entries (formed in float64, then
#   rounded), a value on a midpoint taking the lower code;
# * the page names the 8-bit code book but prints none: it is an input here
#   (256 strictly increasing fp32 values), the same on both sides;
# * decoded absmax = fp32(fp32(book[code] * absmax2) + offset): one fp32
#   product and one fp32 sum, no fused multiply-add.

DQ_BLOCK = 256


def dq_midpoints(book):
    """The 255 decision thresholds of a code book (fp32)."""
    t = np.asarray(book, dtype=np.float32).astype(np.float64)
    if t.shape != (256,) or not np.all(np.diff(t) > 0):
        raise ValueError("the code book must hold 256 strictly increasing values")
    return ((t[:-1] + t[1:]) / 2.0).astype(np.float32)


def compress_absmax(absmax, book):
    """fp32 absmax [n] -> (code uint8 [n], absmax2 float32 [ceil(n/256)],
    offset float32)."""
    a = np.ascontiguousarray(np.asarray(absmax, dtype=np.float32)).reshape(-1)
    if not np.all(np.isfinite(a)):
        raise ValueError("absmax must be finite")
    mids = dq_midpoints(book)
    n = a.size
    if n == 0:
        return np.zeros(0, np.uint8), np.zeros(0, np.float32), np.float32(0)
    offset = np.float32(np.mean(a.astype(np.float64)))
    d = (a - offset).astype(np.float32)                     # fp32 subtraction
    nb = (n + DQ_BLOCK - 1) // DQ_BLOCK
    pad = np.zeros(nb * DQ_BLOCK, np.float32)
    pad[:n] = d
    blocks = pad.reshape(nb, DQ_BLOCK)
    a2 = np.max(np.abs(blocks), axis=1).astype(np.float32)
    safe = np.where(a2 == 0, np.float32(1), a2).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)         # IEEE fp32 division
    x[a2 == 0] = np.float32(0)
    code = np.zeros(blocks.shape, dtype=np.int64)
    for m in mids:
        code += (x > m)
    return code.reshape(-1)[:n].astype(np.uint8), a2, offset


def expand_absmax(code, absmax2, offset, book):
    """Decoded fp32 absmax [n]: fp32(fp32(book[code] * absmax2[i // 256]) + offset)."""
    c = np.asarray(code, dtype=np.uint8).reshape(-1)
    a2 = np.asarray(absmax2, dtype=np.float32).reshape(-1)
    t = np.asarray(book, dtype=np.float32)
    if a2.size != (c.size + DQ_BLOCK - 1) // DQ_BLOCK:
        raise ValueError("absmax2 length does not match the codes")
    prod = (t[c] * a2[np.arange(c.size) // DQ_BLOCK]).astype(np.float32)
    return (prod + np.float32(offset)).astype(np.float32)
