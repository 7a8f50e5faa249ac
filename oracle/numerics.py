"""bfloat16 conversions used by the oracle (test infrastructure only).

bf16 values travel as uint16 bit patterns. The layer's activations, biases and
adapter weights are bf16 model tensors ([experts4bit-qlora page], "Limitations
-- qlora-fused-moe-experts": the expert adapter is kept in the model dtype,
bf16); the grouped kernels take bf16 inputs and accumulate in fp32
([Solutions index], grouped-nf4-gemm entry for the NF4 grouped GEMM).
"""

import numpy as np


def bf16_bits_from_f32(x):
    """Round float32 values to bfloat16, ties to even; return uint16 bits.

    NaN maps to the quiet NaN 0x7FC0. Overflow rounds to +-inf as IEEE
    round-to-nearest-even does. float32 subnormals are rounded like any other
    value (no flushing).
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    r = np.where(np.isnan(x), np.uint64(0x7FC0), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact float32 value of bf16 bit patterns."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits):
    """Exact float64 value of bf16 bit patterns."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def bf16_round_f64(x):
    """Round float64 values once to the nearest bfloat16 value (ties to even);
    returns float64. Used where the layer feeds a value to a bf16 GEMM operand.

    Normal range: 8 significant bits. Below 2^-126 the spacing is fixed at
    2^-133 (bf16 subnormals). Beyond the largest finite bf16 value, rounding
    goes to +-inf as round-to-nearest-even does.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    fin = np.isfinite(x)
    out[~fin] = x[~fin]
    xf = x[fin]
    m, e = np.frexp(xf)                    # xf = m * 2^e, 0.5 <= |m| < 1
    normal = e > -125                      # |x| >= 2^-126
    r = np.empty_like(xf)
    r[normal] = np.ldexp(np.rint(m[normal] * 256.0), e[normal] - 8)
    r[~normal] = np.ldexp(np.rint(np.ldexp(xf[~normal], 133)), -133)
    big = np.abs(r) >= 2.0 ** 128
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    return out


def bf16_other_neighbour_f64(x):
    """The bf16 value next to bf16_round_f64(x) on the other side of x
    (float64). The two bracket x: they are the two roundings of x that a
    computation carrying x with a small error of its own can pick where x lies
    close to their midpoint. Equal to the rounding when x is a bf16 value."""
    x = np.asarray(x, dtype=np.float64)
    r = bf16_round_f64(x)
    bits = r.astype(np.float32).view(np.uint32).astype(np.int64)
    mag, neg = bits & 0x7FFFFFFF, (bits >> 31) & 1
    above = x > r                       # the other neighbour lies above r
    grow = np.where(neg == 0, above, ~above)   # its magnitude is larger than r's
    new_mag = np.where(grow, mag + 0x10000, mag - 0x10000)
    new_neg = neg
    zero = mag == 0                     # r = +-0: the neighbour is +-2^-133 on x's side
    new_mag = np.where(zero, 0x10000, new_mag)
    new_neg = np.where(zero, (x < 0).astype(np.int64), new_neg)
    out_bits = ((new_neg << 31) | new_mag).astype(np.uint32)
    other = out_bits.view(np.float32).astype(np.float64)
    return np.where(x == r, r, other)
