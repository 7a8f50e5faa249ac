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
