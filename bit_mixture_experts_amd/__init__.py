"""moe4: a routed mixture-of-experts expert layer computed directly on 4-bit
expert stacks (NF4 blockwise-absmax or MXFP4), with hand-written HIP kernels for
AMD Instinct MI355X (gfx950).

The compute path is the C library ``libmoe4.so`` (interface in
``include/moe4.h``); ``bit_mixture_experts_amd.moe4`` is its thin Python
binding. Importing this package does not load the library; importing the
binding does, and fails loudly when the library is missing.
"""

__all__ = ["inputs"]
