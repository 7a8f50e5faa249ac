"""Seeded synthetic inputs for the 4-bit routed MoE layer.

This module only draws random numbers: it holds none of the layer's arithmetic
(no quantisation, routing, permutation or GEMM). The library's tests and the
host oracle both consume what it produces.

Two generators:

* ``host_*`` functions draw with numpy, one independent stream per
  (seed, workload, layer, tensor, expert-or-token-count), so a single expert of
  a large stack can be regenerated alone. Parity tests use these.
* ``device_*`` functions draw the same distributions with torch's generator on
  the GPU, for timing runs whose stacks are too large to generate on the host
  in reasonable time (the 36-layer MXFP4 stack is 61 GB). Their values differ
  from the host streams; only shapes and distributions match.

bf16 fields are fp32 draws rounded to bf16 (round to nearest even, by torch's
CPU cast), carried as uint16 bit patterns.
"""

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

# tensor identifiers inside a seed path
_X, _LOGITS, _W_GU, _W_DN, _GU_BLK, _GU_SCL, _DN_BLK, _DN_SCL = 1, 2, 3, 4, 5, 6, 7, 8
_B_GU, _B_DN, _LORA_A, _LORA_B, _DOUT, _ZIPF = 9, 10, 11, 12, 13, 14
_W_ROUTER, _Y_SLOTS = 15, 16


@dataclass(frozen=True)
class LayerSpec:
    """Shape and input distribution of one routed expert layer workload."""
    name: str
    seed_id: int
    fmt: str                 # "nf4" | "mxfp4"
    E: int
    k: int
    H: int
    I: int
    tokens: tuple            # token counts T the workload is measured at
    layout: str = "halves"   # "halves" | "interleaved"
    act: str = "swiglu"      # "swiglu" | "swiglu_clamped"
    alpha: float = 1.702
    limit: float = 7.0
    bias: bool = False
    lora_r: int = 0
    lora_alpha: float = 0.0
    layers: int = 1
    zipf: Optional[float] = None
    weight_std: float = 0.02     # NF4 source weights ~ N(0, weight_std^2)
    bias_std: float = 0.01
    mx_scale_lo: int = 118       # MXFP4 e8m0 scales uniform in [lo, hi]
    mx_scale_hi: int = 130

    @property
    def lora_scale(self):
        return self.lora_alpha / self.lora_r if self.lora_r else 0.0

    def scaled(self, **kw):
        return replace(self, **kw)


# The five workloads: a tiny NF4 layer, Qwen3-30B-A3B-shaped NF4, gpt-oss-20b-
# shaped native MXFP4, LoRA on the Qwen3-shaped NF4 stack (forward + backward),
# and a 36-layer gpt-oss-120b-shaped MXFP4 stack with Zipf-skewed routing.
TINY_NF4 = LayerSpec("tiny_nf4_E8_k2_H256_I512", 1, "nf4", E=8, k=2, H=256, I=512,
                     tokens=(64,))
QWEN3_30B_NF4 = LayerSpec("qwen3_30b_a3b_nf4_E128_k8_H2048_I768", 2, "nf4", E=128, k=8,
                          H=2048, I=768, tokens=(1, 16, 128, 4096))
GPT_OSS_20B_MXFP4 = LayerSpec("gpt_oss_20b_mxfp4_E32_k4_H2880_I2880", 3, "mxfp4", E=32,
                              k=4, H=2880, I=2880, tokens=(1, 64, 2048),
                              layout="interleaved", act="swiglu_clamped", bias=True)
QWEN3_30B_NF4_LORA = LayerSpec("qwen3_30b_a3b_nf4_lora_r8", 4, "nf4", E=128, k=8, H=2048,
                               I=768, tokens=(2048,), lora_r=8, lora_alpha=16.0)
GPT_OSS_120B_STACK = LayerSpec("gpt_oss_120b_mxfp4_stack_36L_E128_k4", 5, "mxfp4", E=128,
                               k=4, H=2880, I=2880, tokens=(1, 8, 32),
                               layout="interleaved", act="swiglu_clamped", bias=True,
                               layers=36, zipf=1.1)

WORKLOADS = (TINY_NF4, QWEN3_30B_NF4, GPT_OSS_20B_MXFP4, QWEN3_30B_NF4_LORA,
             GPT_OSS_120B_STACK)

# Beyond the five: per-expert LoRA over the native MXFP4 gpt-oss-20b-shaped
# experts, with their biases, interleaved gate/up rows and clamped GLU
# (forward + backward), the adapter variant of the MXFP4 training path.
GPT_OSS_20B_MXFP4_LORA = LayerSpec("gpt_oss_20b_mxfp4_lora_r8", 6, "mxfp4", E=32, k=4,
                                   H=2880, I=2880, tokens=(2048,), layout="interleaved",
                                   act="swiglu_clamped", bias=True, lora_r=8, lora_alpha=16.0)


def dq_code_book(kind="dynamic"):
    """A 256-entry, strictly increasing fp32 code book for double-quantised
    absmax (the pages name an 8-bit code book but print none; this one is our
    own construction). "dynamic": 0, +-1 and, per octave [2^-(e+1), 2^-e) for
    e = 0..7, sixteen evenly spaced values (finer steps near zero), trimmed to
    128 positive and 127 negative entries. "linear": 256 evenly spaced values
    from -1 to 1."""
    if kind == "linear":
        return (np.arange(256, dtype=np.float64) * (2.0 / 255.0) - 1.0).astype(np.float32)
    grid = np.array([(16 + f) / 16.0 * 2.0 ** (-e - 1) for e in range(8) for f in range(16)])
    grid = np.sort(grid)                       # 128 values in [2^-8, 31/32]
    pos = np.concatenate([grid[1:], [1.0]])    # 128
    neg = -np.concatenate([grid[2:], [1.0]])   # 127
    book = np.sort(np.concatenate([neg, [0.0], pos])).astype(np.float32)
    assert book.shape == (256,) and np.all(np.diff(book.astype(np.float64)) > 0)
    return book


def _rng(seed, spec, *path):
    return np.random.default_rng(np.random.SeedSequence([int(seed), spec.seed_id,
                                                         *[int(p) for p in path]]))


def to_bf16_bits(a):
    """fp32 -> bf16 bits (round to nearest even) via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


# ---------------------------------------------------------------- host streams

def host_nf4_source(spec, e, layer=0, seed=0):
    """fp32 source weights of expert e: (W_gu [2I,H], W_dn [H,I]) ~ N(0, std^2)."""
    g = _rng(seed, spec, layer, _W_GU, e).standard_normal((2 * spec.I, spec.H),
                                                          dtype=np.float32)
    d = _rng(seed, spec, layer, _W_DN, e).standard_normal((spec.H, spec.I),
                                                          dtype=np.float32)
    s = np.float32(spec.weight_std)
    return g * s, d * s


def host_mxfp4_expert(spec, e, layer=0, seed=0):
    """Released-style MXFP4 bytes of expert e: uniform nibbles (uniform bytes)
    and uniform e8m0 scales. Returns (gu_blocks [2I,H/32,16], gu_scales
    [2I,H/32], dn_blocks [H,I/32,16], dn_scales [H,I/32])."""
    H, I = spec.H, spec.I
    gb = _rng(seed, spec, layer, _GU_BLK, e).integers(0, 256, (2 * I, H // 32, 16),
                                                      dtype=np.uint8)
    gs = _rng(seed, spec, layer, _GU_SCL, e).integers(spec.mx_scale_lo, spec.mx_scale_hi + 1,
                                                      (2 * I, H // 32), dtype=np.uint8)
    db = _rng(seed, spec, layer, _DN_BLK, e).integers(0, 256, (H, I // 32, 16),
                                                      dtype=np.uint8)
    ds = _rng(seed, spec, layer, _DN_SCL, e).integers(spec.mx_scale_lo, spec.mx_scale_hi + 1,
                                                      (H, I // 32), dtype=np.uint8)
    return gb, gs, db, ds


def host_bias(spec, e, layer=0, seed=0):
    """bf16 biases (b_gu [2I], b_dn [H]) ~ N(0, bias_std^2)."""
    bg = _rng(seed, spec, layer, _B_GU, e).standard_normal(2 * spec.I, dtype=np.float32)
    bd = _rng(seed, spec, layer, _B_DN, e).standard_normal(spec.H, dtype=np.float32)
    s = np.float32(spec.bias_std)
    return to_bf16_bits(bg * s), to_bf16_bits(bd * s)


def host_lora(spec, e, layer=0, seed=0):
    """bf16 adapters A [r,H] ~ N(0, 1/H) and B [2I,r] ~ N(0, 0.01^2)."""
    a = _rng(seed, spec, layer, _LORA_A, e).standard_normal((spec.lora_r, spec.H),
                                                            dtype=np.float32)
    b = _rng(seed, spec, layer, _LORA_B, e).standard_normal((2 * spec.I, spec.lora_r),
                                                            dtype=np.float32)
    return (to_bf16_bits(a * np.float32(1.0 / np.sqrt(spec.H))),
            to_bf16_bits(b * np.float32(0.01)))


def host_zipf_bias(spec, layer=0, seed=0):
    """Per-expert router bias -zipf * ln(rank), rank a seeded permutation of
    1..E; zeros when the workload has no skew."""
    if not spec.zipf:
        return np.zeros(spec.E, dtype=np.float32)
    rank = 1 + _rng(seed, spec, layer, _ZIPF, 0).permutation(spec.E)
    return (-spec.zipf * np.log(rank.astype(np.float64))).astype(np.float32)


def host_tokens(spec, T, layer=0, seed=0):
    """(x bf16 bits [T,H] ~ N(0,1), router logits fp32 [T,E] ~ N(0,1) + skew)."""
    x = _rng(seed, spec, layer, _X, T).standard_normal((T, spec.H), dtype=np.float32)
    lg = _rng(seed, spec, layer, _LOGITS, T).standard_normal((T, spec.E), dtype=np.float32)
    lg = (lg + host_zipf_bias(spec, layer, seed)[None, :]).astype(np.float32)
    return to_bf16_bits(x), lg


def host_router(spec, layer=0, seed=0):
    """Router weights W_r bf16 bits [E,H] ~ N(0, 1/H) (so that x W_r^T ~ N(0,1)
    for x ~ N(0,1)) and the fp32 router bias [E] (the Zipf skew, else zeros)."""
    w = _rng(seed, spec, layer, _W_ROUTER, 0).standard_normal((spec.E, spec.H),
                                                              dtype=np.float32)
    return to_bf16_bits(w * np.float32(1.0 / np.sqrt(spec.H))), host_zipf_bias(spec, layer, seed)


def host_slot_outputs(spec, T, layer=0, seed=0):
    """fp32 [T*k, H] ~ N(0,1): stand-in expert outputs, one row per routed slot."""
    return _rng(seed, spec, layer, _Y_SLOTS, T).standard_normal((T * spec.k, spec.H),
                                                                dtype=np.float32)


def host_upstream_grad(spec, T, layer=0, seed=0):
    """bf16 bits [T,H] ~ N(0,1): the gradient arriving at the layer output."""
    d = _rng(seed, spec, layer, _DOUT, T).standard_normal((T, spec.H), dtype=np.float32)
    return to_bf16_bits(d)


def host_stack_mxfp4(spec, layer=0, seed=0):
    """Whole MXFP4 stack of one layer (all experts) on the host."""
    parts = [host_mxfp4_expert(spec, e, layer, seed) for e in range(spec.E)]
    return tuple(np.stack([p[i] for p in parts]) for i in range(4))


def host_stack_bias(spec, layer=0, seed=0):
    parts = [host_bias(spec, e, layer, seed) for e in range(spec.E)]
    return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


def host_stack_lora(spec, layer=0, seed=0):
    parts = [host_lora(spec, e, layer, seed) for e in range(spec.E)]
    return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


# -------------------------------------------------------------- device streams

def device_generator(seed, spec, *path, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([int(seed), spec.seed_id,
                                              *[int(p) for p in path]]).generate_state(1)[0]))
    return g


def device_nf4_source(spec, layer=0, seed=0, device="cuda"):
    """fp32 source stacks (W_gu [E,2I,H], W_dn [E,H,I]) ~ N(0, std^2) on device."""
    import torch
    g = device_generator(seed, spec, layer, _W_GU, device=device)
    wg = torch.randn((spec.E, 2 * spec.I, spec.H), generator=g, device=device,
                     dtype=torch.float32).mul_(spec.weight_std)
    wd = torch.randn((spec.E, spec.H, spec.I), generator=g, device=device,
                     dtype=torch.float32).mul_(spec.weight_std)
    return wg, wd


def device_mxfp4_stack(spec, layer=0, seed=0, device="cuda"):
    """MXFP4 bytes for one layer on device (uniform bytes, uniform scales)."""
    import torch
    g = device_generator(seed, spec, layer, _GU_BLK, device=device)
    H, I, E = spec.H, spec.I, spec.E
    u8 = torch.uint8
    gb = torch.randint(0, 256, (E, 2 * I, H // 32, 16), generator=g, device=device, dtype=u8)
    gs = torch.randint(spec.mx_scale_lo, spec.mx_scale_hi + 1, (E, 2 * I, H // 32),
                       generator=g, device=device, dtype=u8)
    db = torch.randint(0, 256, (E, H, I // 32, 16), generator=g, device=device, dtype=u8)
    ds = torch.randint(spec.mx_scale_lo, spec.mx_scale_hi + 1, (E, H, I // 32),
                       generator=g, device=device, dtype=u8)
    return gb, gs, db, ds


def device_bf16(shape, std, seed, spec, *path, device="cuda"):
    """bf16 tensor ~ N(0, std^2) on device."""
    import torch
    g = device_generator(seed, spec, *path, device=device)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            .mul_(std).to(torch.bfloat16))


def device_router(spec, layer=0, seed=0, device="cuda"):
    """(W_r bf16 [E,H] ~ N(0, 1/H), bias fp32 [E]) on device."""
    import torch
    w = device_bf16((spec.E, spec.H), 1.0 / spec.H ** 0.5, seed, spec, layer, _W_ROUTER,
                    device=device)
    return w, torch.from_numpy(host_zipf_bias(spec, layer, seed)).to(device)


def device_tokens(spec, T, layer=0, seed=0, device="cuda"):
    """(x bf16 [T,H], logits fp32 [T,E]) on device; logits carry the Zipf skew."""
    import torch
    g = device_generator(seed, spec, layer, _X, T, device=device)
    x = torch.randn((T, spec.H), generator=g, device=device).to(torch.bfloat16)
    lg = torch.randn((T, spec.E), generator=g, device=device, dtype=torch.float32)
    lg += torch.from_numpy(host_zipf_bias(spec, layer, seed)).to(device)[None, :]
    return x, lg
