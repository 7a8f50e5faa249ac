"""The routed expert layer, forward and backward, in float64 (test oracle).

Per routed row r of expert e (rows ordered by ``routing.permute``):

    gu = x W_gu[e]^T (+ b_gu[e]) (+ s * (x A_e^T) B_e^T)      s = lora alpha / r
    h  = act(gate, up)                                         gate/up split of gu
    y  = h W_d[e]^T (+ b_d[e])
    out[t] = sum_j w[t, j] * y[row_of_slot[t*k + j]]

Sources: the routed expert GEMM over fused 4-bit stacks with fp32 accumulation
([Solutions index], grouped-nf4-gemm entries for the NF4 and the native MXFP4
grouped GEMMs); fused three-dimensional expert stacks ([experts4bit-qlora page],
"What it does"); the stock epilogue act(gate)*up ([experts4bit-qlora page],
"Limitations -- qlora-fused-moe-experts", epilogue-contract item); gpt-oss
biases, interleaved gate/up rows and a clamped GLU ([MXFP4 page], "Why it
happens" and "Supported scope"); a per-expert low-rank delta added before each
routed expert's activation over a frozen NF4 stack, trained with an input
gradient through the frozen 4-bit weights ([Solutions index], QLoRA fused
experts entry; [experts4bit-qlora page], "Use this when").

Readings (the pages are silent):
* HALVES layout: gate = first I rows of the fused [2I, H] stack, up = last I;
  INTERLEAVED: gate = even rows, up = odd rows.
* Plain SwiGLU: h = g * sigmoid(g) * u.
* Clamped GLU (gpt-oss): g' = min(g, limit), u' = clip(u, -limit, limit),
  h = (u' + 1) * g' * sigmoid(alpha * g'); bias is added before the clamp.
* LoRA sits on gate_up only, A [r, H] and B [2I, r]; scale = alpha / r.
* Backward covers the expert path only (router logits are given inputs):
  dX, dA, dB; the frozen base and biases get no gradient. Clamp derivatives
  pass where the clamp is inactive, boundaries included.
* The clamped GLU is continuous but its derivative jumps at g = limit and at
  u = +-limit. A value computed in fp32 that lies within its rounding error of
  such a point may fall on either side of it, and either side's derivative is
  then a valid result; ``clamp_flip`` names entries whose side is taken
  opposite to the side their oracle value falls on (for comparisons against
  an fp32 computation; the default takes every side as the value says).
* Likewise, the bf16 rounding of dGU (a GEMM operand) is decided on a value
  that an fp32 computation carries with an error of its own: where the exact
  value lies close to a rounding midpoint, either neighbouring bf16 value is
  a valid operand. ``round_flip`` names dGU entries that take the other
  neighbour (the default rounds every entry to the nearest).
* Precision: bf16 model tensors with fp32 accumulation (solutions index,
  grouped-nf4-gemm entries; experts4bit-qlora page, the adapter runs in the
  model dtype, bf16). The oracle rounds to bf16 exactly where a value becomes
  an operand of a bf16 GEMM -- the dequantised NF4 weight
  bf16(fp32(level * absmax)) (MXFP4 values are exact in bf16), h, xa before
  the B product, dGU, and t = dGU B before the A product -- and where the
  interface defines a bf16 tensor (the row-scaled gradient). Every sum and
  every output stays float64. exact=True drops all of these roundings (the
  backward is pinned against finite differences in that mode).
"""

from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

from .formats import dequantize_nf4, dequantize_nf4_bf16, mxfp4_values
from .numerics import (bf16_bits_from_f32, bf16_bits_to_f64, bf16_other_neighbour_f64,
                       bf16_round_f64)
from .routing import permute

HALVES = "halves"
INTERLEAVED = "interleaved"
SWIGLU = "swiglu"
SWIGLU_CLAMPED = "swiglu_clamped"


@dataclass
class ExpertWeights:
    """Dense float64 view of one layer's experts, materialised per expert on
    demand (so a large stack never has to be dense all at once)."""
    E: int
    H: int
    I: int
    layout: str
    act: str
    gu: Callable[[int], np.ndarray]          # e -> [2I, H]
    dn: Callable[[int], np.ndarray]          # e -> [H, I]
    b_gu: Optional[Callable[[int], np.ndarray]] = None   # e -> [2I]
    b_dn: Optional[Callable[[int], np.ndarray]] = None   # e -> [H]
    lora_A: Optional[Callable[[int], np.ndarray]] = None  # e -> [r, H]
    lora_B: Optional[Callable[[int], np.ndarray]] = None  # e -> [2I, r]
    lora_scale: float = 0.0
    alpha: float = 1.702
    limit: float = 7.0
    _cache: dict = field(default_factory=dict, repr=False)

    def expert(self, e):
        if e not in self._cache:
            if len(self._cache) > 8:
                self._cache.clear()
            self._cache[e] = (self.gu(e), self.dn(e))
        return self._cache[e]

    @staticmethod
    def _bias(stack):
        if stack is None:
            return None
        arr = np.asarray(stack, dtype=np.uint16)
        return lambda e: bf16_bits_to_f64(arr[e])

    @classmethod
    def from_nf4(cls, gu_packed, gu_absmax, dn_packed, dn_absmax, *, layout, act,
                 gu_bias=None, dn_bias=None, lora_A=None, lora_B=None,
                 lora_scale=0.0, alpha=1.702, limit=7.0, bf16_weights=True):
        """Stacks: gu_packed [E,2I,H/2], gu_absmax [E,2I,H/64],
        dn_packed [E,H,I/2], dn_absmax [E,H,I/64]; bf16 bits for biases and
        adapters (A [E,r,H], B [E,2I,r]). bf16_weights=False keeps the exact
        level * absmax values instead of the bf16 GEMM operands."""
        E, N2, Hh = gu_packed.shape
        H, I = Hh * 2, N2 // 2
        deq = dequantize_nf4_bf16 if bf16_weights else dequantize_nf4
        return cls(
            E=E, H=H, I=I, layout=layout, act=act,
            gu=lambda e: deq(gu_packed[e], gu_absmax[e]).reshape(2 * I, H),
            dn=lambda e: deq(dn_packed[e], dn_absmax[e]).reshape(H, I),
            b_gu=cls._bias(gu_bias), b_dn=cls._bias(dn_bias),
            lora_A=cls._bias(lora_A), lora_B=cls._bias(lora_B),
            lora_scale=lora_scale, alpha=alpha, limit=limit)

    @classmethod
    def from_mxfp4(cls, gu_blocks, gu_scales, dn_blocks, dn_scales, *, layout, act,
                   gu_bias=None, dn_bias=None, lora_A=None, lora_B=None,
                   lora_scale=0.0, alpha=1.702, limit=7.0):
        """Stacks: gu_blocks [E,2I,H/32,16], gu_scales [E,2I,H/32],
        dn_blocks [E,H,I/32,16], dn_scales [E,H,I/32]."""
        E, N2, KB, _ = gu_blocks.shape
        H, I = KB * 32, N2 // 2
        return cls(
            E=E, H=H, I=I, layout=layout, act=act,
            gu=lambda e: mxfp4_values(gu_blocks[e], gu_scales[e]),
            dn=lambda e: mxfp4_values(dn_blocks[e], dn_scales[e]),
            b_gu=cls._bias(gu_bias), b_dn=cls._bias(dn_bias),
            lora_A=cls._bias(lora_A), lora_B=cls._bias(lora_B),
            lora_scale=lora_scale, alpha=alpha, limit=limit)


def _as_f64(a):
    """bf16 bit patterns (uint16) -> exact float64; float arrays pass through."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def _sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def split_gate_up(gu, layout, I):
    if layout == HALVES:
        return gu[:, :I], gu[:, I:]
    if layout == INTERLEAVED:
        return gu[:, 0::2], gu[:, 1::2]
    raise ValueError("unknown gate/up layout")


def join_gate_up(g, u, layout):
    n, I = g.shape
    out = np.empty((n, 2 * I), dtype=np.float64)
    if layout == HALVES:
        out[:, :I], out[:, I:] = g, u
    elif layout == INTERLEAVED:
        out[:, 0::2], out[:, 1::2] = g, u
    else:
        raise ValueError("unknown gate/up layout")
    return out


def _op(v, exact):
    """A value handed to a bf16 GEMM operand (unchanged when exact)."""
    return v if exact else bf16_round_f64(v)


def gate_up(X, W, e, exact=False):
    """gu = X W_gu[e]^T + bias + LoRA delta, float64 [n, 2I]; also returns
    xa = X A_e^T (float64, before its bf16 rounding; or None)."""
    Wgu, _ = W.expert(e)
    gu = X @ Wgu.T
    if W.b_gu is not None:
        gu = gu + W.b_gu(e)[None, :]
    xa = None
    if W.lora_A is not None:
        xa = X @ W.lora_A(e).T
        gu = gu + W.lora_scale * (_op(xa, exact) @ W.lora_B(e).T)
    return gu, xa


def activation(gu, W):
    g, u = split_gate_up(gu, W.layout, W.I)
    if W.act == SWIGLU:
        return g * _sigmoid(g) * u
    if W.act == SWIGLU_CLAMPED:
        gc = np.minimum(g, W.limit)
        uc = np.clip(u, -W.limit, W.limit)
        return (uc + 1.0) * gc * _sigmoid(W.alpha * gc)
    raise ValueError("unknown activation")


def activation_backward(gu, dh, W, flip=None):
    """d(loss)/d(gu) given d(loss)/d(h), in the stack's gate/up layout.

    flip (clamped GLU only): bool array shaped like gu; where True, the clamp
    of that entry is taken as the other side of its boundary decides (active
    for a value inside [-limit, limit] (up) or <= limit (gate), inactive
    otherwise)."""
    g, u = split_gate_up(gu, W.layout, W.I)
    if W.act == SWIGLU:
        s = _sigmoid(g)
        du = dh * g * s
        dg = dh * u * s * (1.0 + g * (1.0 - s))
    elif W.act == SWIGLU_CLAMPED:
        gc = np.minimum(g, W.limit)
        uc = np.clip(u, -W.limit, W.limit)
        sa = _sigmoid(W.alpha * gc)
        pass_u = (u >= -W.limit) & (u <= W.limit)
        pass_g = g <= W.limit
        if flip is not None:
            fg, fu = split_gate_up(np.asarray(flip, dtype=bool), W.layout, W.I)
            pass_g, pass_u = pass_g ^ fg, pass_u ^ fu
        du = dh * gc * sa * pass_u
        dg = dh * (uc + 1.0) * (sa + W.alpha * gc * sa * (1.0 - sa)) * pass_g
    else:
        raise ValueError("unknown activation")
    return join_gate_up(dg, du, W.layout)


def down(h, W, e):
    _, Wd = W.expert(e)
    y = h @ Wd.T
    if W.b_dn is not None:
        y = y + W.b_dn(e)[None, :]
    return y


def combine(y, row_of_slot, topk_w, T, k):
    """out[t] = sum_j w[t,j] * y[row_of_slot[t*k+j]] (w = None: plain sum)."""
    y = np.asarray(y, dtype=np.float64)
    rows = np.asarray(row_of_slot, dtype=np.int64).reshape(T, k)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        wj = 1.0 if topk_w is None else np.asarray(topk_w, dtype=np.float64)[:, j:j + 1]
        out += wj * y[rows[:, j]]
    return out


def layer_forward(x_bits, topk_idx, topk_w, W, keep=False, exact=False):
    """Whole-layer forward (x: bf16 bits or float64 [T,H]). Returns a dict
    with ``out`` [T,H], ``y`` [T*k,H] and, with keep=True, the per-row
    intermediates (``gu``, ``h`` as the bf16 operand, ``xa``)."""
    x = _as_f64(x_bits)
    T, k = np.asarray(topk_idx).shape
    offsets, slot_of_row, row_of_slot = permute(topk_idx, W.E)
    rows = T * k
    y = np.zeros((rows, W.H))
    res = {"offsets": offsets, "slot_of_row": slot_of_row, "row_of_slot": row_of_slot}
    if keep:
        res["gu"] = np.zeros((rows, 2 * W.I))
        res["h"] = np.zeros((rows, W.I))
        if W.lora_A is not None:
            res["xa"] = np.zeros((rows, W.lora_A(0).shape[0]))
    for e in range(W.E):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            continue
        X = x[slot_of_row[a:b] // k]
        gu, xa = gate_up(X, W, e, exact)
        h = _op(activation(gu, W), exact)
        y[a:b] = down(h, W, e)
        if keep:
            res["gu"][a:b], res["h"][a:b] = gu, h
            if xa is not None:
                res["xa"][a:b] = xa
    res["y"] = y
    res["out"] = combine(y, row_of_slot, topk_w, T, k)
    return res


def token_forward(x_row_bits, experts, weights, W, exact=False):
    """out for one token: sum_j w_j * expert_j(x). For sampled checks at sizes
    where the whole layer is too slow on the host."""
    x = _as_f64(x_row_bits).reshape(1, -1)
    out = np.zeros(W.H)
    for e, w in zip(experts, weights):
        gu, _ = gate_up(x, W, int(e), exact)
        out += float(w) * down(_op(activation(gu, W), exact), W, int(e))[0]
    return out


def layer_backward(x_bits, topk_idx, topk_w, dout_bits, W, exact=False, clamp_flip=None,
                   round_flip=None):
    """Gradient of sum_t <dOut[t], out[t]> with respect to x, A and B.

    Returns dict with ``dx`` [T,H], ``dA`` [E,r,H], ``dB`` [E,2I,r] (zero for
    experts that receive no rows), plus the per-row ``dgu`` and ``dx_perm``.
    Unless exact, the routing weights enter as fp32 (the interface's dtype) and
    the scaled upstream gradient is bf16(fp32(w * dOut)). clamp_flip: None, or
    a bool array [T*k, 2I] in permuted-row order and the stack's gate/up
    layout, passed row by row to ``activation_backward``. round_flip: None, or
    a bool array of the same shape; where True, that dGU entry is rounded to
    the other bf16 neighbour of its exact value (``bf16_other_neighbour_f64``).
    Also returned: ``dgu_exact`` (dGU before its rounding) and ``dh``.
    """
    x = _as_f64(x_bits)
    dout = _as_f64(dout_bits)
    T, k = np.asarray(topk_idx).shape
    w = np.asarray(topk_w, dtype=np.float64).reshape(-1)
    offsets, slot_of_row, row_of_slot = permute(topk_idx, W.E)
    rows = T * k
    dx_perm = np.zeros((rows, W.H))
    dgu_all = np.zeros((rows, 2 * W.I))
    dgu_exact_all = np.zeros((rows, 2 * W.I))
    dh_all = np.zeros((rows, W.I))
    lora = W.lora_A is not None
    r = W.lora_A(0).shape[0] if lora else 0
    dA = np.zeros((W.E, r, W.H))
    dB = np.zeros((W.E, 2 * W.I, r))
    for e in range(W.E):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            continue
        slots = slot_of_row[a:b]
        X = x[slots // k]
        if exact:
            dY = w[slots][:, None] * dout[slots // k]
        else:
            prod = (w[slots].astype(np.float32)[:, None] *
                    dout[slots // k].astype(np.float32)).astype(np.float32)
            dY = bf16_bits_to_f64(bf16_bits_from_f32(prod))
        gu, xa = gate_up(X, W, e, exact)
        Wgu, Wd = W.expert(e)
        dH = dY @ Wd
        flip = None if clamp_flip is None else np.asarray(clamp_flip)[a:b]
        dGU_exact = activation_backward(gu, dH, W, flip)
        dGU = _op(dGU_exact, exact)
        if round_flip is not None and not exact:
            dGU = np.where(np.asarray(round_flip)[a:b], bf16_other_neighbour_f64(dGU_exact), dGU)
        dX = dGU @ Wgu
        if lora:
            A, B = W.lora_A(e), W.lora_B(e)
            t = _op(dGU @ B, exact)
            dX = dX + W.lora_scale * (t @ A)
            dB[e] = W.lora_scale * (dGU.T @ _op(xa, exact))
            dA[e] = W.lora_scale * (t.T @ X)
        dx_perm[a:b] = dX
        dgu_all[a:b] = dGU
        dgu_exact_all[a:b] = dGU_exact
        dh_all[a:b] = dH
    dx = combine(dx_perm, row_of_slot, None, T, k)
    return {"dx": dx, "dA": dA, "dB": dB, "dx_perm": dx_perm, "dgu": dgu_all,
            "dgu_exact": dgu_exact_all, "dh": dh_all,
            "offsets": offsets, "slot_of_row": slot_of_row, "row_of_slot": row_of_slot}
