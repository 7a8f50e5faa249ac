"""Top-k routing and the permutation of token slots by expert (test oracle).

Routing: each token picks k of the E experts from fp32 router logits; the
weights are the softmax over all E, restricted to the chosen k and renormalised
to sum to one. The pages rely on this rule without spelling it out: rounding
noise flips a measurable share of top-k choices between equivalent forwards
([experts4bit-qlora page], "Current measured position", routing-flip claim),
which is why routing parity is defined here on given fp32 logits. The top-k
touches a small part of the expert set per token ([Offload page], "Why it
happens").

Readings (the pages are silent):
* selection is on the logits (softmax is monotone), larger first, equal
  logits -> lower expert index; +0 and -0 compare equal;
* slots are output in selection order;
* the permutation is the stable order of slots s = t*k + j by expert,
  i.e. ascending (expert, t, j).
"""

import numpy as np

from .numerics import bf16_bits_from_f32


def route(logits, k, renormalize=True):
    """Return (topk_idx int32 [T,k], topk_w float64 [T,k])."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if np.isnan(lg).any():
        raise ValueError("NaN logits are outside the definition")
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    experts = np.arange(E)
    for t in range(T):
        row = lg[t].astype(np.float64)
        # lexsort: last key is primary -> descending logit, then ascending index
        order = np.lexsort((experts, -row))
        sel = order[:k]
        idx[t] = sel
        z = np.exp(row - row.max())
        p = z / z.sum()
        ps = p[sel]
        w[t] = ps / ps.sum() if renormalize else ps
    return idx, w


def permute(topk_idx, E):
    """Counting sort of slots by expert.

    Returns (offsets int32 [E+1], slot_of_row int32 [T*k],
    row_of_slot int32 [T*k]). Rows of expert e are offsets[e]..offsets[e+1]-1,
    in ascending slot order.
    """
    e = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    if e.size and (e.min() < 0 or e.max() >= E):
        raise ValueError("expert index out of range")
    slot_of_row = np.argsort(e, kind="stable").astype(np.int32)
    row_of_slot = np.empty_like(slot_of_row)
    row_of_slot[slot_of_row] = np.arange(e.size, dtype=np.int32)
    counts = np.bincount(e, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return offsets, slot_of_row, row_of_slot


def gather_rows(x_bits, slot_of_row, k, row_scale=None):
    """x_perm[r] = x[slot_of_row[r] // k] as bf16 bits.

    With row_scale (float32 [T*k], indexed by slot) the row is
    bf16(fp32(row_scale[s] * x)): an IEEE fp32 product rounded once to bf16,
    as the interface defines it (used to scale the upstream gradient by the
    routing weight before the backward pass).
    """
    x = np.asarray(x_bits, dtype=np.uint16)
    s = np.asarray(slot_of_row, dtype=np.int64)
    rows = x[s // k]
    if row_scale is None:
        return rows.copy()
    xs = (rows.astype(np.uint32) << np.uint32(16)).view(np.float32)
    sc = np.asarray(row_scale, dtype=np.float32).reshape(-1)[s][:, None]
    prod = (sc * xs).astype(np.float32)
    return bf16_bits_from_f32(prod)
