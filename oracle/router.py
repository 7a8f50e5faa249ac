"""The router step in front of the expert path (test oracle).

Forward: fp32 router logits = x W_r^T (+ b_r), the input of ``route``. The
pages treat the logits as the place where equivalent forwards diverge:
rounding noise flips a share of top-k choices, so a GPU-vs-oracle routing
delta is read against a measured flip floor, never against zero
([experts4bit-qlora page], "Current measured position").

Backward: with out[t] = sum_j w[t,j] y[t,j] (y = the expert output of slot
t*k + j, before weighting), the routing-weight gradient is
dw[t,j] = <dOut[t], y[t,j]>; it reaches the logits through the softmax that
made the weights. Renormalised top-k weights are the softmax of the k chosen
logits alone, so d logits[t,e] = w_e (dw_e - sum_j w_j dw_j) for a chosen e
and 0 otherwise; without renormalisation the weights are the full softmax p
and d logits[t,e] = p_e (g_e - sum_j w_j dw_j), g_e = dw_j if e is chosen in
slot j, else 0. The top-k choice itself has no gradient.

Readings (the pages are silent; each also listed in the design notes):
* x and W_r are bf16 (the model dtype) and the logits are accumulated and
  stored in fp32; the oracle's logits are the exact sums (float64 over exact
  bf16 products), and the GPU's fp32 sums must lie within the standard
  worst-case bound of an fp32 dot product of that length;
* the router bias, when present, is fp32 and added to the sum;
* y is the fp32 expert output of each slot and dOut the bf16 upstream
  gradient at the layer output; dw and d logits are fp32 outputs.
"""

import numpy as np

from .numerics import bf16_bits_to_f64

U32 = 2.0 ** -24   # unit roundoff of fp32


def router_logits(x_bits, wr_bits, bias=None):
    """Exact logits (float64 [T,E]): sum_h x[t,h] W_r[e,h] (+ bias[e]). The
    products of two bf16 numbers are exact in float64, and the float64 sum's
    own rounding is far below the fp32 bound the GPU is held to."""
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    w = bf16_bits_to_f64(np.asarray(wr_bits, dtype=np.uint16))
    lg = x @ w.T
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return lg


def router_logits_error_bound(x_bits, wr_bits, bias=None):
    """Worst-case |fp32 result - exact| of each logit for any order of fp32
    additions: gamma_n * (sum_h |x w| + |b|) with n = H (+1 with a bias) and
    gamma_n = n u / (1 - n u), u = 2^-24 (the bf16 x bf16 products are exact
    in fp32), plus u * (sum |x w| + |b|) of slack for a partial sum formed in
    wider precision and rounded once to fp32."""
    x = np.abs(bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16)))
    w = np.abs(bf16_bits_to_f64(np.asarray(wr_bits, dtype=np.uint16)))
    mag = x @ w.T
    n = x.shape[1]
    if bias is not None:
        mag = mag + np.abs(np.asarray(bias, dtype=np.float32).astype(np.float64))[None, :]
        n += 1
    gamma = n * U32 / (1.0 - n * U32)
    return gamma * mag + U32 * mag


def routing_weight_grad(dout_bits, y, row_of_slot, k):
    """dw[t,j] = <dOut[t], y[row_of_slot[t*k + j]]> in float64; y [T*k, H]
    holds the slots' expert outputs in permuted-row order."""
    d = bf16_bits_to_f64(np.asarray(dout_bits, dtype=np.uint16))
    yy = np.asarray(y, dtype=np.float64)
    T = d.shape[0]
    rows = np.asarray(row_of_slot, dtype=np.int64).reshape(T, k)
    return np.einsum("th,tjh->tj", d, yy[rows])


def routing_logit_grad(topk_idx, topk_w, dw, E, renormalize=True, logits=None):
    """d logits [T,E] (float64) from dw [T,k] through the routing softmax.
    With renormalize=False the full softmax of ``logits`` (fp32 [T,E]) gives p."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    g = np.asarray(dw, dtype=np.float64)
    T, k = idx.shape
    out = np.zeros((T, E))
    for t in range(T):
        s = float(np.dot(w[t], g[t]))
        if renormalize:
            for j in range(k):
                out[t, idx[t, j]] = w[t, j] * (g[t, j] - s)
        else:
            row = np.asarray(logits, dtype=np.float32)[t].astype(np.float64)
            z = np.exp(row - row.max())
            p = z / z.sum()
            ge = np.zeros(E)
            ge[idx[t]] = g[t]
            out[t] = p * (ge - s)
    return out
