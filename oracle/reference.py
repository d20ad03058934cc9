"""Plain float64 reference of what one batch-1 decode step computes.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Source: the page "The Neutrino Engine" (fermionresearch.com).

* Section "A 104 microsecond floor inside a 694 microsecond step": every
  decoder layer applies its attention and feed-forward projection matrices to
  the current activation vector; at batch one each weight is used for one
  multiply-accumulate per token; the output projection scores the final hidden
  state against the whole vocabulary.
* Section "The file is not the traffic": projection weights are ternary and
  carry row scales; the two vocabulary tables are int8 with 151,936 rows of
  4,096; input embedding reads only the selected rows, output projection reads
  the whole output table.
* Intro and section "The same weights take four execution paths": decode is
  greedy, so the next token is the argmax of the logits.

Readings where the pages are silent (each listed in the design notes):
row scales are float32 and multiply the finished dot product once
(y_r = s_r * sum_k W_rk x_k); activations are float32; argmax ties go to the
lowest index; embedding dequantisation is one float32 product E[id,k] * e[id].

Every product w * x here is exact in float64 (w is -1, 0, +1 or an int8 and x
is a float32), and sums are float64 dot products, so results carry only the
rounding of float64 summation.  Matrices are processed in row blocks purely to
bound memory; each output row is computed the same way regardless.

Pins (tests marked "not gpu"): balanced-ternary closed form over every
ternary row of length 8, one-hot inputs, all-ones and zero matrices, sign and
linearity invariants, non-square shapes, permutation invariance, planted
argmax and ties, exact power-of-two dequantisation.
"""
from __future__ import annotations

import numpy as np

_ROW_BLOCK = 2048


def _rowwise_dot(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """sum_k w[r, k] * x[..., k] in float64 for every row r.

    x is (K,) or (B, K); the result is (R,) or (B, R)."""
    x64 = np.asarray(x, dtype=np.float64)
    rows = w.shape[0]
    if x64.ndim == 1:
        out = np.empty(rows, dtype=np.float64)
        for r0 in range(0, rows, _ROW_BLOCK):
            out[r0:r0 + _ROW_BLOCK] = w[r0:r0 + _ROW_BLOCK].astype(np.float64) @ x64
        return out
    out = np.empty((x64.shape[0], rows), dtype=np.float64)
    for r0 in range(0, rows, _ROW_BLOCK):
        out[:, r0:r0 + _ROW_BLOCK] = x64 @ w[r0:r0 + _ROW_BLOCK].astype(np.float64).T
    return out


def ternary_gemv(w: np.ndarray, scale: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y[r] = scale[r] * sum_k w[r, k] * x[k]   (x may be a (B, K) batch).

    w: int8 (R, K) with entries in {-1, 0, +1}; scale: float32 (R,);
    x: float32 (K,) or (B, K).  Returns float64."""
    w = np.asarray(w)
    if w.ndim != 2:
        raise ValueError("w must be 2-D")
    if not np.isin(w, (-1, 0, 1)).all():
        raise ValueError("ternary weights must be in {-1, 0, +1}")
    return np.asarray(scale, dtype=np.float64) * _rowwise_dot(w, x)


def ternary_gemv_magnitude(w: np.ndarray, scale: np.ndarray, x: np.ndarray) -> np.ndarray:
    """|scale[r]| * sum_k |w[r, k]| * |x[k]|: the size of the terms that a row
    sums.  Used as the cancellation floor of the element-wise parity bound."""
    return np.abs(np.asarray(scale, dtype=np.float64)) * _rowwise_dot(np.abs(np.asarray(w)), np.abs(x))


def int8_logits(table: np.ndarray, scale: np.ndarray, h: np.ndarray) -> np.ndarray:
    """logit[v] = scale[v] * sum_k table[v, k] * h[k]   (h may be (B, K)).

    table: int8 (V, K); scale: float32 (V,); h: float32.  Returns float64."""
    table = np.asarray(table)
    if table.dtype != np.int8:
        raise ValueError("vocabulary table must be int8")
    return np.asarray(scale, dtype=np.float64) * _rowwise_dot(table, h)


def int8_logits_magnitude(table: np.ndarray, scale: np.ndarray, h: np.ndarray) -> np.ndarray:
    return np.abs(np.asarray(scale, dtype=np.float64)) * _rowwise_dot(np.abs(np.asarray(table, dtype=np.int16)), np.abs(h))


def greedy_token(logits: np.ndarray):
    """Greedy decode of one logit vector: (token, gap).

    token is the index of the largest logit, the lowest such index on ties;
    gap is the largest logit minus the largest logit at any other index
    (0 when the maximum is tied)."""
    logits = np.asarray(logits, dtype=np.float64)
    if logits.ndim != 1 or logits.size == 0:
        raise ValueError("need a non-empty 1-D logit vector")
    token = int(np.argmax(logits))  # first occurrence of the maximum
    if logits.size == 1:
        return token, float("inf")
    rest = np.delete(logits, token)
    return token, float(logits[token] - rest.max())


def accepted_tokens(logits: np.ndarray, tol: float) -> np.ndarray:
    """Indices whose logit lies within tol of the maximum (the ids a greedy
    decode may legitimately return when the top logits are that close)."""
    logits = np.asarray(logits, dtype=np.float64)
    return np.flatnonzero(logits >= logits.max() - tol)


def embed_gather(table: np.ndarray, scale: np.ndarray, ids, dequant: bool = True):
    """Rows table[ids], their scales, and optionally the float32 dequantised
    rows table[id, k] * scale[id] (one float32 product, rounded once)."""
    table = np.asarray(table)
    ids = np.asarray(ids, dtype=np.int64)
    if ids.size and (ids.min() < 0 or ids.max() >= table.shape[0]):
        raise IndexError("token id out of range")
    rows = table[ids].copy()
    scales = np.asarray(scale, dtype=np.float32)[ids].copy()
    deq = None
    if dequant:
        deq = rows.astype(np.float32) * scales[:, None]
    return rows, scales, deq


def decode_step(levels, out_table, out_scale, h, emb_table, emb_scale, token_in):
    """One decode step of the fixed-input weight stream.

    levels: sequence over layers of sequences of (w, scale, x), in decoder
    order (q|k|v stacked, o, gate|up stacked, down).  Each level is a ternary
    GEMV of its own fixed input; the output projection scores h against the
    whole output table and the greedy token is its argmax; the embedding row
    of token_in is gathered.  Returns a dict with every level output, the
    logits, the token and the gathered row."""
    outs = [[ternary_gemv(w, s, x) for (w, s, x) in layer] for layer in levels]
    logits = int8_logits(out_table, out_scale, h)
    token, gap = greedy_token(logits)
    rows, scales, deq = embed_gather(emb_table, emb_scale, [token_in])
    return {"levels": outs, "logits": logits, "token": token, "gap": gap,
            "emb_row": rows[0], "emb_scale": scales[0], "emb_deq": deq[0]}
