"""Plain float64 reference of a chained batch-1 decode step: every level's
input is formed from earlier outputs, as in a real decoder layer.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Source: the page "The Neutrino Engine" (fermionresearch.com).

* Section "A 104 microsecond floor inside a 694 microsecond step": a decoder
  layer applies its attention and feed-forward matrices to the current
  activations, so each projection waits for the one before it; most of the
  measured step went to these dependency chains, not to DRAM.
* Section "The file is not the traffic": the layer matrices are ternary with
  row scales, the vocabulary tables int8 with 151,936 rows of 4,096; the
  KV-cache section gives 8 key/value heads of 128 per layer, so the query
  heads are grouped over them.

What the pages leave open and is read here (each listed in the design notes):
the glue between projections is the usual pre-norm decoder layer: RMSNorm
with a learned float32 gain (eps 1e-6) before the attention and before the
feed-forward block, residual adds after o and after down, SwiGLU
(silu(gate) * up) between gate|up and down, and a final RMSNorm before the
output projection; the step's first hidden state is the dequantised
embedding row of the previous token.  Attention is taken at the first
position of a sequence: with one cached key the softmax weight is exactly 1,
so every query head's output is the value vector of its key/value head (the
query and key projections are streamed but cannot change the result).

Everything is float64 except the embedding dequantisation, which is the
float32 product of the table entry and the row scale (rounded once), as in
reference.embed_gather.

Pins (tests marked "not gpu"): RMSNorm on constant and hand-worked vectors
and its scale invariance; SiLU at 0, at ln 3 (sigmoid 3/4) and the odd part
identity silu(x) - silu(-x) = x; one-position attention against a softmax
attention over one key and over repeated identical keys, and its group and
head-size special cases; whole steps against a scalar-loop brute force on
tiny shapes, and with zero o and down matrices (the hidden state is then the
embedding row in every layer).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import reference

EPS = 1e-6


def rms_norm(h: np.ndarray, gamma: np.ndarray, eps: float = EPS) -> np.ndarray:
    """gamma * h / sqrt(mean(h^2) + eps), in float64."""
    h = np.asarray(h, dtype=np.float64)
    return np.asarray(gamma, dtype=np.float64) * h / np.sqrt(np.mean(h * h) + eps)


def silu(g: np.ndarray) -> np.ndarray:
    """g * sigmoid(g), in float64 (written g / (1 + e^-g); e^-g may overflow
    to inf for very negative g, which gives the correct limit -0)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(gate_up: np.ndarray, inter: int) -> np.ndarray:
    """silu(gate) * up for the stacked gate|up output (gate first)."""
    gu = np.asarray(gate_up, dtype=np.float64)
    return silu(gu[:inter]) * gu[inter:2 * inter]


def attention_one_position(v: np.ndarray, n_heads: int, head_dim: int, group: int) -> np.ndarray:
    """Grouped-query attention output when the cache holds one position:
    query head j reads key/value head j // group, whose single softmax
    weight is 1, so its output is that head's value vector."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(n_heads * head_dim, dtype=np.float64)
    for j in range(n_heads):
        kv = j // group
        out[j * head_dim:(j + 1) * head_dim] = v[kv * head_dim:(kv + 1) * head_dim]
    return out


@dataclass
class ChainShape:
    hidden: int
    inter: int
    n_heads: int      # query heads
    n_kv: int         # key/value heads
    head_dim: int

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv

    @property
    def q_rows(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_rows(self) -> int:
        return self.n_kv * self.head_dim


def layer(h: np.ndarray, mats: dict, gammas: tuple, shape: ChainShape, eps: float = EPS) -> dict:
    """One pre-norm decoder layer at the first position.

    mats: "qkv", "o", "gate_up", "down" -> (w int8 ternary, scale float32);
    gammas: (attention-norm gain, feed-forward-norm gain).
    Returns every formed input, every level output and the new hidden state."""
    g_attn, g_mlp = gammas
    x_qkv = rms_norm(h, g_attn, eps)
    y_qkv = reference.ternary_gemv(*mats["qkv"], x_qkv)
    v = y_qkv[shape.q_rows + shape.kv_rows:shape.q_rows + 2 * shape.kv_rows]
    x_o = attention_one_position(v, shape.n_heads, shape.head_dim, shape.group)
    y_o = reference.ternary_gemv(*mats["o"], x_o)
    h_mid = np.asarray(h, dtype=np.float64) + y_o
    x_gu = rms_norm(h_mid, g_mlp, eps)
    y_gu = reference.ternary_gemv(*mats["gate_up"], x_gu)
    x_down = swiglu(y_gu, shape.inter)
    y_down = reference.ternary_gemv(*mats["down"], x_down)
    return {"x": [x_qkv, x_o, x_gu, x_down], "y": [y_qkv, y_o, y_gu, y_down],
            "h_mid": h_mid, "h_out": h_mid + y_down}


def chained_step(layers, gammas, g_final, shape: ChainShape, out_table, out_scale, emb_table, emb_scale,
                 token_in: int, eps: float = EPS) -> dict:
    """Whole chained step: embedding row of token_in -> every layer in order
    -> final RMSNorm -> int8 output projection -> greedy token."""
    _, _, deq = reference.embed_gather(emb_table, emb_scale, [token_in])
    h = deq[0].astype(np.float64)
    per_layer = []
    for mats, gm in zip(layers, gammas):
        r = layer(h, mats, gm, shape, eps)
        per_layer.append(r)
        h = r["h_out"]
    x_out = rms_norm(h, g_final, eps)
    logits = reference.int8_logits(out_table, out_scale, x_out)
    token, gap = reference.greedy_token(logits)
    return {"h0": deq[0], "layers": per_layer, "h_final": h, "x_out": x_out, "logits": logits,
            "token": token, "gap": gap}
