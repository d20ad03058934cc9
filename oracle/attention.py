"""Plain float64 reference of grouped-query decode attention over a 16-bit
key/value cache.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Source: the page "The Neutrino Engine" (fermionresearch.com), KV-cache
section: the cache holds, per layer, 8 key/value heads of 128 values at 2
bytes each for keys and for values, so it grows by 147,456 bytes per token
over 36 layers and overtakes the weights after about 26,000 tokens; at
decode every cached position is read once per token.

Readings (the pages give sizes only): the 16-bit type is bfloat16; the
cache of one layer is position-major, K[t][kv][d] and V[t][kv][d]; query
head j reads key/value head j // group; scores are q_j . k_t times a given
scale (1/sqrt(head_dim) in a transformer), softmax over the positions,
output the softmax-weighted sum of the value vectors.  Everything is float64
after decoding the bfloat16 bits (a bfloat16 is the upper 16 bits of a
float32).

Pins (tests marked "not gpu"): decoding of hand-made bfloat16 bit patterns;
one cached position reduces to oracle.chain's one-position attention;
identical keys give the mean of the values; a dominant score selects its
value vector; a constant added to every score of a head leaves the output
unchanged; permuting positions leaves it unchanged; a scalar-loop brute
force on tiny caches.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> values: the pattern is the upper
    half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def gqa_decode(q: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, n_heads: int, n_kv: int, head_dim: int,
               scale: float) -> np.ndarray:
    """q: float32 [n_heads * head_dim]; k_bits, v_bits: uint16 bfloat16
    [ctx, n_kv, head_dim].  Returns float64 [n_heads * head_dim]."""
    group = n_heads // n_kv
    q = np.asarray(q, dtype=np.float64).reshape(n_heads, head_dim)
    k = bf16_to_f64(k_bits).reshape(-1, n_kv, head_dim)
    v = bf16_to_f64(v_bits).reshape(-1, n_kv, head_dim)
    out = np.empty((n_heads, head_dim), dtype=np.float64)
    for j in range(n_heads):
        kv = j // group
        s = (k[:, kv, :] @ q[j]) * scale
        p = np.exp(s - s.max())
        out[j] = (p @ v[:, kv, :]) / p.sum()
    return out.reshape(-1)
