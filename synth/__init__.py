"""Seeded synthetic inputs for the packed ternary decode workloads.

This module only draws numbers; it holds none of the method's arithmetic.
Both the CPU oracle and the GPU path take their inputs from here, so the two
sides see bit-identical logical arrays.

Distributions follow the workloads of the page "The Neutrino Engine"
(fermionresearch.com), section "The file is not the traffic": 36 decoder
layers whose q/k/v/o/gate/up/down projections are ternary with per-row
scales, and two untied int8 vocabulary tables of 151,936 x 4,096.  The pages
give no value distributions; the ones used here are:

* ternary weights: iid uniform over {-1, 0, +1} (p = 1/3 each), int8;
* ternary row scales: U[0.01, 0.1], drawn in float64, stored as float32;
* activations: N(0, 1), drawn in float64, stored as float32;
* int8 tables: iid uniform integers in [-127, 127] (-128 never occurs);
* int8 row scales: U[0.001, 0.01], float32;
* token ids: uniform integers in [0, rows).

Seeding: every array has a numpy ``SeedSequence`` key ``[workload, layer,
item]`` and is drawn from its own ``default_rng`` in a fixed order (weights,
then scales).  Activations have their own keys.  The single 1024 x 1024 GEMV
uses ``default_rng(0)`` and draws W, then s, then x.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

HIDDEN = 4096
INTERMEDIATE = 12288
N_LAYERS = 36
VOCAB = 151936
KV_HEADS = 8
HEAD_DIM = 128

# (rows, cols) of each projection in one decoder layer of the 8B shape.
LAYER_SHAPES = {
    "q": (4096, 4096),
    "k": (1024, 4096),
    "v": (1024, 4096),
    "o": (4096, 4096),
    "gate": (12288, 4096),
    "up": (12288, 4096),
    "down": (4096, 12288),
}
MATRIX_ORDER = ("q", "k", "v", "o", "gate", "up", "down")
MATRIX_INDEX = {m: i for i, m in enumerate(MATRIX_ORDER)}

# Dependency levels of one layer: matrices that read the same input vector are
# stacked by rows and run as one GEMV.  (level name, member matrices, input length)
LEVELS = (
    ("qkv", ("q", "k", "v"), HIDDEN),
    ("o", ("o",), HIDDEN),
    ("gate_up", ("gate", "up"), HIDDEN),
    ("down", ("down",), INTERMEDIATE),
)

# Workload ids used as the first element of every seed key.
W_SINGLE, W_LAYER, W_VOCAB, W_STEP, W_BATCH = 1, 2, 3, 4, 5
# Item ids of the chained step's RMSNorm gains: 200 (attention norm), 201
# (feed-forward norm) inside a layer; the final norm is layer -1's item 202.
GAIN_ATTN, GAIN_MLP, GAIN_FINAL = 200, 201, 202

# Item ids inside a layer: 0..6 are the matrices, 100+i the level inputs.
X_ITEM_BASE = 100


def rng_for(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def ternary(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """iid uniform {-1, 0, +1} as int8, row-major (rows, cols)."""
    return rng.integers(-1, 2, size=(rows, cols), dtype=np.int8)


def uniform_f32(rng: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    return rng.uniform(lo, hi, size=n).astype(np.float32)


def normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape).astype(np.float32)


def int8_uniform(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    return rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)


@dataclass
class TernaryMatrix:
    w: np.ndarray      # int8 (rows, cols), values in {-1, 0, 1}
    scale: np.ndarray  # float32 (rows,)


def ternary_matrix(key, rows: int, cols: int, scale_lo=0.01, scale_hi=0.1) -> TernaryMatrix:
    rng = rng_for(*key)
    w = ternary(rng, rows, cols)
    s = uniform_f32(rng, rows, scale_lo, scale_hi)
    return TernaryMatrix(w, s)


def single_gemv(rows: int = 1024, cols: int = 1024, seed: int = 0):
    """The single-GEMV workload: W, then s, then x from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    w = ternary(rng, rows, cols)
    s = uniform_f32(rng, rows, 0.01, 0.1)
    x = normal_f32(rng, cols)
    return w, s, x


def layer(workload: int, layer_idx: int, shapes=None) -> dict:
    """All seven ternary matrices of one decoder layer."""
    shapes = shapes or LAYER_SHAPES
    return {m: ternary_matrix((workload, layer_idx, MATRIX_INDEX[m]), *shapes[m]) for m in MATRIX_ORDER}


def layer_inputs(workload: int, layer_idx: int, batch: int | None = None, hidden=HIDDEN, inter=INTERMEDIATE) -> dict:
    """Fixed N(0,1) inputs of the four levels (one shared by q/k/v, one for o,
    one shared by gate/up, one of the intermediate length for down)."""
    out = {}
    for i, (name, _, _) in enumerate(LEVELS):
        n = inter if name == "down" else hidden
        shape = n if batch is None else (batch, n)
        out[name] = normal_f32(rng_for(workload, layer_idx, X_ITEM_BASE + i), shape)
    return out


def stacked(mats: dict, names) -> TernaryMatrix:
    """Stack member matrices of a level by rows (q|k|v, gate|up)."""
    return TernaryMatrix(np.concatenate([mats[n].w for n in names], axis=0),
                         np.concatenate([mats[n].scale for n in names], axis=0))


@dataclass
class Int8Table:
    q: np.ndarray      # int8 (rows, cols)
    scale: np.ndarray  # float32 (rows,)


def int8_table(key, rows: int = VOCAB, cols: int = HIDDEN, scale_lo=0.001, scale_hi=0.01) -> Int8Table:
    rng = rng_for(*key)
    q = int8_uniform(rng, rows, cols)
    t = uniform_f32(rng, rows, scale_lo, scale_hi)
    return Int8Table(q, t)


def vocab_workload(rows: int = VOCAB, cols: int = HIDDEN, n_ids: int = 64, workload: int = W_VOCAB):
    """Output table + scales, hidden state, embedding table + scales, ids."""
    out_table = int8_table((workload, 0), rows, cols)
    emb_table = int8_table((workload, 1), rows, cols)
    ids = rng_for(workload, 2).integers(0, rows, size=n_ids).astype(np.int32)
    h = normal_f32(rng_for(workload, 3), cols)
    return out_table, emb_table, ids, h


def batch_inputs(batch: int, n: int, j: int) -> np.ndarray:
    return normal_f32(rng_for(W_BATCH, batch, j), (batch, n))


def n_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def parallel_map(fn, items):
    """Run independent generator calls on a thread pool (numpy releases the
    GIL for most of the drawing); results keep the order of ``items``."""
    with ThreadPoolExecutor(n_workers()) as ex:
        return list(ex.map(fn, items))


def norm_gain(workload: int, layer: int, item: int, n: int) -> np.ndarray:
    """RMSNorm gain of a chained step: float32 U[0.5, 1.5] (the pages give
    none; trained gains sit around 1)."""
    return uniform_f32(rng_for(workload, layer if layer >= 0 else 1_000_000, item), n, 0.5, 1.5)


W_ATTN = 6  # workload id of the decode-attention inputs


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (input
    generation only; finite inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def kv_cache(layer: int, ctx: int, n_kv: int = KV_HEADS, head_dim: int = HEAD_DIM, seed: int = 0):
    """One layer's bfloat16 key and value caches [ctx, n_kv, head_dim] of
    N(0,1) values, and an N(0,1) float32 query for 4 query heads per
    key/value head."""
    rng = rng_for(W_ATTN, seed, layer)
    k = bf16_bits(rng.standard_normal((ctx, n_kv, head_dim)).astype(np.float32))
    v = bf16_bits(rng.standard_normal((ctx, n_kv, head_dim)).astype(np.float32))
    q = rng.standard_normal(4 * n_kv * head_dim).astype(np.float32)
    return q, k, v


W_OUTLIER = 7  # workload id of the outlier activation vectors


def outlier_vector(n: int, seed: int, background: str = "normal", n_outliers: int = 6, n_quiet: int = 2) -> np.ndarray:
    """An activation vector with massive outliers, as decoder hidden states
    carry them: a background of N(0, 1) values ("normal") or of N(0, 1) x 1e-3
    values ("small"); `n_outliers` positions set to +-3e3 or +-1e4; and
    `n_quiet` aligned 64-value stretches whose values are U(-1e-3, 1e-3)
    except one +-1e4 outlier at a random place inside (an outlier among small
    values).  float32; drawn in float64."""
    rng = rng_for(W_OUTLIER, n, seed)
    x = rng.standard_normal(n)
    if background == "small":
        x *= 1e-3
    elif background != "normal":
        raise ValueError(background)
    stretches = n // 64
    quiet = rng.choice(stretches, size=min(n_quiet, stretches), replace=False) if stretches else []
    for s in quiet:
        x[64 * s:64 * s + 64] = rng.uniform(-1e-3, 1e-3, size=64)
        x[64 * s + rng.integers(0, 64)] = rng.choice([-1e4, 1e4])
    free = np.setdiff1d(np.arange(n), np.concatenate([np.arange(64 * s, 64 * s + 64) for s in quiet]) if len(quiet) else [])
    pos = rng.choice(free, size=min(n_outliers, len(free)), replace=False)
    x[pos] = rng.choice([-1e4, -3e3, 3e3, 1e4], size=len(pos))
    return x.astype(np.float32)
