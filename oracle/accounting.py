"""Byte accounting of the 8B-shape model and its per-token traffic.

TEST INFRASTRUCTURE ONLY.

Closed forms from the layer shapes (q 4096x4096, k 1024x4096, v 1024x4096,
o 4096x4096, gate 12288x4096, up 12288x4096, down 4096x12288; 36 layers; two
int8 vocabulary tables of 151,936 x 4,096; 8 KV heads of 128 dims).  The page
"The Neutrino Engine" prints the totals these must reproduce:

* section "The file is not the traffic": a per-layer weight slab of
  72,351,744 bytes split 21.7 % attention / 78.3 % feed-forward; a 2.60 GB
  ternary lane that is 67.2 % of a 3.88 GB file; 1.24 GB (32.1 %) for the two
  vocabulary tables; 26 MB of metadata, row scales and norm vectors;
* section "A 104 microsecond floor ...": about 16 GB at fp16, about four
  times the artifact; about 1.5 TB/s of weight traffic at 396 tok/s;
* section "At 26K tokens, the cache becomes larger than the model":
  147,456 bytes (144 KiB) of keys and values per position, 0.60 / 2.42 /
  4.83 / 6.04 GB at 4,096 / 16,384 / 32,768 / 40,960 tokens, larger than the
  file after about 26,000 tokens, four times less than caching all 32 query
  heads.

The page gives no split of the 26 MB; only its total is used (its
composition is parity unpinned).
"""
from __future__ import annotations

LAYER_SHAPES = {
    "q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
    "gate": (12288, 4096), "up": (12288, 4096), "down": (4096, 12288),
}
ATTENTION = ("q", "k", "v", "o")
FEED_FORWARD = ("gate", "up", "down")
N_LAYERS = 36
VOCAB = 151936
HIDDEN = 4096
N_TABLES = 2
METADATA_BYTES = 26_000_000
KV_HEADS, HEAD_DIM, Q_HEADS = 8, 128, 32
KV_ELEM_BYTES = 2          # 16 bits per cached element
SLAB_BITS_PER_WEIGHT = 3   # 72,351,744 * 8 / weights_per_layer
T2_BITS_PER_WEIGHT = 2     # the build's packed format
SCALE_BYTES = 4            # float32 row scales


def weights_per_layer() -> int:
    return sum(r * c for r, c in LAYER_SHAPES.values())


def rows_per_layer() -> int:
    return sum(r for r, _ in LAYER_SHAPES.values())


def attention_share() -> float:
    att = sum(LAYER_SHAPES[m][0] * LAYER_SHAPES[m][1] for m in ATTENTION)
    return att / weights_per_layer()


def feed_forward_share() -> float:
    ff = sum(LAYER_SHAPES[m][0] * LAYER_SHAPES[m][1] for m in FEED_FORWARD)
    return ff / weights_per_layer()


def slab_bytes(bits_per_weight: int = SLAB_BITS_PER_WEIGHT) -> int:
    return weights_per_layer() * bits_per_weight // 8


def ternary_lane_bytes(bits_per_weight: int = SLAB_BITS_PER_WEIGHT) -> int:
    return N_LAYERS * slab_bytes(bits_per_weight)


def vocab_table_bytes() -> int:
    return N_TABLES * VOCAB * HIDDEN


def file_bytes() -> int:
    return ternary_lane_bytes() + vocab_table_bytes() + METADATA_BYTES


def fp16_params() -> int:
    return N_LAYERS * weights_per_layer() + N_TABLES * VOCAB * HIDDEN


def fp16_bytes() -> int:
    return 2 * fp16_params()


def kv_bytes_per_position() -> int:
    return N_LAYERS * KV_HEADS * HEAD_DIM * 2 * KV_ELEM_BYTES   # K and V


def kv_bytes(tokens: int) -> int:
    return tokens * kv_bytes_per_position()


def kv_crossover_tokens() -> int:
    """Smallest context whose cache exceeds the file."""
    return file_bytes() // kv_bytes_per_position() + 1


def kv_all_heads_ratio() -> float:
    return Q_HEADS / KV_HEADS


def file_traffic_rate(tokens_per_s: float) -> float:
    """Bytes per second if every token moved the whole file (how the page's
    'about 1.5 TB/s' and 'about 97 GB/s' figures relate to the token rate)."""
    return file_bytes() * tokens_per_s


def step_bytes(bits_per_weight: int = T2_BITS_PER_WEIGHT, n_layers: int = N_LAYERS) -> dict:
    """Algorithmic bytes one batch-1 step must read: every packed projection
    weight and its row scale, the whole output table and its scales, and one
    embedding row and its scale.  Activations are reported apart."""
    w = n_layers * weights_per_layer() * bits_per_weight // 8
    s = n_layers * rows_per_layer() * SCALE_BYTES
    out_table = VOCAB * HIDDEN + VOCAB * SCALE_BYTES
    emb_row = HIDDEN + SCALE_BYTES
    return {"ternary_weights": w, "ternary_scales": s, "output_table": out_table,
            "embedding_row": emb_row, "total": w + s + out_table + emb_row}


def level_bytes(rows: int, cols: int, bits_per_weight: int = T2_BITS_PER_WEIGHT) -> int:
    """Weights plus float32 row scales of one packed ternary GEMV."""
    return rows * cols * bits_per_weight // 8 + rows * SCALE_BYTES


def draft_cycle_fraction(draft_steps: int = 6, draft_ratio: float = 1 / 12) -> float:
    """Bytes of `draft_steps` draft steps plus one verify pass, relative to
    draft_steps + 1 plain steps (page section on speculative decoding)."""
    return (draft_steps * draft_ratio + 1) / (draft_steps + 1)


# ---------------------------------------------------------------- base-3 packing
# Five ternary weights per byte (3^5 = 243 <= 256): a row of c weights stores
# ceil(c / 5) bytes.  Its device arrangement cuts a row into 30-weight groups
# of 6 bytes and pads it to whole windows of 8 groups (48 bytes).
B3_TRITS = 5
B3_GROUP_BYTES = 6
B3_WINDOW_GROUPS = 8


def b3_row_bytes(cols: int) -> int:
    return -(-cols // B3_TRITS)


def b3_device_row_bytes(cols: int) -> int:
    groups = -(-b3_row_bytes(cols) // B3_GROUP_BYTES)
    return -(-groups // B3_WINDOW_GROUPS) * B3_WINDOW_GROUPS * B3_GROUP_BYTES


def b3_layer_bytes(device: bool = False) -> int:
    """Packed bytes of one layer's seven projections (row scales apart):
    stored form, or the device arrangement the kernels stream."""
    per_row = b3_device_row_bytes if device else b3_row_bytes
    return sum(r * per_row(c) for r, c in LAYER_SHAPES.values())


def b3_step_bytes(device: bool = False, n_layers: int = N_LAYERS) -> dict:
    """step_bytes() with the projections in the base-3 format."""
    w = n_layers * b3_layer_bytes(device)
    s = n_layers * rows_per_layer() * SCALE_BYTES
    out_table = VOCAB * HIDDEN + VOCAB * SCALE_BYTES
    emb_row = HIDDEN + SCALE_BYTES
    return {"ternary_weights": w, "ternary_scales": s, "output_table": out_table,
            "embedding_row": emb_row, "total": w + s + out_table + emb_row}
