"""Encoder, decoder and device arrangement of the base-3 packed ternary format
"B3" (five weights per byte), written from its specification (not from the
library's packer or tiler).

TEST INFRASTRUCTURE ONLY.

Page "The Neutrino Engine", section "A 104 microsecond floor inside a 694
microsecond step": weight bytes over bandwidth bound a decode step, and a
smaller artifact lowers that bound on every backend.  A ternary weight
carries log2(3) = 1.585 bits; five of them (3^5 = 243 <= 256) fit one byte,
0.2 bytes per weight against the 2-bit format's 0.25 and against the pages'
72,351,744-byte slab per layer (section "The file is not the traffic").  The
pages do not describe their format's internals, so B3 is this library's own:
parity unpinned against the pages, pinned by hand-derived byte fixtures,
exhaustive code checks and round trips.

Specification (stored form):

* a logical matrix W in {-1, 0, +1}^(rows x cols), rows >= 0, cols >= 1;
* row-major: row r occupies bytes [r * B, (r + 1) * B) with
  B = ceil(cols / 5);
* byte m of a row holds the weights k = 5 m + i, i = 0..4, as base-3 digits
  d_i = w_k + 1 in {0, 1, 2}, least significant first:
      byte = d_0 + 3 d_1 + 9 d_2 + 27 d_3 + 81 d_4;
  weights past the end of the row (k >= cols) are 0 (digit 1);
* byte values 243..255 never occur in a valid blob;
* no header; row scales are kept separately as float32.

Device arrangement (the loader's load-time re-arrangement of the stored
values, page "The Neutrino Engine", section "The same weights take four
execution paths"):

* a row's bytes are cut into groups of 6 (30 weights); the row is padded
  with zero-weight bytes (value 121, all digits 1) to a whole number of
  8-group windows (48 bytes, 240 weights);
* rows are padded to a multiple of 16 with zero-weight rows (bytes 121);
* tile (rb, t) covers rows 16 rb .. 16 rb + 15 and groups 8 t .. 8 t + 7; the
  tiles follow each other row block by row block, t ascending, 768 bytes
  each;
* inside a tile, the 12 bytes at offset 12 L (L = 16 g + i, g < 4, i < 16)
  are group 8 t + g of row 16 rb + i followed by group 8 t + 4 + g of the same
  row.
"""
from __future__ import annotations

import numpy as np

TRITS = 5                 # weights per byte
GROUP_BYTES = 6           # bytes per 30-weight group
GROUP_WEIGHTS = TRITS * GROUP_BYTES
WINDOW_GROUPS = 8         # groups per tile column window
TILE_ROWS = 16
TILE_BYTES = TILE_ROWS * WINDOW_GROUPS * GROUP_BYTES   # 768
LANE_BYTES = 2 * GROUP_BYTES                            # 12
ZERO_BYTE = sum(3 ** i for i in range(TRITS))           # 121: five zero weights
MAX_CODE = 3 ** TRITS - 1                               # 242


def row_bytes(cols: int) -> int:
    """Stored bytes per row: ceil(cols / 5)."""
    if cols < 1:
        raise ValueError("cols must be >= 1")
    return -(-cols // TRITS)


def packed_nbytes(rows: int, cols: int) -> int:
    if rows < 0:
        raise ValueError("rows must be >= 0")
    return rows * row_bytes(cols)


def encode(w: np.ndarray) -> np.ndarray:
    """Pack an int (rows, cols) ternary matrix into a uint8 blob."""
    w = np.asarray(w)
    rows, cols = w.shape
    B = row_bytes(cols)
    if not np.isin(w, (-1, 0, 1)).all():
        raise ValueError("not ternary")
    digits = np.ones((rows, B * TRITS), dtype=np.int64)  # padding weights are 0: digit 1
    digits[:, :cols] = w.astype(np.int64) + 1
    digits = digits.reshape(rows, B, TRITS)
    out = np.zeros((rows, B), dtype=np.int64)
    for i in range(TRITS):
        out += digits[:, :, i] * 3 ** i
    return out.astype(np.uint8).reshape(-1)


def decode(blob, rows: int, cols: int) -> np.ndarray:
    """Unpack a blob into an int8 (rows, cols) matrix; rejects bytes > 242."""
    if isinstance(blob, np.ndarray):
        b = np.ascontiguousarray(blob, dtype=np.uint8).reshape(-1)
    else:
        b = np.frombuffer(bytes(blob), dtype=np.uint8)
    B = row_bytes(cols)
    if b.size != packed_nbytes(rows, cols):
        raise ValueError("blob size does not match rows * ceil(cols / 5)")
    v = b.astype(np.int64).reshape(rows, B)
    if (v > MAX_CODE).any():
        r, m = np.argwhere(v > MAX_CODE)[0]
        raise ValueError(f"invalid byte {v[r, m]} at row {r}, byte {m}")
    out = np.empty((rows, B, TRITS), dtype=np.int8)
    for i in range(TRITS):
        out[:, :, i] = (v // 3 ** i) % 3 - 1
    return out.reshape(rows, B * TRITS)[:, :cols]


def window_count(cols: int) -> int:
    """8-group windows (tiles) per row block."""
    groups = -(-row_bytes(cols) // GROUP_BYTES)
    return -(-groups // WINDOW_GROUPS)


def tiled_nbytes(rows: int, cols: int) -> int:
    if rows < 1:
        raise ValueError("rows must be >= 1")
    return -(-rows // TILE_ROWS) * window_count(cols) * TILE_BYTES


def tile(blob: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """The device arrangement of a stored blob, as a flat uint8 array."""
    b = np.ascontiguousarray(blob, dtype=np.uint8).reshape(-1)
    if b.size != packed_nbytes(rows, cols):
        raise ValueError("blob size does not match rows * ceil(cols / 5)")
    B = row_bytes(cols)
    T = window_count(cols)
    nrb = -(-rows // TILE_ROWS)
    padded = np.full((nrb * TILE_ROWS, T * WINDOW_GROUPS * GROUP_BYTES), ZERO_BYTE, np.uint8)
    padded[:rows, :B] = b.reshape(rows, B)
    # axes: row block, row in block (i), window (t), half (h: groups g / g + 4), g, byte
    v = padded.reshape(nrb, TILE_ROWS, T, 2, 4, GROUP_BYTES)
    # to: row block, window, g, i, half, byte  (lane L = 16 g + i; 12 bytes per lane)
    return np.ascontiguousarray(v.transpose(0, 2, 4, 1, 3, 5)).reshape(-1)


def decode_tiled(flat: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Reads the logical matrix back from the device arrangement, lane by
    lane (each lane's 12 bytes are two 30-weight groups), as a kernel sees
    it; independent of `tile`."""
    flat = np.ascontiguousarray(flat, dtype=np.uint8).reshape(-1)
    if flat.size != tiled_nbytes(rows, cols):
        raise ValueError("size does not match the B3 device arrangement")
    T = window_count(cols)
    nrb = flat.size // (T * TILE_BYTES)
    w = np.zeros((nrb * TILE_ROWS, T * WINDOW_GROUPS * GROUP_WEIGHTS), np.int8)
    for rb in range(nrb):
        for t in range(T):
            base = (rb * T + t) * TILE_BYTES
            for L in range(64):
                g, i = divmod(L, 16)
                lane = flat[base + LANE_BYTES * L: base + LANE_BYTES * (L + 1)].astype(np.int64)
                if (lane > MAX_CODE).any():
                    raise ValueError("invalid byte in the device arrangement")
                for half in range(2):
                    q = WINDOW_GROUPS * t + 4 * half + g
                    for j in range(GROUP_BYTES):
                        code = int(lane[GROUP_BYTES * half + j])
                        for d in range(TRITS):
                            w[TILE_ROWS * rb + i, GROUP_WEIGHTS * q + TRITS * j + d] = (code // 3 ** d) % 3 - 1
    pad = w[rows:]
    tail = w[:, cols:]
    if pad.any() or tail.any():
        raise ValueError("padding holds nonzero weights")
    return w[:rows, :cols]
