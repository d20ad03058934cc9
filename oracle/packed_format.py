"""Encoder and decoder of the 2-bit packed ternary format "T2", written from
its specification (not from the library's packer).

TEST INFRASTRUCTURE ONLY.

The pages name their own packed tensor type but never describe its internals,
so T2 is the build's own format.  It is parity unpinned against the pages and
pinned by hand-written byte fixtures and round trips.

Specification:

* a logical matrix W in {-1, 0, +1}^(rows x cols), cols a multiple of 64;
* row-major: row r occupies bytes [r*cols/4, (r+1)*cols/4), a whole number of
  16-byte chunks;
* each row is a sequence of little-endian 32-bit words; word j holds the 16
  weights k = 16*j + m, m = 0..15;
* weight m of a word has its 2-bit code at bit position
      p(m) = 8*((m % 8) // 2) + 4*(m // 8) + 2*(m % 2),
  i.e. byte b of the word holds weights 2b, 2b+1 in its low nibble and
  8+2b, 9+2b in its high nibble, lower index in the lower bits;
* the code is the two's complement of w in 2 bits: 0 -> 0b00, +1 -> 0b01,
  -1 -> 0b11; 0b10 never occurs in a valid blob;
* the blob is exactly rows*cols/4 bytes, with no header; row scales are kept
  separately as float32.
"""
from __future__ import annotations

import numpy as np

# Device tile arrangement (load-time re-arrangement of the stored values, page
# "The Neutrino Engine", section "The same weights take four execution
# paths"), written from its definition:
#
# * input: a row-major byte matrix of `rows` rows of `row_bytes` bytes
#   (row_bytes a multiple of 64);
# * rows are padded with zero bytes to a multiple of 16;
# * tiles of 16 rows x 64 bytes (1 KiB) follow each other row-block by
#   row-block, and within a row block from the left: tile (rb, tc) is the
#   (rb * row_bytes / 64 + tc)-th 1 KiB of the output;
# * inside a tile, the byte of row 16 rb + i and column 64 tc + 16 q + b
#   (i < 16, q < 4, b < 16) sits at offset 256 q + 16 i + b.
TILE_ROWS = 16
TILE_BYTES = 64

INVALID_CODE = 0b10


def bit_position(m: int) -> int:
    """Bit offset, inside its 32-bit word, of weight m (0..15) of the word."""
    return 8 * ((m % 8) // 2) + 4 * (m // 8) + 2 * (m % 2)


def packed_nbytes(rows: int, cols: int) -> int:
    if rows < 0 or cols < 0 or cols % 64:
        raise ValueError("cols must be a non-negative multiple of 64")
    return rows * cols // 4


def encode(w: np.ndarray) -> np.ndarray:
    """Pack an int (rows, cols) ternary matrix into a uint8 blob."""
    w = np.asarray(w)
    rows, cols = w.shape
    packed_nbytes(rows, cols)
    if not np.isin(w, (-1, 0, 1)).all():
        raise ValueError("not ternary")
    codes = np.where(w < 0, 0b11, w).astype(np.uint32).reshape(rows, cols // 16, 16)
    words = np.zeros((rows, cols // 16), dtype=np.uint32)
    for m in range(16):
        words |= codes[:, :, m] << np.uint32(bit_position(m))
    return words.astype("<u4").view(np.uint8).reshape(-1)


def decode(blob, rows: int, cols: int) -> np.ndarray:
    """Unpack a blob into an int8 (rows, cols) matrix; rejects code 0b10."""
    if isinstance(blob, np.ndarray):
        b = np.ascontiguousarray(blob, dtype=np.uint8).reshape(-1)
    else:
        b = np.frombuffer(bytes(blob), dtype=np.uint8)
    if b.size != packed_nbytes(rows, cols):
        raise ValueError("blob size does not match rows*cols/4")
    words = b.view("<u4").reshape(rows, cols // 16)
    out = np.empty((rows, cols // 16, 16), dtype=np.int8)
    for m in range(16):
        code = (words >> np.uint32(bit_position(m))) & np.uint32(3)
        if (code == INVALID_CODE).any():
            r, j = np.argwhere(code == INVALID_CODE)[0]
            raise ValueError(f"invalid code 0b10 at row {r}, col {16 * j + m}")
        out[:, :, m] = np.where(code == 0b11, -1, code).astype(np.int8)
    return out.reshape(rows, cols)


def tiled_nbytes(rows: int, row_bytes: int) -> int:
    if rows < 1 or row_bytes < TILE_BYTES or row_bytes % TILE_BYTES:
        raise ValueError("rows >= 1 and row_bytes a positive multiple of 64")
    return -(-rows // TILE_ROWS) * TILE_ROWS * row_bytes


def tile16x64(mat: np.ndarray) -> np.ndarray:
    """The tile arrangement of a (rows, row_bytes) uint8 matrix, as a flat
    uint8 array: pad the rows with zeros, cut into 16 x 64 tiles, and inside a
    tile put the four 16-byte column quarters one after another, each holding
    the 16 rows' slices of that quarter in row order."""
    mat = np.ascontiguousarray(mat, dtype=np.uint8)
    rows, row_bytes = mat.shape
    out_rows = tiled_nbytes(rows, row_bytes) // row_bytes
    padded = np.zeros((out_rows, row_bytes), np.uint8)
    padded[:rows] = mat
    # axes: row block, row in block (i), tile column, quarter (q), byte (b)
    t = padded.reshape(out_rows // TILE_ROWS, TILE_ROWS, row_bytes // TILE_BYTES, 4, 16)
    # to: row block, tile column, quarter, row in block, byte
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1, 4)).reshape(-1)


def untile16x64(flat: np.ndarray, rows: int, row_bytes: int) -> np.ndarray:
    """Inverse of tile16x64 (drops the padding rows)."""
    flat = np.ascontiguousarray(flat, dtype=np.uint8).reshape(-1)
    n = tiled_nbytes(rows, row_bytes)
    if flat.size != n:
        raise ValueError("size does not match the tiled arrangement")
    out_rows = n // row_bytes
    t = flat.reshape(out_rows // TILE_ROWS, row_bytes // TILE_BYTES, 4, TILE_ROWS, 16)
    return np.ascontiguousarray(t.transpose(0, 3, 1, 2, 4)).reshape(out_rows, row_bytes)[:rows]
