"""The packed-blob header, written from its specification (not from the
library's code).

TEST INFRASTRUCTURE ONLY.

Page "The Neutrino Engine", sections "The same weights take four execution
paths" and "What ships": every path reads the same stored values, and a
converted pack must match the engine token for token.  The header lets a
reader check, before use, that a packed blob holds the logical matrix it
claims, whatever its packing: the checksum is taken over the logical values,
so the 2-bit and the base-3 packings of one matrix carry the same one.  The
pages do not describe a header; this one is the library's own.

Specification (64 bytes, little-endian):

    offset  size  field
    0       4     magic          0x42475750 ("PWGB")
    4       2     version        1
    6       2     layout         1 T2 row-major, 2 T2 tiled, 3 base-3 stored,
                                 4 base-3 device arrangement
    8       8     rows           int64, >= 1
    16      8     cols           int64, >= 1
    24      8     payload_bytes  bytes of the packed payload that follows
    32      8     logical_fnv1a  FNV-1a 64 of W as int8, row-major (rows*cols bytes)
    40      8     header_fnv1a   FNV-1a 64 of bytes 0..39
    48      16    reserved       zero

FNV-1a 64 (Fowler, Noll, Vo): h = 14695981039346656037; for each byte b:
h = (h xor b) * 1099511628211 mod 2^64.
"""
from __future__ import annotations

import struct

import numpy as np

from . import base3_format as b3
from . import packed_format as pf

MAGIC = 0x42475750
VERSION = 1
T2, T2_TILED, B3, B3_TILED = 1, 2, 3, 4
FNV_OFFSET = 14695981039346656037
FNV_PRIME = 1099511628211
_FMT = "<IHHqqQQQ16s"


def fnv1a64(data: bytes) -> int:
    h = FNV_OFFSET
    for b in data:
        h = ((h ^ b) * FNV_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def payload_bytes(layout: int, rows: int, cols: int) -> int:
    if layout == T2:
        return pf.packed_nbytes(rows, cols)
    if layout == T2_TILED:
        return pf.tiled_nbytes(rows, cols // 4)
    if layout == B3:
        return b3.packed_nbytes(rows, cols)
    if layout == B3_TILED:
        return b3.tiled_nbytes(rows, cols)
    raise ValueError("unknown layout")


def make(layout: int, w: np.ndarray) -> bytes:
    """The 64-byte header of the logical matrix w in the given layout."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    rows, cols = w.shape
    head = struct.pack("<IHHqqQQ", MAGIC, VERSION, layout, rows, cols, payload_bytes(layout, rows, cols),
                       fnv1a64(w.tobytes()))
    return head + struct.pack("<Q", fnv1a64(head)) + bytes(16)


def parse(header: bytes) -> dict:
    magic, version, layout, rows, cols, nbytes, logical, hsum, reserved = struct.unpack(_FMT, header)
    return {"magic": magic, "version": version, "layout": layout, "rows": rows, "cols": cols,
            "payload_bytes": nbytes, "logical_fnv1a": logical, "header_fnv1a": hsum, "reserved": reserved}


def decode_payload(layout: int, payload: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """The logical matrix a payload holds (each layout through the oracle's
    own decoder of that format)."""
    p = np.ascontiguousarray(payload, dtype=np.uint8).reshape(-1)
    if layout == T2:
        return pf.decode(p, rows, cols)
    if layout == T2_TILED:
        return pf.decode(pf.untile16x64(p, rows, cols // 4).reshape(-1), rows, cols)
    if layout == B3:
        return b3.decode(p, rows, cols)
    if layout == B3_TILED:
        return b3.decode_tiled(p, rows, cols)
    raise ValueError("unknown layout")
