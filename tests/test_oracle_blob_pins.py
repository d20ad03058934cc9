"""Pins of the oracle's packed-blob header: FNV-1a 64 against the published
test vectors of its authors, the 64-byte field layout, and a checksum that
depends on the logical values only (the 2-bit and base-3 packings of one
matrix carry the same one)."""
import numpy as np

from oracle import base3_format as b3
from oracle import blob_header as bh
from oracle import packed_format as pf


def test_fnv1a64_published_vectors():
    assert bh.fnv1a64(b"") == 0xCBF29CE484222325
    assert bh.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert bh.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_header_fields_and_checksum():
    w = np.array([[1, -1, 0] * 22 + [1, 0]], np.int8)   # 1 x 68
    head = bh.make(bh.B3, w)
    assert len(head) == 64
    f = bh.parse(head)
    assert (f["magic"], f["version"], f["layout"], f["rows"], f["cols"]) == (0x42475750, 1, 3, 1, 68)
    assert head[:4] == b"PWGB"
    assert f["payload_bytes"] == 14                     # ceil(68 / 5)
    assert f["logical_fnv1a"] == bh.fnv1a64(w.astype(np.int8).tobytes())
    assert f["header_fnv1a"] == bh.fnv1a64(head[:40])
    assert f["reserved"] == bytes(16)


def test_checksum_is_the_same_for_every_packing_and_decodes_back():
    rng = np.random.default_rng(3)
    w = rng.integers(-1, 2, size=(20, 256)).astype(np.int8)
    sums = {bh.parse(bh.make(layout, w))["logical_fnv1a"] for layout in (bh.T2, bh.T2_TILED, bh.B3, bh.B3_TILED)}
    assert len(sums) == 1
    payloads = {bh.T2: pf.encode(w), bh.T2_TILED: pf.tile16x64(pf.encode(w).reshape(20, 64)),
                bh.B3: b3.encode(w), bh.B3_TILED: b3.tile(b3.encode(w), 20, 256)}
    for layout, p in payloads.items():
        assert p.size == bh.payload_bytes(layout, 20, 256)
        assert np.array_equal(bh.decode_payload(layout, p, 20, 256), w)
    w2 = w.copy()
    w2[7, 100] = -w2[7, 100] if w2[7, 100] else 1
    assert bh.parse(bh.make(bh.T2, w2))["logical_fnv1a"] != sums.pop()
