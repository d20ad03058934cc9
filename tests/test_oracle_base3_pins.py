"""Pins of the oracle's base-3 format (five ternary weights per byte) against
facts that do not come from the oracle: hand-derived bytes and tile offsets,
the exhaustive list of the 243 five-digit words, round trips, the padding
rule, an independent lane-by-lane reader of the device arrangement, and the
per-layer byte counts from the layer shapes."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import accounting as acc
from oracle import base3_format as b3
from oracle import reference as ref

RNG = np.random.default_rng(31)


def test_b3_hand_derived_bytes(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "b3_bytes.json")))
    for case in spec["cases"]:
        w = np.array(case["weights"], np.int8)
        blob = bytes.fromhex(case["bytes_hex"])
        assert b3.encode(w).tobytes() == blob, case["derivation"]
        assert np.array_equal(b3.decode(blob, *w.shape), w)


def test_b3_every_five_weight_word_has_its_own_code():
    """All 3^5 weight words, enumerated with the first weight varying
    fastest, get the codes 0..242 in order: the code is the base-3 number
    with the first weight as its least significant digit."""
    words = [tuple(reversed(t)) for t in itertools.product((-1, 0, 1), repeat=5)]
    w = np.array(words, np.int8)
    codes = b3.encode(w)
    assert codes.tolist() == list(range(243))
    assert np.array_equal(b3.decode(codes, 243, 5), w)


def test_b3_round_trip_padding_and_invalid_bytes():
    for rows, cols in ((1, 1), (3, 4), (5, 5), (7, 9), (16, 64), (17, 1024), (4, 4096), (2, 12288), (3, 1001)):
        w = RNG.integers(-1, 2, size=(rows, cols)).astype(np.int8)
        blob = b3.encode(w)
        assert blob.size == rows * -(-cols // 5) == b3.packed_nbytes(rows, cols)
        assert int(blob.max()) <= 242
        assert np.array_equal(b3.decode(blob, rows, cols), w)
        # the weights past the row end are zero: every digit above the last
        # weight of the last byte is 1
        tail = cols % 5
        if tail:
            last = blob.reshape(rows, -1)[:, -1].astype(np.int64)
            assert ((last // 3 ** tail) == sum(3 ** i for i in range(5 - tail))).all()
    bad = b3.encode(np.zeros((2, 10), np.int8)).copy()
    bad[3] = 243
    with pytest.raises(ValueError):
        b3.decode(bad, 2, 10)
    with pytest.raises(ValueError):
        b3.encode(np.array([[2, 0]]))
    with pytest.raises(ValueError):
        b3.decode(bad[:-1], 2, 10)


def _fixture_blob(rows, cols):
    B = -(-cols // 5)
    r = np.arange(rows)[:, None]
    m = np.arange(B)[None, :]
    return ((7 * r + 3 * m) % 243).astype(np.uint8)


def test_b3_tile_hand_derived_offsets(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "b3_tile.json")))
    rows, cols = fx["matrix"]["rows"], fx["matrix"]["cols"]
    stored = _fixture_blob(rows, cols)
    t = b3.tile(stored.reshape(-1), rows, cols)
    assert t.size == fx["tiled_bytes"] == b3.tiled_nbytes(rows, cols)
    for case in fx["cases"]:
        assert t[case["offset"]] == stored[case["row"], case["byte"]], case["derivation"]
    for case in fx["padding_offsets"]:
        assert t[case["offset"]] == 121, case["derivation"]


def test_b3_tile_is_a_permutation_plus_zero_weight_padding():
    for rows, cols in ((1, 1), (16, 240), (17, 60), (33, 1024), (40, 4096), (5, 12288), (19, 1001)):
        w = RNG.integers(-1, 2, size=(rows, cols)).astype(np.int8)
        blob = b3.encode(w)
        t = b3.tile(blob, rows, cols)
        assert t.size == -(-rows // 16) * b3.window_count(cols) * 768
        # every stored byte appears once; everything else is the zero word
        # (counted through distinct marker values on a second, synthetic blob)
        marker = (np.arange(blob.size) % 242).astype(np.uint8)
        tm = b3.tile(marker, rows, cols)
        assert t.size - blob.size == int((tm == 121).sum()) - int((marker == 121).sum())
        # the independent lane reader recovers the matrix and finds only
        # zero weights in the padding
        assert np.array_equal(b3.decode_tiled(t, rows, cols), w)


def test_b3_tiled_lane_reader_catches_a_misplaced_group():
    rows, cols = 16, 240
    w = RNG.integers(-1, 2, size=(rows, cols)).astype(np.int8)
    t = b3.tile(b3.encode(w), rows, cols).copy()
    # swap the two groups of lane 5: the reader must see a different matrix
    lane = t[12 * 5: 12 * 6].copy()
    t[12 * 5: 12 * 5 + 6], t[12 * 5 + 6: 12 * 6] = lane[6:], lane[:6]
    assert not np.array_equal(b3.decode_tiled(t, rows, cols), w)


def test_b3_gemv_equals_the_2_bit_formats_gemv_on_the_same_weights():
    """The format carries the same logical matrix: the plain GEMV of the
    decoded weights equals the float64 definition computed from w."""
    rows, cols = 33, 1001
    w = RNG.integers(-1, 2, size=(rows, cols)).astype(np.int8)
    s = RNG.uniform(0.01, 0.1, rows)
    x = RNG.standard_normal(cols)
    wd = b3.decode(b3.encode(w), rows, cols)
    want = np.array([s[r] * sum(float(w[r, k]) * x[k] for k in range(cols)) for r in range(rows)])
    assert np.allclose(ref.ternary_gemv(wd, s, x), want, rtol=1e-12, atol=1e-12)


def test_b3_layer_bytes_from_the_layer_shapes():
    # q, k, v, o, gate, up: 4,096 columns -> 820 bytes a row; down: 12,288 -> 2,458
    rows_4096 = 4096 + 1024 + 1024 + 4096 + 12288 + 12288
    assert acc.b3_layer_bytes() == rows_4096 * 820 + 4096 * 2458 == 38_617_088
    assert acc.b3_layer_bytes() == sum(b3.packed_nbytes(r, c) for r, c in acc.LAYER_SHAPES.values())
    # device arrangement: 137 groups -> 18 windows of 48 bytes; 410 -> 52
    assert acc.b3_layer_bytes(device=True) == rows_4096 * 18 * 48 + 4096 * 52 * 48 == 40_304_640
    assert acc.b3_layer_bytes(device=True) == sum(
        b3.tiled_nbytes(r, c) for r, c in acc.LAYER_SHAPES.values())
    # against the pages' 72,351,744-byte slab (3 bits a weight) and the 2-bit format
    assert abs(acc.b3_layer_bytes() / acc.slab_bytes() - 0.5337) < 1e-4
    assert acc.b3_layer_bytes() < acc.slab_bytes(2) < acc.slab_bytes()
    # the step floor at 8 TB/s: 252.3 us stored, 259.9 us as arranged
    assert round(acc.b3_step_bytes()["total"] / 8e12 * 1e6, 1) == 252.3
    assert round(acc.b3_step_bytes(device=True)["total"] / 8e12 * 1e6, 1) == 259.9
