"""Pins of the CPU oracle against facts that do not come from the oracle:
closed forms, invariants, brute force on tiny inputs, planted answers and
hand-derived fixtures.  Each test is chosen so that a plausible slip in the
oracle (a dropped term, a flipped sign, a transposed operand, a wrong index,
a wrong tie rule) fails it."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import packed_format as pf
from oracle import reference as ref

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- ternary GEMV
def test_every_ternary_row_of_length_8_is_its_balanced_ternary_number():
    """With x_k = 3**k, sum_k w_k 3**k is the balanced-ternary number whose
    digits are the row; the 3**8 = 6561 rows map one-to-one onto the integers
    -3280..3280.  A misplaced, dropped or sign-flipped weight breaks this."""
    rows = np.array(list(itertools.product((-1, 0, 1), repeat=8)), dtype=np.int8)
    x = np.array([3.0 ** k for k in range(8)], dtype=np.float32)
    y = ref.ternary_gemv(rows, np.ones(len(rows), np.float32), x)
    expect = np.array([sum(int(d) * 3 ** k for k, d in enumerate(r)) for r in rows], dtype=np.float64)
    assert np.array_equal(y, expect)
    assert sorted(y.astype(np.int64).tolist()) == list(range(-3280, 3281))


def test_one_hot_input_reads_one_column_not_one_row():
    w = RNG.integers(-1, 2, size=(7, 192), dtype=np.int8)   # non-square: transposition fails
    s = RNG.uniform(0.01, 0.1, 7).astype(np.float32)
    for k in (0, 5, 191):
        x = np.zeros(192, np.float32)
        x[k] = 1.0
        assert np.array_equal(ref.ternary_gemv(w, s, x), s.astype(np.float64) * w[:, k])


def test_all_ones_matrix_gives_scaled_sum_and_zero_matrix_gives_zero():
    x = RNG.standard_normal(256).astype(np.float32)
    s = RNG.uniform(0.01, 0.1, 3).astype(np.float32)
    y1 = ref.ternary_gemv(np.ones((3, 256), np.int8), s, x)
    assert np.allclose(y1, s.astype(np.float64) * math.fsum(x.astype(np.float64)), rtol=1e-14, atol=0)
    assert not ref.ternary_gemv(np.zeros((3, 256), np.int8), s, x).any()


def test_negating_weights_negates_output_and_linearity_in_x_and_scale():
    w = RNG.integers(-1, 2, size=(9, 128), dtype=np.int8)
    s = RNG.uniform(0.01, 0.1, 9).astype(np.float32)
    x1 = RNG.standard_normal(128).astype(np.float32)
    x2 = RNG.standard_normal(128).astype(np.float32)
    y1, y2 = ref.ternary_gemv(w, s, x1), ref.ternary_gemv(w, s, x2)
    assert np.array_equal(ref.ternary_gemv(-w, s, x1), -y1)
    a, b = 0.5, -2.0   # powers of two: the float64 combination of the inputs is exact
    y12 = ref.ternary_gemv(w, s, a * x1.astype(np.float64) + b * x2.astype(np.float64))
    assert np.allclose(y12, a * y1 + b * y2, rtol=1e-13, atol=1e-13)
    assert np.allclose(ref.ternary_gemv(w, 2 * s, x1), 2 * y1, rtol=0, atol=0)


def test_joint_column_permutation_leaves_output_unchanged():
    w = RNG.integers(-1, 2, size=(5, 320), dtype=np.int8)
    s = RNG.uniform(0.01, 0.1, 5).astype(np.float32)
    x = RNG.standard_normal(320).astype(np.float32)
    p = RNG.permutation(320)
    assert np.allclose(ref.ternary_gemv(w[:, p], s, x[p]), ref.ternary_gemv(w, s, x), rtol=1e-13, atol=1e-13)


def test_brute_force_fsum_on_tiny_matrix_and_batch_rows():
    w = RNG.integers(-1, 2, size=(6, 64), dtype=np.int8)
    s = RNG.uniform(0.01, 0.1, 6).astype(np.float32)
    xb = RNG.standard_normal((3, 64)).astype(np.float32)
    y = ref.ternary_gemv(w, s, xb)
    assert y.shape == (3, 6)
    for b in range(3):
        for r in range(6):
            exact = float(s[r]) * math.fsum(int(w[r, k]) * float(xb[b, k]) for k in range(64))
            assert abs(y[b, r] - exact) <= 1e-15 * max(1.0, abs(exact)) + 1e-15


def test_magnitude_bounds_the_output_and_equals_it_for_same_signs():
    w = RNG.integers(-1, 2, size=(8, 128), dtype=np.int8)
    s = RNG.uniform(0.01, 0.1, 8).astype(np.float32)
    x = RNG.standard_normal(128).astype(np.float32)
    assert (np.abs(ref.ternary_gemv(w, s, x)) <= ref.ternary_gemv_magnitude(w, s, x) * (1 + 1e-14)).all()
    xp = np.abs(x)
    wp = np.abs(w)
    assert np.allclose(ref.ternary_gemv(wp, s, xp), ref.ternary_gemv_magnitude(wp, s, xp), rtol=1e-14)


def test_rejects_non_ternary_weights():
    with pytest.raises(ValueError):
        ref.ternary_gemv(np.full((1, 64), 2, np.int8), np.ones(1, np.float32), np.ones(64, np.float32))


# --------------------------------------------------------- int8 logits, argmax
def test_int8_products_are_exact_and_sum_matches_fsum():
    q = RNG.integers(-127, 128, size=(4, 96), dtype=np.int8)
    t = RNG.uniform(0.001, 0.01, 4).astype(np.float32)
    h = RNG.standard_normal(96).astype(np.float32)
    lg = ref.int8_logits(q, t, h)
    for v in range(4):
        exact = float(t[v]) * math.fsum(int(q[v, k]) * float(h[k]) for k in range(96))
        assert abs(lg[v] - exact) <= 1e-15 * abs(exact) + 1e-15


def test_int8_one_hot_reads_a_column():
    q = RNG.integers(-127, 128, size=(11, 64), dtype=np.int8)
    t = RNG.uniform(0.001, 0.01, 11).astype(np.float32)
    h = np.zeros(64, np.float32)
    h[17] = 1.0
    assert np.array_equal(ref.int8_logits(q, t, h), t.astype(np.float64) * q[:, 17])


def test_int8_magnitude_is_the_sum_of_absolute_terms():
    """The cancellation floor of the logits comparison:
    |t_v| * sum_k |Q_vk| * |h_k|, pinned against a scalar-loop fsum, against
    the logit itself where no term cancels, and at the int8 minimum -128
    (whose absolute value does not fit in int8)."""
    rng = np.random.default_rng(11)
    q = rng.integers(-128, 128, size=(7, 9), dtype=np.int8)
    q[0, 0] = -128
    t = rng.uniform(-0.01, 0.01, size=7).astype(np.float32)
    h = rng.standard_normal(9).astype(np.float32)
    mag = ref.int8_logits_magnitude(q, t, h)
    for v in range(7):
        want = abs(float(t[v])) * math.fsum(abs(int(q[v, k])) * abs(float(h[k])) for k in range(9))
        assert mag[v] == pytest.approx(want, rel=1e-15)
    assert (mag >= np.abs(ref.int8_logits(q, t, h)) * (1 - 1e-15)).all()
    # no cancellation: every term of a row has the same sign
    qp = np.abs(q.astype(np.int16)).clip(0, 127).astype(np.int8)
    hp = np.abs(h)
    assert np.allclose(ref.int8_logits_magnitude(qp, t, hp), np.abs(ref.int8_logits(qp, t, hp)), rtol=1e-15, atol=0)
    # a row whose terms cancel exactly: logit 0, magnitude the full sum
    qc = np.array([[1, -1, 2, -2]], np.int8)
    hc = np.array([3.0, 3.0, -0.5, -0.5], np.float32)
    assert ref.int8_logits(qc, np.ones(1, np.float32), hc)[0] == 0.0
    assert ref.int8_logits_magnitude(qc, np.ones(1, np.float32), hc)[0] == 8.0
    # -128 and a negative scale: 128 * |h| * |t|
    m1 = ref.int8_logits_magnitude(np.array([[-128]], np.int8), np.array([-0.5], np.float32), np.array([-2.0], np.float32))
    assert m1[0] == 128.0
    # invariant under negating h or the table
    assert np.array_equal(ref.int8_logits_magnitude(q, t, -h), mag)
    qn = (-q.astype(np.int16)).clip(-127, 127).astype(np.int8)
    qs = q.copy()
    qs[q == -128] = -127
    assert np.array_equal(ref.int8_logits_magnitude(qn, t, h), ref.int8_logits_magnitude(qs, t, h))


def test_planted_maximum_is_found():
    v, k = 1000, 64
    q = RNG.integers(-100, 101, size=(v, k), dtype=np.int8)
    t = RNG.uniform(0.001, 0.005, v).astype(np.float32)
    h = np.zeros(k, np.float32)
    h[3] = 1.0
    q[:, 3] = np.clip(q[:, 3], -100, 100)
    q[777, 3] = 127
    t[777] = 0.01
    token, gap = ref.greedy_token(ref.int8_logits(q, t, h))
    assert token == 777
    assert gap > 0


def test_ties_go_to_the_lowest_index_and_report_zero_gap():
    logits = np.array([0.5, 2.0, -1.0, 2.0, 2.0])
    assert ref.greedy_token(logits) == (1, 0.0)
    assert list(ref.accepted_tokens(logits, 0.0)) == [1, 3, 4]
    assert ref.greedy_token(np.array([3.0, 1.0, 2.5])) == (0, 0.5)


# ------------------------------------------------------------------ gather
def test_gather_returns_the_named_rows_and_power_of_two_dequant_is_exact():
    e = RNG.integers(-127, 128, size=(50, 64), dtype=np.int8)
    sc = (2.0 ** -RNG.integers(3, 10, 50)).astype(np.float32)
    ids = [49, 0, 7, 7]
    rows, scales, deq = ref.embed_gather(e, sc, ids)
    for i, tid in enumerate(ids):
        assert np.array_equal(rows[i], e[tid])
        assert scales[i] == sc[tid]
        # power-of-two scale: the product is exact, so it equals the real product
        assert all(float(deq[i, k]) == int(e[tid, k]) * float(sc[tid]) for k in range(64))
    with pytest.raises(IndexError):
        ref.embed_gather(e, sc, [50])


def test_gather_dequant_rounds_once_like_a_float32_product():
    e = np.array([[127, -127, 3, -1] * 16], dtype=np.int8)
    sc = np.array([0.0037], dtype=np.float32)
    _, _, deq = ref.embed_gather(e, sc, [0])
    # the float64 product of a float32 and a small int is exact; rounding it
    # once to float32 is the correctly rounded float32 product
    exact = e[0].astype(np.float64) * np.float64(sc[0])
    assert np.array_equal(deq[0], exact.astype(np.float32))


# ---------------------------------------------------------------- T2 format
def test_t2_hand_derived_bytes(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "t2_bytes.json")))
    for case in spec["cases"]:
        w = np.zeros((case["rows"], case["cols"]), np.int8)
        for k, v in case["nonzero"].items():
            w[0, int(k)] = v
        blob = bytes.fromhex(case["bytes_hex"])
        assert pf.encode(w).tobytes() == blob
        assert np.array_equal(pf.decode(blob, case["rows"], case["cols"]), w)


def test_t2_bit_positions_tile_the_word():
    assert sorted(pf.bit_position(m) for m in range(16)) == list(range(0, 32, 2))


def test_t2_round_trip_and_invalid_code():
    w = RNG.integers(-1, 2, size=(13, 192), dtype=np.int8)
    blob = pf.encode(w)
    assert blob.size == pf.packed_nbytes(13, 192) == 13 * 192 // 4
    assert np.array_equal(pf.decode(blob, 13, 192), w)
    bad = blob.copy()
    bad[5] = (bad[5] & 0xFC) | 0b10
    with pytest.raises(ValueError):
        pf.decode(bad, 13, 192)
    with pytest.raises(ValueError):
        pf.packed_nbytes(1, 100)


# ---------------------------------------------------------------- tile arrangement
def _fixture_matrix(rows, row_bytes):
    r, c = np.meshgrid(np.arange(rows), np.arange(row_bytes), indexing="ij")
    return ((r * 128 + c) % 251).astype(np.uint8)


def test_tile_hand_derived_offsets(golden_dir):
    import json
    fx = json.load(open(os.path.join(golden_dir, "tile16x64.json")))
    rows, rb = fx["matrix"]["rows"], fx["matrix"]["row_bytes"]
    m = _fixture_matrix(rows, rb)
    t = pf.tile16x64(m)
    assert t.size == fx["tiled_bytes"] == pf.tiled_nbytes(rows, rb)
    for case in fx["cases"]:
        assert t[case["offset"]] == m[case["row"], case["col"]], case["derivation"]
    for case in fx["zero_offsets"]:
        assert t[case["offset"]] == 0, case["derivation"]


def test_tile_is_a_permutation_plus_zero_padding_and_inverts():
    for rows, rb in ((1, 64), (16, 64), (17, 128), (40, 192), (33, 3072)):
        m = RNG.integers(0, 256, size=(rows, rb), dtype=np.uint8)
        t = pf.tile16x64(m)
        pad = t.size - m.size
        assert pad == (-(-rows // 16) * 16 - rows) * rb
        assert np.array_equal(np.sort(t), np.sort(np.concatenate([m.reshape(-1), np.zeros(pad, np.uint8)])))
        assert np.array_equal(pf.untile16x64(t, rows, rb), m)


def test_tile_one_kib_tile_holds_one_16_row_block_of_one_window():
    """Brute force on a matrix whose bytes name their own (row, column):
    every 1 KiB tile holds exactly the 16 x 64 bytes of one (row block,
    column window), and every 16-byte unit holds 16 consecutive bytes of one
    row."""
    rows, rb = 48, 256
    ids = np.arange(rows * rb, dtype=np.int64).reshape(rows, rb)
    lo, hi = (ids % 256).astype(np.uint8), (ids // 256).astype(np.uint8)
    tl, th = pf.tile16x64(lo), pf.tile16x64(hi)
    flat_id = th.astype(np.int64) * 256 + tl
    row, col = flat_id // rb, flat_id % rb
    for tile in range(flat_id.size // 1024):
        r, c = row[1024 * tile:1024 * (tile + 1)], col[1024 * tile:1024 * (tile + 1)]
        assert len(set((r // 16).tolist())) == 1 and len(set((c // 64).tolist())) == 1
        assert len(set(zip(r.tolist(), c.tolist()))) == 1024
    units_r, units_c = row.reshape(-1, 16), col.reshape(-1, 16)
    assert (units_r == units_r[:, :1]).all() and (np.diff(units_c, axis=1) == 1).all()


def test_tile_rejects_bad_shapes():
    for rows, rb in ((0, 64), (4, 32), (4, 100)):
        with pytest.raises(ValueError):
            pf.tiled_nbytes(rows, rb)


# ---------------------------------------------------------------- decode step
def test_decode_step_composes_the_parts():
    levels = []
    for _ in range(2):
        layer = []
        for r, k in ((24, 64), (8, 64), (40, 64), (8, 128)):
            layer.append((RNG.integers(-1, 2, size=(r, k), dtype=np.int8),
                          RNG.uniform(0.01, 0.1, r).astype(np.float32),
                          RNG.standard_normal(k).astype(np.float32)))
        levels.append(layer)
    q = RNG.integers(-127, 128, size=(100, 64), dtype=np.int8)
    t = RNG.uniform(0.001, 0.01, 100).astype(np.float32)
    h = RNG.standard_normal(64).astype(np.float32)
    e = RNG.integers(-127, 128, size=(100, 64), dtype=np.int8)
    es = RNG.uniform(0.001, 0.01, 100).astype(np.float32)
    out = ref.decode_step(levels, q, t, h, e, es, 42)
    assert out["token"] == int(np.argmax(out["logits"]))
    assert np.array_equal(out["emb_row"], e[42])
    assert np.array_equal(out["levels"][1][3], ref.ternary_gemv(*levels[1][3]))
