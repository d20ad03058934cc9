"""GPU parity of the base-3 path (five weights per byte) against the oracle,
through the C ABI: the device arrangement bit for bit against the oracle's
tile(), and the GEMV on it against the float64 GEMV of the logical matrix.

Inputs come from synth/; expected values from oracle/ only.  Criteria:
tests/parity.py."""
import numpy as np
import pytest

import synth
from oracle import base3_format as b3
from oracle import reference as ref
from tests.parity import assert_gemv
from tests.test_gpu_kernels import ACT_KINDS, activation_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import packed_weight_gemv_amd as pwg  # noqa: E402

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def b3_on_gpu(w):
    rows, cols = w.shape
    blob = dev(pwg.pack_weights_b3(w))
    return pwg.tile_b3(blob, rows, cols)


def run_b3(w, s, x):
    rows, cols = w.shape
    y = pwg.ternary_gemv_b3(b3_on_gpu(w), dev(s), rows, cols, dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy()


TILE_SHAPES = [(1, 1), (3, 7), (16, 240), (17, 60), (33, 1001), (40, 4096), (5, 12288), (19, 16384)]


@pytest.mark.parametrize("shape", TILE_SHAPES, ids=[f"{r}x{c}" for r, c in TILE_SHAPES])
def test_b3_tiling_matches_oracle_bit_for_bit(shape):
    rows, cols = shape
    w = synth.ternary(synth.rng_for(120, rows, cols), rows, cols)
    blob = pwg.pack_weights_b3(w)
    t = pwg.tile_b3(dev(blob), rows, cols)
    torch.cuda.synchronize()
    want = b3.tile(blob, rows, cols)
    assert pwg.b3_tiled_size(rows, cols) == want.size
    assert np.array_equal(t.cpu().numpy()[:want.size], want)


def test_b3_single_gemv_1024_seed0():
    w, s, x = synth.single_gemv()
    y = run_b3(w, s, x)
    assert_gemv(y, ref.ternary_gemv(w, s, x), ref.ternary_gemv_magnitude(w, s, x), "1024x1024")


SHAPES = [(1, 1), (1, 5), (3, 29), (2, 30), (5, 31), (7, 239), (9, 240), (11, 241), (37, 1001), (64, 2048),
          (1000, 4096), (257, 4100), (65, 12288), (33, 16384), (6144, 4096), (4096, 12288), (24576, 4096)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
def test_b3_gemv_shapes(shape):
    """Ragged widths (not a multiple of 5, 30 or 240), ragged row blocks, the
    layer's level shapes."""
    rows, cols = shape
    m = synth.ternary_matrix((121, rows, cols), rows, cols)
    x = synth.normal_f32(synth.rng_for(122, rows, cols), cols)
    y = run_b3(m.w, m.scale, x)
    assert_gemv(y, ref.ternary_gemv(m.w, m.scale, x), ref.ternary_gemv_magnitude(m.w, m.scale, x), str(shape))


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("kind", ACT_KINDS)
def test_b3_activation_ranges(kind, seed):
    rows, cols = 513, 4096
    m = synth.ternary_matrix((123, 0), rows, cols)
    x = activation_case(kind, cols, seed)
    y = run_b3(m.w, m.scale, x)
    assert_gemv(y, ref.ternary_gemv(m.w, m.scale, x), ref.ternary_gemv_magnitude(m.w, m.scale, x), f"{kind} {seed}")


def test_b3_zero_input_and_extreme_weights():
    cols = 4096
    m = synth.ternary_matrix((124, 0), 300, cols)
    assert not run_b3(m.w, m.scale, np.zeros(cols, np.float32)).any()
    w = np.stack([np.ones(cols, np.int8), -np.ones(cols, np.int8), np.zeros(cols, np.int8),
                  np.tile(np.array([1, -1], np.int8), cols // 2)])
    s = np.array([0.5, 0.25, 1.0, 0.125], np.float32)
    x = synth.normal_f32(synth.rng_for(125, 0), cols)
    y = run_b3(w, s, x)
    assert y[2] == 0.0
    assert_gemv(y, ref.ternary_gemv(w, s, x), ref.ternary_gemv_magnitude(w, s, x), "extreme")


def test_b3_negated_weights_negate_the_output_exactly():
    rows, cols = 777, 4096
    m = synth.ternary_matrix((126, 0), rows, cols)
    x = synth.normal_f32(synth.rng_for(126, 1), cols)
    assert np.array_equal(run_b3(-m.w, m.scale, x), -run_b3(m.w, m.scale, x))


@pytest.mark.parametrize("batch", [4, 16])
def test_b3_batch(batch):
    rows, cols = 1536, 4096
    m = synth.ternary_matrix((127, batch), rows, cols)
    xb = synth.batch_inputs(batch, cols, 0)
    y = run_b3(m.w, m.scale, xb)
    assert y.shape == (batch, rows)
    yr = ref.ternary_gemv(m.w, m.scale, xb)
    for b in range(batch):
        assert_gemv(y[b], yr[b], ref.ternary_gemv_magnitude(m.w, m.scale, xb[b]), f"batch row {b}")


def test_b3_is_deterministic_and_matches_a_sample_of_a_large_matrix():
    """393,216 x 4,096 (the q/k/v/o/gate/up rows of nine layers, 345 MB in
    the device arrangement): repeated calls are identical, and sampled rows
    match the oracle."""
    rows, cols = 393216, 4096
    rng = synth.rng_for(128, 0)
    w = synth.ternary(rng, rows, cols)
    s = synth.uniform_f32(rng, rows, 0.01, 0.1)
    x = synth.normal_f32(rng, cols)
    wt, sd, xd = b3_on_gpu(w), dev(s), dev(x)
    outs = [pwg.ternary_gemv_b3(wt, sd, rows, cols, xd).cpu().numpy() for _ in range(2)]
    assert np.array_equal(outs[0], outs[1])
    pick = np.sort(synth.rng_for(128, 1).choice(rows, 2048, replace=False))
    pick = np.concatenate([pick, [0, 15, 16, rows - 1]])
    ws, ss = w[pick], s[pick]
    assert_gemv(outs[0][pick], ref.ternary_gemv(ws, ss, x), ref.ternary_gemv_magnitude(ws, ss, x), "sampled rows")
