"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Every input comes from the seeded generators in synth/; expected values come
from oracle/ only.  Criteria: tests/parity.py."""
import numpy as np
import pytest

import synth
from oracle import reference as ref
from tests.parity import assert_gemv, token_ok

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import packed_weight_gemv_amd as pwg  # noqa: E402

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def packed_on_gpu(w):
    return dev(pwg.pack_weights(w))


def run_ternary(w, s, x):
    rows, cols = w.shape
    y = pwg.ternary_gemv(packed_on_gpu(w), dev(s), rows, cols, dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ------------------------------------------------------------------ ternary GEMV
def test_single_gemv_1024_seed0():
    w, s, x = synth.single_gemv()
    y = run_ternary(w, s, x)
    assert_gemv(y, ref.ternary_gemv(w, s, x), ref.ternary_gemv_magnitude(w, s, x), "1024x1024")


SHAPES = [(1, 64), (3, 128), (5, 192), (7, 320), (2, 448), (37, 1024), (64, 2048), (1000, 4096),
          (257, 4160), (65, 12288), (33, 16384), (1, 8192), (6144, 4096), (4096, 12288), (24576, 4096)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
def test_ternary_shapes(shape):
    rows, cols = shape
    m = synth.ternary_matrix((90, rows, cols), rows, cols)
    x = synth.normal_f32(synth.rng_for(91, rows, cols), cols)
    y = run_ternary(m.w, m.scale, x)
    assert_gemv(y, ref.ternary_gemv(m.w, m.scale, x), ref.ternary_gemv_magnitude(m.w, m.scale, x), str(shape))


def test_ternary_zero_input_gives_exact_zero():
    m = synth.ternary_matrix((92, 0), 300, 4096)
    y = run_ternary(m.w, m.scale, np.zeros(4096, np.float32))
    assert not y.any()


def activation_case(kind, cols, seed):
    """Activation vectors that stress a rounding of x relative to a block
    maximum: massive outliers on an N(0, 1) or a 1e-3 background (with
    outliers among values near 1e-3), one outlier, tiny and huge vectors, a
    different magnitude in every 64-element stretch."""
    if kind == "outliers":
        return synth.outlier_vector(cols, seed)
    if kind == "outliers_small":
        return synth.outlier_vector(cols, seed, background="small")
    x = synth.normal_f32(synth.rng_for(94, seed), cols).astype(np.float64)
    if kind == "outlier":
        x[min(1234, cols - 1)] = 3000.0
    elif kind == "tiny":
        x *= 1e-30
    elif kind == "huge":
        x *= 1e30
    elif kind == "mixed_scales":
        x *= 10.0 ** np.repeat(np.arange(-8, 8), -(-cols // 16))[:cols]
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


ACT_KINDS = ["outlier", "outliers", "outliers_small", "tiny", "huge", "mixed_scales"]


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("kind", ACT_KINDS)
def test_ternary_activation_ranges(kind, seed):
    rows, cols = 513, 4096
    m = synth.ternary_matrix((93, 0), rows, cols)
    x = activation_case(kind, cols, seed)
    y = run_ternary(m.w, m.scale, x)
    assert_gemv(y, ref.ternary_gemv(m.w, m.scale, x), ref.ternary_gemv_magnitude(m.w, m.scale, x), f"{kind} {seed}")


@pytest.mark.parametrize("shape", [(24576, 4096), (4096, 12288), (1000, 16384)], ids=["gate_up", "down", "widest"])
def test_ternary_outliers_level_shapes(shape):
    rows, cols = shape
    m = synth.ternary_matrix((93, rows, cols), rows, cols)
    for bg in ("normal", "small"):
        x = synth.outlier_vector(cols, 5, background=bg)
        y = run_ternary(m.w, m.scale, x)
        assert_gemv(y, ref.ternary_gemv(m.w, m.scale, x), ref.ternary_gemv_magnitude(m.w, m.scale, x), f"{shape} {bg}")


def test_ternary_extreme_weights():
    cols = 4096
    w = np.stack([np.ones(cols, np.int8), -np.ones(cols, np.int8), np.zeros(cols, np.int8),
                  np.tile(np.array([1, -1], np.int8), cols // 2)])
    s = np.array([0.5, 0.25, 1.0, 0.125], np.float32)
    x = synth.normal_f32(synth.rng_for(95, 0), cols)
    y = run_ternary(w, s, x)
    assert y[2] == 0.0
    assert_gemv(y, ref.ternary_gemv(w, s, x), ref.ternary_gemv_magnitude(w, s, x), "extreme")


@pytest.mark.parametrize("batch", [4, 8, 16])
def test_ternary_batch(batch):
    rows, cols = 1536, 4096
    m = synth.ternary_matrix((96, batch), rows, cols)
    xb = synth.batch_inputs(batch, cols, 0)
    y = run_ternary(m.w, m.scale, xb)
    assert y.shape == (batch, rows)
    yr = ref.ternary_gemv(m.w, m.scale, xb)
    for b in range(batch):
        assert_gemv(y[b], yr[b], ref.ternary_gemv_magnitude(m.w, m.scale, xb[b]), f"batch row {b}")


BATCH_SHAPES = [(5, 64, 4), (1536, 4096, 16), (257, 8192, 8), (1000, 12288, 4), (33, 16384, 16), (4099, 4096, 8)]


@pytest.mark.parametrize("shape", BATCH_SHAPES, ids=[f"{r}x{c}xB{b}" for r, c, b in BATCH_SHAPES])
def test_ternary_batch_weights_read_once(shape):
    """Row-major batches (one matrix-core pass per vector): every width class,
    ragged row tails, widths that are not a multiple of 256."""
    rows, cols, batch = shape
    m = synth.ternary_matrix((103, rows, cols), rows, cols)
    xb = synth.batch_inputs(batch, cols, 3)
    y = run_ternary(m.w, m.scale, xb)
    yr = ref.ternary_gemv(m.w, m.scale, xb)
    for b in range(batch):
        assert_gemv(y[b], yr[b], ref.ternary_gemv_magnitude(m.w, m.scale, xb[b]), f"{shape} vector {b}")


def test_ternary_is_deterministic():
    m = synth.ternary_matrix((97, 0), 24576, 4096)
    x = synth.normal_f32(synth.rng_for(97, 1), 4096)
    wp, sp, xp = packed_on_gpu(m.w), dev(m.scale), dev(x)
    outs = [pwg.ternary_gemv(wp, sp, 24576, 4096, xp).cpu().numpy() for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


# ------------------------------------------------------------ int8 projection
def run_argmax(q, t, h, logits=True):
    qd, td, hd = dev(q), dev(t), dev(h)
    lo = torch.empty((h.shape[0], q.shape[0]) if h.ndim == 2 else q.shape[0], dtype=torch.float32, device=DEV) if logits else None
    tok = pwg.int8_gemv_argmax(qd, td, hd, logits_out=lo)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), (lo.cpu().numpy() if logits else None)


I8_SHAPES = [(1, 64), (100, 128), (999, 1024), (5000, 4096), (3, 8192)]


@pytest.mark.parametrize("shape", I8_SHAPES, ids=[f"{r}x{c}" for r, c in I8_SHAPES])
def test_int8_argmax_shapes(shape):
    rows, cols = shape
    tab = synth.int8_table((98, rows, cols), rows, cols)
    h = synth.normal_f32(synth.rng_for(99, rows), cols)
    tok, lg = run_argmax(tab.q, tab.scale, h)
    lr = ref.int8_logits(tab.q, tab.scale, h)
    assert_gemv(lg, lr, ref.int8_logits_magnitude(tab.q, tab.scale, h), str(shape))
    assert token_ok(tok[0], lr)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("kind", ACT_KINDS)
def test_int8_activation_ranges(kind, seed):
    rows, cols = 3000, 4096
    tab = synth.int8_table((99, 7), rows, cols)
    h = activation_case(kind, cols, seed)
    tok, lg = run_argmax(tab.q, tab.scale, h)
    lr = ref.int8_logits(tab.q, tab.scale, h)
    assert_gemv(lg, lr, ref.int8_logits_magnitude(tab.q, tab.scale, h), f"{kind} {seed}")
    assert token_ok(tok[0], lr)


def test_vocab_projection_full_size_and_gather():
    """151,936 x 4,096 int8 output table + argmax, and 64 embedding rows."""
    out_t, emb_t, ids, h = synth.vocab_workload()
    tok, lg = run_argmax(out_t.q, out_t.scale, h)
    lr = ref.int8_logits(out_t.q, out_t.scale, h)
    assert_gemv(lg, lr, ref.int8_logits_magnitude(out_t.q, out_t.scale, h), "vocab")
    assert token_ok(tok[0], lr)
    rows, scales, deq = pwg.embed_gather(dev(emb_t.q), dev(emb_t.scale), dev(ids))
    torch.cuda.synchronize()
    er, es, ed = ref.embed_gather(emb_t.q, emb_t.scale, ids)
    assert np.array_equal(rows.cpu().numpy(), er)
    assert np.array_equal(scales.cpu().numpy(), es)
    assert np.array_equal(deq.cpu().numpy(), ed)


def test_argmax_ties_go_to_lowest_index():
    rows, cols = 20000, 4096
    tab = synth.int8_table((100, 0), rows, cols)
    h = synth.normal_f32(synth.rng_for(100, 1), cols)
    lr = ref.int8_logits(tab.q, tab.scale, h)
    top = int(np.argmax(lr))
    q = tab.q.copy()
    t = tab.scale.copy()
    for dup in (17, 9000, rows - 1):   # identical rows score identical logits
        q[dup] = q[top]
        t[dup] = t[top]
    tok, _ = run_argmax(q, t, h, logits=False)
    assert tok[0] == min(17, top)


def test_argmax_batch():
    rows, cols, batch = 30000, 4096, 4
    tab = synth.int8_table((101, 0), rows, cols)
    hb = synth.batch_inputs(batch, cols, 7)
    tok, lg = run_argmax(tab.q, tab.scale, hb)
    lr = ref.int8_logits(tab.q, tab.scale, hb)
    for b in range(batch):
        assert token_ok(tok[b], lr[b])
        assert_gemv(lg[b], lr[b], ref.int8_logits_magnitude(tab.q, tab.scale, hb[b]), f"batch {b}")


# cols a multiple of 1,024: matrix-core kernel; (777, 768, 4): the VALU kernel per vector
I8_BATCH_SHAPES = [(999, 1024, 8), (5000, 4096, 16), (257, 2048, 4), (3, 8192, 4), (70001, 4096, 8),
                   (1000, 1024, 16), (777, 768, 4)]


@pytest.mark.parametrize("shape", I8_BATCH_SHAPES, ids=[f"{r}x{c}xB{b}" for r, c, b in I8_BATCH_SHAPES])
def test_argmax_batch_shapes(shape):
    rows, cols, batch = shape
    tab = synth.int8_table((104, rows, cols), rows, cols)
    hb = synth.batch_inputs(batch, cols, 11)
    tok, lg = run_argmax(tab.q, tab.scale, hb)
    lr = ref.int8_logits(tab.q, tab.scale, hb)
    for b in range(batch):
        assert token_ok(tok[b], lr[b]), f"{shape} vector {b}"
        assert_gemv(lg[b], lr[b], ref.int8_logits_magnitude(tab.q, tab.scale, hb[b]), f"{shape} vector {b}")


def test_argmax_batch_vector_ranges():
    """Vectors of very different magnitudes in one batch (each section of
    each vector takes its own exponent) and a zero vector."""
    rows, cols, batch = 5000, 4096, 8
    tab = synth.int8_table((106, 0), rows, cols)
    hb = synth.batch_inputs(batch, cols, 13).astype(np.float64)
    for b in range(batch):
        hb[b] *= 2.0 ** (12 * (b - 4))
    hb[5] = 0.0
    hb = hb.astype(np.float32)
    tok, lg = run_argmax(tab.q, tab.scale, hb)
    lr = ref.int8_logits(tab.q, tab.scale, hb)
    for b in range(batch):
        if b == 5:
            assert not lg[b].any() and tok[b] == 0
            continue
        assert token_ok(tok[b], lr[b]), f"vector {b}"
        assert_gemv(lg[b], lr[b], ref.int8_logits_magnitude(tab.q, tab.scale, hb[b]), f"vector {b}")


def test_argmax_batch_ties_per_column():
    """Every column keeps the lowest index among equal maxima."""
    rows, cols, batch = 20000, 4096, 4
    tab = synth.int8_table((105, 0), rows, cols)
    hb = synth.batch_inputs(batch, cols, 12)
    q, t = tab.q.copy(), tab.scale.copy()
    lr = ref.int8_logits(q, t, hb)
    tops = [int(np.argmax(lr[b])) for b in range(batch)]
    for top in tops:            # duplicate each column's best row further down and further up
        for dup in (min(top + 5000, rows - 1), max(top - 7000, 0)):
            q[dup], t[dup] = q[top], t[top]
    lr2 = ref.int8_logits(q, t, hb)
    tok, _ = run_argmax(q, t, hb, logits=False)
    for b in range(batch):
        best = lr2[b].max()
        assert tok[b] == int(np.flatnonzero(lr2[b] == best)[0]), f"vector {b}"


def test_gather_invalid_ids_give_zero_rows_and_nan_scale():
    tab = synth.int8_table((102, 0), 500, 256)
    ids = np.array([3, -1, 500, 499], np.int32)
    rows, scales, deq = pwg.embed_gather(dev(tab.q), dev(tab.scale), dev(ids))
    torch.cuda.synchronize()
    r, s, d = rows.cpu().numpy(), scales.cpu().numpy(), deq.cpu().numpy()
    assert np.array_equal(r[0], tab.q[3]) and np.array_equal(r[3], tab.q[499])
    assert not r[1].any() and not r[2].any() and not d[1].any()
    assert np.isnan(s[1]) and np.isnan(s[2]) and s[0] == tab.scale[3]


# ------------------------------------------------------------------ tiled arrangement
from oracle import packed_format as pf  # noqa: E402

TILE_SHAPES = [(1, 64), (17, 128), (16, 1024), (37, 1024), (1000, 3072), (4096, 1024), (24576, 1024), (1003, 4096)]


@pytest.mark.parametrize("shape", TILE_SHAPES, ids=[f"{r}x{b}" for r, b in TILE_SHAPES])
def test_tile_rows_matches_oracle_bit_for_bit(shape):
    rows, row_bytes = shape
    m = np.random.default_rng(rows * 31 + row_bytes).integers(0, 256, size=shape, dtype=np.uint8)
    out = pwg.tile_rows(dev(m), rows, row_bytes)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[: pwg.tiled_size(rows, row_bytes)]
    assert np.array_equal(got, pf.tile16x64(m))


def test_tile_rows_full_vocabulary_table_sampled():
    """The 151,936 x 4,096 int8 output table: sampled tiles against the oracle
    arrangement of the rows they cover."""
    rows, cols = 151936, 4096
    tab = synth.int8_table((106, 0), rows, cols)
    out = pwg.tile_rows(dev(tab.q.view(np.uint8)), rows, cols)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    tiles_per_block = cols // 64
    for rb in np.unique(np.concatenate([[0, rows // 16 - 1], rng.integers(0, rows // 16, 24)])):
        block = tab.q.view(np.uint8)[16 * rb: 16 * rb + 16]
        want = pf.tile16x64(block)
        got = out[rb * 16 * cols: (rb + 1) * 16 * cols].cpu().numpy()
        assert got.size == tiles_per_block * 1024 and np.array_equal(got, want), f"row block {rb}"


# ------------------------------------------------------------------ batched passes on tiled weights
def tiled_t2(w):
    rows, cols = w.shape
    return pwg.tile_rows(packed_on_gpu(w), rows, cols // 4)


TILED_BATCH_SHAPES = [(6144, 4096, 4), (1000, 4096, 16), (4096, 12288, 8), (100, 2048, 16), (24576, 4096, 16),
                      (17, 16384, 4)]


@pytest.mark.parametrize("shape", TILED_BATCH_SHAPES, ids=[f"{r}x{c}xB{b}" for r, c, b in TILED_BATCH_SHAPES])
def test_ternary_batch_tiled(shape):
    """Matrix-core batched ternary GEMV: the 8B level shapes, ragged row
    tails, fewer row blocks than CUs, the widest rows."""
    rows, cols, batch = shape
    m = synth.ternary_matrix((107, rows, cols), rows, cols)
    xb = synth.batch_inputs(batch, cols, 14)
    y = pwg.ternary_gemv_tiled(tiled_t2(m.w), dev(m.scale), rows, cols, dev(xb))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    yr = ref.ternary_gemv(m.w, m.scale, xb)
    for b in range(batch):
        assert_gemv(y[b], yr[b], ref.ternary_gemv_magnitude(m.w, m.scale, xb[b]), f"{shape} vector {b}")


def test_ternary_batch_tiled_vector_ranges():
    """Vectors of very different magnitudes, a zero vector and a one-hot
    vector (y = s * W[:, k] exactly) in one batch."""
    rows, cols, batch = 2000, 4096, 8
    m = synth.ternary_matrix((108, 0), rows, cols)
    xb = synth.batch_inputs(batch, cols, 15).astype(np.float64)
    for b in range(batch):
        xb[b] *= 2.0 ** (12 * (b - 4))
    xb[5] = 0.0
    xb[6] = 0.0
    xb[6, 777] = 1.0
    xb = xb.astype(np.float32)
    y = pwg.ternary_gemv_tiled(tiled_t2(m.w), dev(m.scale), rows, cols, dev(xb)).cpu().numpy()
    yr = ref.ternary_gemv(m.w, m.scale, xb)
    assert not y[5].any()
    assert np.array_equal(y[6], (m.scale * m.w[:, 777]).astype(np.float32))
    for b in (0, 1, 2, 3, 4, 7):
        assert_gemv(y[b], yr[b], ref.ternary_gemv_magnitude(m.w, m.scale, xb[b]), f"vector {b}")


TILED1_SHAPES = [(1, 256), (37, 1024), (6144, 4096), (4096, 12288), (1000, 16384), (24576, 4096)]


@pytest.mark.parametrize("shape", TILED1_SHAPES, ids=[f"{r}x{c}" for r, c in TILED1_SHAPES])
def test_ternary_tiled_batch1_matches_oracle_and_row_major(shape):
    """Batch 1 on the tiled arrangement: the same kernel as the row-major
    blob (the same tile slices reach the same lanes), so the outputs are
    identical bit for bit; both meet the oracle criterion, outliers included."""
    rows, cols = shape
    m = synth.ternary_matrix((110, rows, cols), rows, cols)
    for x in (synth.normal_f32(synth.rng_for(111, rows), cols), synth.outlier_vector(cols, 3)):
        yt = pwg.ternary_gemv_tiled(tiled_t2(m.w), dev(m.scale), rows, cols, dev(x)).cpu().numpy()
        yr = run_ternary(m.w, m.scale, x)
        assert np.array_equal(yt.view(np.uint32), yr.view(np.uint32))
        assert_gemv(yt, ref.ternary_gemv(m.w, m.scale, x), ref.ternary_gemv_magnitude(m.w, m.scale, x), str(shape))


@pytest.mark.parametrize("batch", [4, 8, 16])
def test_ternary_batch_tiled_outliers(batch):
    """Massive outliers inside every vector (N(0, 1) background, outliers
    among values near 1e-3): the batched pass rounds each vector to 31 bits
    per 1,024-value block."""
    rows, cols = 3000, 4096
    m = synth.ternary_matrix((108, 1), rows, cols)
    xb = np.stack([synth.outlier_vector(cols, 20 + b) for b in range(batch)])
    y = pwg.ternary_gemv_tiled(tiled_t2(m.w), dev(m.scale), rows, cols, dev(xb)).cpu().numpy()
    yr = ref.ternary_gemv(m.w, m.scale, xb)
    for b in range(batch):
        assert_gemv(y[b], yr[b], ref.ternary_gemv_magnitude(m.w, m.scale, xb[b]), f"vector {b}")


@pytest.mark.parametrize("batch", [4, 16])
def test_argmax_batch_outliers(batch):
    rows, cols = 5000, 4096
    tab = synth.int8_table((106, 1), rows, cols)
    hb = np.stack([synth.outlier_vector(cols, 40 + b) for b in range(batch)])
    tok, lg = run_argmax(tab.q, tab.scale, hb)
    lr = ref.int8_logits(tab.q, tab.scale, hb)
    for b in range(batch):
        assert token_ok(tok[b], lr[b]), f"vector {b}"
        assert_gemv(lg[b], lr[b], ref.int8_logits_magnitude(tab.q, tab.scale, hb[b]), f"vector {b}")


TILED_I8_SHAPES = [(5000, 4096, 16), (999, 1024, 8), (70001, 4096, 4), (3, 8192, 16)]


@pytest.mark.parametrize("shape", TILED_I8_SHAPES, ids=[f"{r}x{c}xB{b}" for r, c, b in TILED_I8_SHAPES])
def test_argmax_batch_tiled(shape):
    """The tiled table gives the same tokens and logits, bit for bit, as the
    row-major table (same digits, same exact sums), and matches the oracle."""
    rows, cols, batch = shape
    tab = synth.int8_table((109, rows, cols), rows, cols)
    hb = synth.batch_inputs(batch, cols, 16)
    qt = pwg.tile_rows(dev(tab.q.view(np.uint8)), rows, cols)
    lo_t = torch.empty((batch, rows), dtype=torch.float32, device=DEV)
    tok_t = pwg.int8_gemv_argmax_tiled(qt, dev(tab.scale), rows, cols, dev(hb), logits_out=lo_t)
    tok_r, lg_r = run_argmax(tab.q, tab.scale, hb)
    torch.cuda.synchronize()
    tok_t, lg_t = tok_t.cpu().numpy(), lo_t.cpu().numpy()
    assert np.array_equal(tok_t, tok_r)
    assert np.array_equal(lg_t.view(np.uint32), lg_r.view(np.uint32))
    lr = ref.int8_logits(tab.q, tab.scale, hb)
    for b in range(batch):
        assert token_ok(tok_t[b], lr[b]), f"{shape} vector {b}"
        assert_gemv(lg_t[b], lr[b], ref.int8_logits_magnitude(tab.q, tab.scale, hb[b]), f"{shape} vector {b}")
