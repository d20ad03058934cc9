"""GPU parity of the batched pass (pwg_decode_step_weights with batch 4, 8 or
16 on tiled weights): every level's outputs and every vector's logits and
token against the oracle, bit-identical results to the per-call tiled entry
points, the gathered embedding rows, repeated passes and graph replay."""
import numpy as np
import pytest

import synth
from oracle import reference as ref
from tests.parity import assert_gemv, token_ok

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import packed_weight_gemv_amd as pwg  # noqa: E402

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


class BatchPass:
    """Host arrays (for the oracle) and the device description of one pass."""

    def __init__(self, shapes, vocab, hidden, batch, seed, with_logits=True, deq=True):
        self.shapes, self.vocab, self.hidden, self.batch = shapes, vocab, hidden, batch
        self.mats = [synth.ternary_matrix((130, seed, i), r, c) for i, (r, c) in enumerate(shapes)]
        self.tab = synth.int8_table((131, seed), vocab, hidden)
        self.emb = synth.int8_table((132, seed), vocab, hidden)
        self.w_dev = [pwg.tile_rows(dev(pwg.pack_weights(m.w)), m.w.shape[0], m.w.shape[1] // 4) for m in self.mats]
        self.q_dev = pwg.tile_rows(dev(self.tab.q.view(np.uint8)), vocab, hidden)
        levels = []
        for m, wd, (r, c) in zip(self.mats, self.w_dev, shapes):
            levels.append((wd, dev(m.scale), torch.empty((batch, c), dtype=torch.float32, device=DEV),
                           torch.empty((batch, r), dtype=torch.float32, device=DEV), r, c))
        self.desc = pwg.StepDesc(
            levels=levels, out_table=self.q_dev, out_scale=dev(self.tab.scale),
            h=torch.empty((batch, hidden), dtype=torch.float32, device=DEV),
            emb_table=dev(self.emb.q), emb_scale=dev(self.emb.scale),
            token_in=torch.empty(batch, dtype=torch.int32, device=DEV),
            token_out=torch.empty(batch, dtype=torch.int32, device=DEV),
            emb_row_out=torch.empty((batch, hidden), dtype=torch.int8, device=DEV),
            emb_scale_out=torch.empty(batch, dtype=torch.float32, device=DEV),
            emb_deq_out=torch.empty((batch, hidden), dtype=torch.float32, device=DEV) if deq else None,
            logits_out=torch.empty((batch, vocab), dtype=torch.float32, device=DEV) if with_logits else None,
            schedule=pwg.SCHEDULE_STREAM, weight_layout=pwg.LAYOUT_TILED, vocab=vocab, hidden=hidden, batch=batch)
        need = pwg.step_workspace_bytes(self.desc)
        assert need > 0
        self.desc.workspace = torch.zeros(need, dtype=torch.uint8, device=DEV)
        self.desc._c = None

    def set_inputs(self, j):
        """Fresh seeded inputs (copied into the same device buffers)."""
        self.xs = [synth.batch_inputs(self.batch, c, 1000 * j + i) for i, (_, c) in enumerate(self.shapes)]
        self.h = synth.batch_inputs(self.batch, self.hidden, 1000 * j + 999)
        self.ids = synth.rng_for(133, j).integers(0, self.vocab, self.batch).astype(np.int32)
        for lv, x in zip(self.desc.levels, self.xs):
            lv[2].copy_(torch.from_numpy(x))
        self.desc.h.copy_(torch.from_numpy(self.h))
        self.desc.token_in.copy_(torch.from_numpy(self.ids))
        torch.cuda.synchronize()

    def outputs(self):
        d = self.desc
        return {
            "levels": [lv[3].cpu().numpy() for lv in d.levels],
            "tokens": d.token_out.cpu().numpy(),
            "logits": None if d.logits_out is None else d.logits_out.cpu().numpy(),
            "emb_row": d.emb_row_out.cpu().numpy(),
            "emb_scale": d.emb_scale_out.cpu().numpy(),
            "emb_deq": None if d.emb_deq_out is None else d.emb_deq_out.cpu().numpy(),
        }

    def per_call(self):
        """The same products through pwg_ternary_gemv_tiled and
        pwg_int8_gemv_argmax_tiled."""
        ys = [pwg.ternary_gemv_tiled(wd, lv[1], r, c, lv[2]).cpu().numpy()
              for wd, lv, (r, c) in zip(self.w_dev, self.desc.levels, self.shapes)]
        lo = torch.empty((self.batch, self.vocab), dtype=torch.float32, device=DEV)
        tok = pwg.int8_gemv_argmax_tiled(self.q_dev, self.desc.out_scale, self.vocab, self.hidden, self.desc.h,
                                         logits_out=lo)
        torch.cuda.synchronize()
        return ys, tok.cpu().numpy(), lo.cpu().numpy()

    def check(self, out, rows_sample=None):
        """Oracle parity of every vector (all rows, or the sampled rows of
        each level), logits, tokens and embedding rows."""
        for i, (m, x, y) in enumerate(zip(self.mats, self.xs, out["levels"])):
            rows = np.arange(m.w.shape[0]) if rows_sample is None else rows_sample(m.w.shape[0], i)
            yr = ref.ternary_gemv(m.w[rows], m.scale[rows], x)
            for b in range(self.batch):
                assert_gemv(y[b][rows], yr[b], ref.ternary_gemv_magnitude(m.w[rows], m.scale[rows], x[b]),
                            f"level {i} vector {b}")
        lr = ref.int8_logits(self.tab.q, self.tab.scale, self.h)
        vrows = np.arange(self.vocab) if rows_sample is None else rows_sample(self.vocab, -1)
        q, t = self.tab.q[vrows], self.tab.scale[vrows]
        for b in range(self.batch):
            assert token_ok(out["tokens"][b], lr[b]), f"vector {b}"
            if out["logits"] is not None:
                assert_gemv(out["logits"][b][vrows], lr[b][vrows], ref.int8_logits_magnitude(q, t, self.h[b]),
                            f"logits vector {b}")
        er, es, ed = ref.embed_gather(self.emb.q, self.emb.scale, self.ids)
        assert np.array_equal(out["emb_row"], er)
        assert np.array_equal(out["emb_scale"], es)
        if out["emb_deq"] is not None:
            assert np.array_equal(out["emb_deq"], ed)


def run(p, stream=None):
    pwg.decode_step_weights(p.desc, stream=stream)
    torch.cuda.synchronize()
    pwg.step_status(p.desc)
    return p.outputs()


def same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


SMALL = [(300, 2048), (1000, 4096), (64, 6144), (2000, 2048), (17, 12288)]


@pytest.mark.parametrize("batch", [4, 8, 16])
def test_small_pass_matches_oracle_and_per_call(batch):
    """Ragged row tails, levels with fewer row blocks than an item, widths
    2,048 .. 12,288; two passes in a row with new inputs (the claim and
    arrival counters start from zero again)."""
    p = BatchPass(SMALL, vocab=5003, hidden=1024, batch=batch, seed=batch)
    pwg.step_plan(p.desc)
    for j in range(2):
        p.set_inputs(10 * batch + j)
        out = run(p)
        p.check(out)
        ys, tok, lo = p.per_call()
        for i, (a, b) in enumerate(zip(out["levels"], ys)):
            assert same_bits(a, b), f"level {i}"
        assert np.array_equal(out["tokens"], tok)
        assert same_bits(out["logits"], lo)


def test_8b_layer_and_vocab_batch16():
    """One 8B-shape layer (q|k|v, o, gate|up, down) and the 151,936 x 4,096
    output table at 16 vectors, the configuration the pass is timed on:
    sampled rows of every level and every vector's token and logits against
    the oracle; every output bit-identical to the per-call entry points."""
    shapes = [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]
    p = BatchPass(shapes, vocab=151936, hidden=4096, batch=16, seed=99)
    pwg.step_plan(p.desc)
    p.set_inputs(7)
    out = run(p)
    ys, tok, lo = p.per_call()
    for i, (a, b) in enumerate(zip(out["levels"], ys)):
        assert same_bits(a, b), f"level {i}"
    assert np.array_equal(out["tokens"], tok)
    assert same_bits(out["logits"], lo)

    def sample(n, i):
        return np.unique(np.concatenate([[0, n - 1], synth.rng_for(134, i + 1).integers(0, n, 200)]))

    p.check(out, rows_sample=sample)


def test_graph_replay_matches_eager():
    p = BatchPass(SMALL[:3], vocab=2000, hidden=2048, batch=8, seed=5)
    pwg.step_plan(p.desc)
    p.set_inputs(3)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        pwg.decode_step_weights(p.desc, stream=s)
        s.synchronize()
        eager = p.outputs()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            pwg.decode_step_weights(p.desc, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        for lv in p.desc.levels:  # eager work between replays: clobber the outputs
            lv[3].fill_(float("nan"))
        p.desc.logits_out.fill_(float("nan"))
        p.desc.emb_deq_out.fill_(float("nan"))
        p.desc.token_out.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = p.outputs()
        for a, b in zip(got["levels"], eager["levels"]):
            assert same_bits(a, b), f"replay {rep}"
        assert same_bits(got["logits"], eager["logits"])
        assert np.array_equal(got["tokens"], eager["tokens"])
        assert np.array_equal(got["emb_deq"], eager["emb_deq"])
    pwg.step_status(p.desc)
    p.check(got)


def test_no_logits_no_deq_and_token_aliasing():
    """logits_out and emb_deq_out may be null; token_in and token_out may be
    the same buffer (the pass reads every id before it writes a token)."""
    p = BatchPass(SMALL[:2], vocab=3001, hidden=1024, batch=4, seed=6, with_logits=False, deq=False)
    p.desc.token_out = p.desc.token_in
    p.desc._c = None
    pwg.step_plan(p.desc)
    p.set_inputs(4)
    out = run(p)
    p.check(out)


@pytest.mark.parametrize("kind", ["zero", "onehot", "ranges", "outliers"])
def test_vector_ranges(kind):
    """A zero vector gives exact zeros, a one-hot vector gives s * W[:, k]
    exactly, vectors 2^-48 .. 2^36 apart in size stay within the bound, and
    vectors with massive outliers inside them (+-3e3 and +-1e4 at several
    places, and outliers among values near 1e-3) meet the same criteria, for
    the ternary levels and for h."""
    p = BatchPass([(500, 4096), (100, 2048)], vocab=1500, hidden=1024, batch=8, seed=7)
    pwg.step_plan(p.desc)
    p.set_inputs(5)
    xs = [x.astype(np.float64) for x in p.xs]
    if kind == "zero":
        for x in xs:
            x[3] = 0.0
    elif kind == "onehot":
        for x in xs:
            x[2] = 0.0
            x[2, 333] = 1.0
    elif kind == "ranges":
        for x in xs:
            for b in range(8):
                x[b] *= 2.0 ** (12 * (b - 4))
    else:
        for i, x in enumerate(xs):
            for b in range(8):
                x[b] = synth.outlier_vector(x.shape[1], 100 * i + b)
        p.h = np.stack([synth.outlier_vector(p.hidden, 900 + b) for b in range(8)])
        p.desc.h.copy_(torch.from_numpy(p.h))
    p.xs = [x.astype(np.float32) for x in xs]
    for lv, x in zip(p.desc.levels, p.xs):
        lv[2].copy_(torch.from_numpy(x))
    torch.cuda.synchronize()
    out = run(p)
    if kind == "zero":
        for y in out["levels"]:
            assert not y[3].any()
    if kind == "onehot":
        for m, y in zip(p.mats, out["levels"]):
            assert np.array_equal(y[2], (m.scale * m.w[:, 333]).astype(np.float32))
    p.check(out)


EDGE = [
    ([], 4000, 1024, 8),                      # the output table only; hidden of one operand slice
    ([(1, 2048)], 1, 1024, 16),               # one row everywhere (row blocks padded to 16)
    ([(33, 16384), (16, 2048)], 777, 8192, 4),  # wide K for both kinds
]


@pytest.mark.parametrize("case", EDGE, ids=["vocab-only", "one-row", "wide-k"])
def test_edge_shapes(case):
    shapes, vocab, hidden, batch = case
    p = BatchPass(shapes, vocab=vocab, hidden=hidden, batch=batch, seed=8)
    pwg.step_plan(p.desc)
    for j in range(2):
        p.set_inputs(60 + j)
        out = run(p)
        p.check(out)
        if hidden <= 8192:
            ys, tok, lo = p.per_call()
            for i, (a, b) in enumerate(zip(out["levels"], ys)):
                assert same_bits(a, b), f"level {i}"
            assert np.array_equal(out["tokens"], tok)
            assert same_bits(out["logits"], lo)
