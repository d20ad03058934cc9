"""GPU parity of whole decode steps (every schedule) against the oracle,
including replay from a captured HIP graph."""
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
from packed_weight_gemv_amd.workload import build_step  # noqa: E402

SMALL = {"q": (256, 256), "k": (64, 256), "v": (64, 256), "o": (256, 256),
         "gate": (768, 256), "up": (768, 256), "down": (256, 768)}


def outputs(wl):
    d = wl.desc
    return {
        "levels": [lv[3].cpu().numpy() for lv in d.levels],
        "token": int(d.token_out.cpu()[0]),
        "emb_row": d.emb_row_out.cpu().numpy(),
        "emb_scale": float(d.emb_scale_out.cpu()[0]),
        "emb_deq": d.emb_deq_out.cpu().numpy(),
        "logits": None if d.logits_out is None else d.logits_out.cpu().numpy(),
    }


def check_against_oracle(wl, out, token_in, full_levels):
    """Sampled rows of every level (all rows when full_levels), the logits,
    the token and the gathered embedding row."""
    for smp, y in zip(wl.samples, out["levels"]):
        yr = ref.ternary_gemv(smp.w, smp.scale, smp.x)
        mag = ref.ternary_gemv_magnitude(smp.w, smp.scale, smp.x)
        assert_gemv(y[smp.rows], yr, mag, f"layer {smp.layer} {smp.level}")
    if full_levels:
        for layer in range(len(wl.level_shapes) // 4):
            mats = synth.layer(synth.W_STEP, layer, SMALL)
            xs = synth.layer_inputs(synth.W_STEP, layer, hidden=256, inter=768)
            for i, (name, members, _) in enumerate(synth.LEVELS):
                m = synth.stacked(mats, members)
                assert_gemv(out["levels"][4 * layer + i], ref.ternary_gemv(m.w, m.scale, xs[name]),
                            ref.ternary_gemv_magnitude(m.w, m.scale, xs[name]), f"full {layer} {name}")
    lr = ref.int8_logits(wl.out_table.q, wl.out_table.scale, wl.h)
    if out["logits"] is not None:
        assert_gemv(out["logits"], lr, ref.int8_logits_magnitude(wl.out_table.q, wl.out_table.scale, wl.h), "logits")
    assert token_ok(out["token"], lr)
    er, es, ed = ref.embed_gather(wl.emb_table.q, wl.emb_table.scale, [token_in])
    assert np.array_equal(out["emb_row"], er[0])
    assert out["emb_scale"] == es[0]
    assert np.array_equal(out["emb_deq"], ed[0])


SCHEDULES = [pwg.SCHEDULE_LEVELS, pwg.SCHEDULE_STREAM, pwg.SCHEDULE_PERSISTENT]
SCHED_IDS = ["levels", "stream", "persistent"]
ORDERED = [pwg.SCHEDULE_LEVELS, pwg.SCHEDULE_PERSISTENT]
ORDERED_IDS = ["levels", "persistent"]


@pytest.mark.parametrize("schedule", SCHEDULES, ids=SCHED_IDS)
def test_small_step_matches_oracle_everywhere(schedule):
    wl = build_step(n_layers=3, shapes=SMALL, vocab=1000, hidden=256, with_logits=True, schedule=schedule)
    pwg.step_plan(wl.desc)
    pwg.decode_step_weights(wl.desc)
    torch.cuda.synchronize()
    pwg.step_status(wl.desc)
    check_against_oracle(wl, outputs(wl), wl.token0, full_levels=True)


@pytest.mark.parametrize("schedule", SCHEDULES, ids=SCHED_IDS)
def test_8b_shape_two_layers_full_vocab_sampled(schedule):
    wl = build_step(n_layers=2, with_logits=True, schedule=schedule)
    assert [s[2:] for s in wl.level_shapes[:4]] == [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]
    pwg.step_plan(wl.desc)
    pwg.decode_step_weights(wl.desc)
    torch.cuda.synchronize()
    pwg.step_status(wl.desc)
    out = outputs(wl)
    check_against_oracle(wl, out, wl.token0, full_levels=False)
    # the next step gathers the row of the token this step produced
    pwg.decode_step_weights(wl.desc)
    torch.cuda.synchronize()
    pwg.step_status(wl.desc)
    check_against_oracle(wl, outputs(wl), out["token"], full_levels=False)


@pytest.mark.parametrize("schedule", SCHEDULES, ids=SCHED_IDS)
def test_graph_replay_matches_eager(schedule):
    wl = build_step(n_layers=2, shapes=SMALL, vocab=1000, hidden=256, with_logits=True, schedule=schedule)
    pwg.step_plan(wl.desc)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        # two eager steps: the second gathers the row of the first step's token,
        # as every later step does (h is fixed, so the token no longer changes)
        pwg.decode_step_weights(wl.desc, stream=s)
        pwg.decode_step_weights(wl.desc, stream=s)
        s.synchronize()
        eager = outputs(wl)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            pwg.decode_step_weights(wl.desc, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        for lv in wl.desc.levels:      # eager work between replays: clobber outputs
            lv[3].fill_(float("nan"))
        wl.desc.logits_out.fill_(float("nan"))
        wl.desc.emb_deq_out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs(wl)
        for a, b in zip(got["levels"], eager["levels"]):
            assert np.array_equal(a, b), f"replay {rep}"
        assert np.array_equal(got["logits"], eager["logits"])
        assert got["token"] == eager["token"]
        assert np.array_equal(got["emb_deq"], eager["emb_deq"])
    pwg.step_status(wl.desc)
    check_against_oracle(wl, got, eager["token"], full_levels=True)


def test_persistent_level_trace():
    """The persistent schedule's level trace: a traced step computes what an
    untraced one does, bit for bit, and each workgroup's stamps of a level
    come in event order, each level's start after the previous level's
    arrivals of every workgroup (the barrier), and every one is written."""
    wl = build_step(n_layers=2, shapes=SMALL, vocab=1000, hidden=256, with_logits=True,
                    schedule=pwg.SCHEDULE_PERSISTENT)
    pwg.step_plan(wl.desc)
    pwg.decode_step_weights(wl.desc)
    torch.cuda.synchronize()
    plain = outputs(wl)
    nbytes = pwg.step_trace_bytes(wl.desc)
    nl = len(wl.desc.levels)
    assert nbytes > 0 and nbytes % ((nl + 1) * pwg.TRACE_EVENTS * 8) == 0
    grid = nbytes // ((nl + 1) * pwg.TRACE_EVENTS * 8)
    trace = torch.zeros(nbytes // 8, dtype=torch.int64, device="cuda:0")
    pwg.step_set_trace(wl.desc, trace)
    wl.desc.token_in.fill_(int(wl.token0))
    pwg.decode_step_weights(wl.desc)
    torch.cuda.synchronize()
    pwg.step_status(wl.desc)
    traced = outputs(wl)
    for a, b in zip(traced["levels"], plain["levels"]):
        assert np.array_equal(a, b)
    assert np.array_equal(traced["logits"], plain["logits"]) and traced["token"] == plain["token"]
    t = trace.cpu().numpy().reshape(nl + 1, grid, pwg.TRACE_EVENTS)
    ev = {n: i for i, n in enumerate(pwg.TRACE_EVENT_NAMES)}
    order = ["wait", "passed", "sources", "start", "converted", "products", "arrived"]
    for li in range(nl):
        for a, b in zip(order, order[1:]):
            assert (t[li, :, ev[a]] <= t[li, :, ev[b]]).all(), (li, a, b)
        assert (t[li, :, ev["arrived"]] > 0).all()
        if li > 0:   # nobody starts a level before every workgroup arrived at the one before
            assert t[li, :, ev["passed"]].min() >= t[li - 1, :, ev["arrived"]].max(), li
    for a, b in zip(order[:5], order[1:6]):
        assert (t[nl, :, ev[a]] <= t[nl, :, ev[b]]).all(), ("projection", a, b)
    assert t[nl, :, ev["passed"]].min() >= t[nl - 1, :, ev["arrived"]].max()
    pwg.step_set_trace(wl.desc, None)


@pytest.mark.parametrize("schedule", [pwg.SCHEDULE_STREAM], ids=["stream"])
def test_many_steps_stay_identical(schedule):
    """Claim counters are reset by every step's last workgroup; 50
    back-to-back steps must all finish (no timeout) and give the same outputs
    as the first."""
    wl = build_step(n_layers=4, shapes=SMALL, vocab=1000, hidden=256, with_logits=True, schedule=schedule)
    pwg.step_plan(wl.desc)
    pwg.decode_step_weights(wl.desc)
    pwg.decode_step_weights(wl.desc)
    torch.cuda.synchronize()
    first = outputs(wl)
    for _ in range(50):
        pwg.decode_step_weights(wl.desc)
    torch.cuda.synchronize()
    pwg.step_status(wl.desc)
    last = outputs(wl)
    for a, b in zip(first["levels"], last["levels"]):
        assert np.array_equal(a, b)
    assert np.array_equal(first["logits"], last["logits"]) and first["token"] == last["token"]


def test_stream_launch_after_changed_description_is_refused():
    """The stream kernels read every pointer and shape from the device plan:
    after a level's input buffer is replaced, a launch without a new plan is
    refused (nothing is enqueued), and after planning again the step reads the
    new buffer."""
    wl = build_step(n_layers=1, shapes=SMALL, vocab=1000, hidden=256, with_logits=True, schedule=pwg.SCHEDULE_STREAM)
    d = wl.desc
    pwg.step_plan(d)
    pwg.decode_step_weights(d)
    torch.cuda.synchronize()
    lv = [list(t) for t in d.levels]
    x_new = synth.normal_f32(synth.rng_for(150, 0), lv[1][5])
    lv[1][2] = torch.from_numpy(x_new).to("cuda:0")
    d.levels = [tuple(t) for t in lv]
    d._c = None
    with pytest.raises(pwg.PwgError, match="planned"):
        pwg.decode_step_weights(d)
    pwg.step_plan(d)
    pwg.decode_step_weights(d)
    torch.cuda.synchronize()
    pwg.step_status(d)
    m = synth.stacked(synth.layer(synth.W_STEP, 0, SMALL), synth.LEVELS[1][1])
    assert_gemv(d.levels[1][3].cpu().numpy(), ref.ternary_gemv(m.w, m.scale, x_new),
                ref.ternary_gemv_magnitude(m.w, m.scale, x_new), "o after re-plan")


def chain_levels(wl):
    """Rewires a built step so that every level reads a prefix of the previous
    level's output and h is the last level's output: a chained step, in which
    each level depends on the one before it."""
    d = wl.desc
    lv = [list(t) for t in d.levels]
    for i in range(1, len(lv)):
        lv[i][2] = lv[i - 1][3][: lv[i][5]]
    d.levels = [tuple(t) for t in lv]
    d.h = lv[-1][3][: d.hidden]
    d._c = None
    return lv[0][2]


def chained_oracle(mats, x0, out_table):
    """Composes the oracle's GEMVs level by level over the stacked level
    matrices `mats`; each level output is rounded to float32, the type the
    step stores it in."""
    x = x0
    ys = []
    for m in mats:
        xin = x[: m.w.shape[1]]
        ys.append((m, xin, ref.ternary_gemv(m.w, m.scale, xin)))
        x = ys[-1][2].astype(np.float32)
    h = x[: out_table.q.shape[1]]
    return ys, h, ref.int8_logits(out_table.q, out_table.scale, h)


@pytest.mark.parametrize("size", ["small", "8b"])
@pytest.mark.parametrize("schedule", ORDERED, ids=ORDERED_IDS)
def test_chained_levels_see_previous_outputs(schedule, size):
    """The ordered schedules must honour level dependencies: level L+1 reads
    what level L wrote in the same step.  Two steps with different first
    inputs also rule out stale cached activations from the step before."""
    n_layers, shapes, vocab, hidden = (3, SMALL, 1000, 256) if size == "small" else (2, None, synth.VOCAB, synth.HIDDEN)
    wl = build_step(n_layers=n_layers, shapes=shapes, vocab=vocab, hidden=hidden, with_logits=True, schedule=schedule)
    x0 = chain_levels(wl)
    pwg.step_plan(wl.desc)
    x0_host = x0.cpu().numpy().copy()
    layers = [synth.layer(synth.W_STEP, layer, shapes) for layer in range(n_layers)]
    mats = [synth.stacked(lm, members) for lm in layers for _, members, _ in synth.LEVELS]
    del layers
    token_in = wl.token0
    for step, factor in enumerate((1.0, -0.5)):
        x0.copy_(torch.from_numpy(x0_host * np.float32(factor)))   # exact scaling
        print(f"chained step {step} schedule {schedule} size {size}", flush=True)
        pwg.decode_step_weights(wl.desc)
        torch.cuda.synchronize()
        pwg.step_status(wl.desc)
        out = outputs(wl)
        ys, h, lr = chained_oracle(mats, x0_host * np.float32(factor), wl.out_table)
        for i, ((m, xin, yr), y) in enumerate(zip(ys, out["levels"])):
            assert_gemv(y, yr, ref.ternary_gemv_magnitude(m.w, m.scale, xin), f"step {step} level {i}")
        assert_gemv(out["logits"], lr, ref.int8_logits_magnitude(wl.out_table.q, wl.out_table.scale, h), "logits")
        assert token_ok(out["token"], lr)
        er, _, _ = ref.embed_gather(wl.emb_table.q, wl.emb_table.scale, [token_in])
        assert np.array_equal(out["emb_row"], er[0])
        token_in = out["token"]


# ------------------------------------------------------------------ stream schedule edge cases
RAGGED = {"q": (4000, 4096), "k": (37, 4096), "v": (1, 4096), "o": (4096, 4096),
          "gate": (100, 4096), "up": (3000, 4096), "down": (1029, 12288)}


def test_stream_ragged_rows_prefetch_path():
    """Row counts that are not multiples of 16 (a one-row level included), a
    ragged vocabulary, on widths that take the prefetching kernel (tiles per
    block a multiple of 16)."""
    wl = build_step(n_layers=2, shapes=RAGGED, vocab=1000, hidden=4096, with_logits=True,
                    schedule=pwg.SCHEDULE_STREAM)
    pwg.step_plan(wl.desc)
    pwg.decode_step_weights(wl.desc)
    torch.cuda.synchronize()
    pwg.step_status(wl.desc)
    out = outputs(wl)
    for layer in range(2):
        mats = synth.layer(synth.W_STEP, layer, RAGGED)
        xs = synth.layer_inputs(synth.W_STEP, layer, hidden=4096, inter=12288)
        for i, (name, members, _) in enumerate(synth.LEVELS):
            m = synth.stacked(mats, members)
            assert_gemv(out["levels"][4 * layer + i], ref.ternary_gemv(m.w, m.scale, xs[name]),
                        ref.ternary_gemv_magnitude(m.w, m.scale, xs[name]), f"ragged {layer} {name}")
    check_against_oracle(wl, out, wl.token0, full_levels=False)


@pytest.mark.parametrize("kind", ["outlier", "outliers", "outliers_small", "tiny", "huge", "mixed", "zero"])
def test_stream_activation_ranges(kind):
    """The matrix-core operands carry one E8M0 scale per 32 inputs (ternary)
    or one exponent per 256 (h): one outlier, massive outliers on an N(0, 1)
    or a 1e-3 background (outliers among values near 1e-3 included), tiny and
    huge magnitudes, a different magnitude in every block, all-zero inputs;
    h takes the same kind of vector."""
    wl = build_step(n_layers=1, shapes=SMALL, vocab=1000, hidden=256, with_logits=True,
                    schedule=pwg.SCHEDULE_STREAM)
    d = wl.desc
    xs = {}
    for i, lv in enumerate(d.levels):
        x = synth.normal_f32(synth.rng_for(140 + i, 0), lv[5]).astype(np.float64)
        if kind == "outlier":
            x[7] = 3000.0
        elif kind in ("outliers", "outliers_small"):
            x = synth.outlier_vector(len(x), 30 + i, "normal" if kind == "outliers" else "small").astype(np.float64)
        elif kind == "tiny":
            x *= 1e-30
        elif kind == "huge":
            x *= 1e30
        elif kind == "mixed":
            x *= 10.0 ** np.repeat(np.arange(-8, 8), -(-len(x) // 16))[: len(x)]
        else:
            x[:] = 0.0
        xs[i] = x.astype(np.float32)
        lv[2].copy_(torch.from_numpy(xs[i]))
    if kind in ("outliers", "outliers_small"):
        wl.h = synth.outlier_vector(d.h.shape[0], 77, "normal" if kind == "outliers" else "small")
        d.h.copy_(torch.from_numpy(wl.h))
    pwg.step_plan(d)
    pwg.decode_step_weights(d)
    torch.cuda.synchronize()
    pwg.step_status(d)
    out = outputs(wl)
    mats = synth.layer(synth.W_STEP, 0, SMALL)
    for i, (name, members, _) in enumerate(synth.LEVELS):
        m = synth.stacked(mats, members)
        y, yr = out["levels"][i], ref.ternary_gemv(m.w, m.scale, xs[i])
        mag = ref.ternary_gemv_magnitude(m.w, m.scale, xs[i])
        if kind == "zero":
            assert not y.any()
        else:
            assert_gemv(y, yr, mag, f"{kind} {name}")
    if kind in ("outliers", "outliers_small"):
        lr = ref.int8_logits(wl.out_table.q, wl.out_table.scale, wl.h)
        assert_gemv(out["logits"], lr, ref.int8_logits_magnitude(wl.out_table.q, wl.out_table.scale, wl.h), kind)
        assert token_ok(out["token"], lr)
