"""Chained decode step on the GPU (every level's input formed from earlier
outputs: RMSNorm, one-position grouped-query attention, SwiGLU, residual
sums) against the oracle, on the two ordered schedules.

Each level is checked against the oracle applied to the GPU's own inputs of
that level (the formed vector's sources as the GPU left them), so every
formation and every GEMV is held to its own bound:
  * residual sums bit for bit (one float32 addition, rounded once);
  * attention outputs bit for bit (a copy);
  * RMSNorm and SwiGLU vectors within 1e-5 of each element's oracle value
    (float32 sum of squares, root, quotient, expf against float64), or
    within float32's smallest normal number 2^-126 where the value is that
    small (float32 holds no relative precision there: silu of a very negative
    gate underflows);
  * level outputs and logits at the GEMV bound of tests/parity.py;
  * the token exactly (or within the oracle's near-tie set).
The whole chain is also run by the oracle from the same token: the final
residual stream within 1e-4 relative L2 of it (float32 rounding carried
through every layer) and the same greedy token."""
import numpy as np
import pytest

import synth
from oracle import chain as ch
from oracle import reference as ref
from tests.parity import assert_gemv, token_ok

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import packed_weight_gemv_amd as pwg  # noqa: E402
from packed_weight_gemv_amd.workload import build_step, make_chained  # noqa: E402

FORM_RTOL = 1e-5
FLT_MIN_NORMAL = 2.0 ** -126
CHAIN_REL_L2 = 1e-4

# 4 query heads over 1 key/value head of 128, or 8 over 2 of 64
CHAIN_SMALL = {"q": (512, 512), "k": (128, 512), "v": (128, 512), "o": (512, 512),
               "gate": (1536, 512), "up": (1536, 512), "down": (512, 1536)}
SCHEDULES = [pwg.SCHEDULE_LEVELS, pwg.SCHEDULE_PERSISTENT]
SCHED_IDS = ["levels", "persistent"]


def run(cs):
    pwg.step_plan(cs.desc)
    pwg.decode_step_weights(cs.desc)
    torch.cuda.synchronize()
    pwg.step_status(cs.desc)


def f32_sum(a, b):
    return (np.asarray(a, np.float64) + np.asarray(b, np.float64)).astype(np.float32)


def assert_formed(x_gpu, x_ref, what):
    x_ref = np.asarray(x_ref, np.float64)
    d = np.abs(x_gpu.astype(np.float64) - x_ref)
    assert np.isfinite(x_gpu).all(), what
    bad = (d > FORM_RTOL * np.abs(x_ref)) & (d > FLT_MIN_NORMAL)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements, worst {float((d / np.maximum(np.abs(x_ref), 1e-300)).max())}"


def level_weights(wl, shapes, n_layers):
    """Host (w, s, rows) per level: all rows for small shapes, the sampled
    rows kept by the workload for the 8B shape."""
    out = []
    if shapes is not None:
        for layer in range(n_layers):
            mats = synth.layer(synth.W_STEP, layer, shapes)
            for _, members, _ in synth.LEVELS:
                m = synth.stacked(mats, members)
                out.append((m.w, m.scale, None))
    else:
        out = [(s.w, s.scale, s.rows) for s in wl.samples]
    return out


def check_teacher_forced(wl, cs, token, weights):
    d = cs.desc
    n_layers = len(d.levels) // 4
    hidden = d.hidden
    x = [t.cpu().numpy() for t in cs.x]
    y = [t.cpu().numpy() for t in cs.y]
    hs = [(a.cpu().numpy(), b.cpu().numpy()) for a, b in cs.h]
    _, _, deq = ref.embed_gather(wl.emb_table.q, wl.emb_table.scale, [token])
    for layer in range(n_layers):
        i0 = 4 * layer
        ga, gm = cs.gains[layer]
        h_l = deq[0] if layer == 0 else f32_sum(hs[layer - 1][1], y[i0 - 1])
        assert np.array_equal(hs[layer][0], h_l), f"layer {layer}: residual entering the layer"
        assert_formed(x[i0], ch.rms_norm(h_l, ga, cs.eps), f"layer {layer}: qkv input")
        q_rows, inter = d.levels[i0 + 1][5], d.levels[i0 + 3][5]
        kv_rows = (d.levels[i0][4] - q_rows) // 2
        v = y[i0][q_rows + kv_rows:]
        attn = ch.attention_one_position(v, q_rows // cs.head_dim, cs.head_dim, q_rows // kv_rows)
        assert np.array_equal(x[i0 + 1], attn.astype(np.float32)), f"layer {layer}: attention output"
        h_mid = f32_sum(h_l, y[i0 + 1])
        assert np.array_equal(hs[layer][1], h_mid), f"layer {layer}: residual after attention"
        assert_formed(x[i0 + 2], ch.rms_norm(h_mid, gm, cs.eps), f"layer {layer}: gate|up input")
        assert_formed(x[i0 + 3], ch.swiglu(y[i0 + 2], inter), f"layer {layer}: down input")
        for j in range(4):
            w, s, rows = weights[i0 + j]
            got = y[i0 + j] if rows is None else y[i0 + j][rows]
            assert_gemv(got, ref.ternary_gemv(w, s, x[i0 + j]), ref.ternary_gemv_magnitude(w, s, x[i0 + j]),
                        f"layer {layer} level {j}")
    h_fin = f32_sum(hs[-1][1], y[-1])
    assert np.array_equal(cs.h_final.cpu().numpy(), h_fin), "final residual"
    h_out = d.h.cpu().numpy()
    assert_formed(h_out, ch.rms_norm(h_fin, cs.g_final, cs.eps), "output projection input")
    logits = ref.int8_logits(wl.out_table.q, wl.out_table.scale, h_out)
    if d.logits_out is not None:
        assert_gemv(d.logits_out.cpu().numpy(), logits,
                    ref.int8_logits_magnitude(wl.out_table.q, wl.out_table.scale, h_out), "logits")
    tok = int(d.token_out.cpu()[0])
    assert token_ok(tok, logits)
    assert hidden == h_out.size
    return tok


def oracle_chain(wl, cs, weights, shape, token):
    n_layers = len(cs.desc.levels) // 4
    layers = []
    for layer in range(n_layers):
        ws = weights[4 * layer:4 * layer + 4]
        layers.append({m: (w, s) for m, (w, s, _) in zip(("qkv", "o", "gate_up", "down"), ws)})
    return ch.chained_step(layers, cs.gains, cs.g_final, shape, wl.out_table.q, wl.out_table.scale,
                           wl.emb_table.q, wl.emb_table.scale, token, cs.eps)


@pytest.mark.parametrize("head_dim", [128, 64])
@pytest.mark.parametrize("schedule", SCHEDULES, ids=SCHED_IDS)
def test_small_chained_steps_match_oracle(schedule, head_dim):
    n_layers = 3
    wl = build_step(n_layers=n_layers, shapes=CHAIN_SMALL, vocab=3000, hidden=512, with_logits=True,
                    schedule=pwg.SCHEDULE_LEVELS)
    cs = make_chained(wl, schedule=schedule, head_dim=head_dim)
    weights = level_weights(wl, CHAIN_SMALL, n_layers)
    shape = ch.ChainShape(512, 1536, 512 // head_dim, 128 // head_dim, head_dim)
    token = wl.token0
    for step in range(2):  # the second step starts from the first step's token
        run(cs)
        new = check_teacher_forced(wl, cs, token, weights)
        r = oracle_chain(wl, cs, weights, shape, token)
        h = cs.h_final.cpu().numpy().astype(np.float64)
        rel = np.linalg.norm(h - r["h_final"]) / np.linalg.norm(r["h_final"])
        assert rel <= CHAIN_REL_L2, f"step {step}: final residual rel L2 {rel}"
        assert token_ok(new, r["logits"]), f"step {step}"
        token = new


@pytest.mark.parametrize("kv_rows,head_dim", [(512, 64), (256, 64), (128, 32)], ids=["group1", "group2", "hd32"])
@pytest.mark.parametrize("schedule", SCHEDULES, ids=SCHED_IDS)
def test_chained_attention_groupings(schedule, kv_rows, head_dim):
    """One-position attention with every query head on its own key/value head
    (group 1), two per key/value head, and heads of 32 values: the gather of
    value rows into the o projection's input against the oracle."""
    n_layers = 2
    shapes = dict(CHAIN_SMALL, k=(kv_rows, 512), v=(kv_rows, 512))
    wl = build_step(n_layers=n_layers, shapes=shapes, vocab=3000, hidden=512, with_logits=True,
                    schedule=pwg.SCHEDULE_LEVELS)
    cs = make_chained(wl, schedule=schedule, head_dim=head_dim)
    weights = level_weights(wl, shapes, n_layers)
    shape = ch.ChainShape(512, 1536, 512 // head_dim, kv_rows // head_dim, head_dim)
    token = wl.token0
    run(cs)
    new = check_teacher_forced(wl, cs, token, weights)
    r = oracle_chain(wl, cs, weights, shape, token)
    h = cs.h_final.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(h - r["h_final"]) / np.linalg.norm(r["h_final"])
    assert rel <= CHAIN_REL_L2, f"final residual rel L2 {rel}"
    assert token_ok(new, r["logits"])


@pytest.mark.parametrize("schedule", SCHEDULES, ids=SCHED_IDS)
def test_schedules_form_the_first_input_alike(schedule):
    """Both ordered schedules form vectors with workgroups of 512 threads in
    one reduction order, so the first formed input (from the embedding row,
    before any GEMV) is identical bit for bit, and the token the same."""
    wl = build_step(n_layers=2, shapes=CHAIN_SMALL, vocab=3000, hidden=512, with_logits=False,
                    schedule=pwg.SCHEDULE_LEVELS)
    a = make_chained(wl, schedule=pwg.SCHEDULE_LEVELS)
    b = make_chained(wl, schedule=schedule)
    run(a)
    run(b)
    assert torch.equal(a.x[0], b.x[0]) and torch.equal(a.h[0][0], b.h[0][0])
    assert int(a.desc.token_out.cpu()[0]) == int(b.desc.token_out.cpu()[0])


@pytest.mark.parametrize("schedule", SCHEDULES, ids=SCHED_IDS)
def test_8b_shape_two_layers_full_vocab(schedule):
    wl = build_step(n_layers=2, with_logits=True, schedule=pwg.SCHEDULE_LEVELS)
    cs = make_chained(wl, schedule=schedule)
    weights = level_weights(wl, None, 2)
    run(cs)
    check_teacher_forced(wl, cs, wl.token0, weights)


@pytest.mark.parametrize("schedule", SCHEDULES, ids=SCHED_IDS)
def test_graph_replay_of_a_chained_step(schedule):
    """A captured chained step replayed several times, each replay starting
    from the previous token, matches eager steps from the same tokens."""
    wl = build_step(n_layers=2, shapes=CHAIN_SMALL, vocab=3000, hidden=512, with_logits=False,
                    schedule=pwg.SCHEDULE_LEVELS)
    cs = make_chained(wl, schedule=schedule)
    pwg.step_plan(cs.desc)
    eager = []
    t0 = wl.token0
    for _ in range(3):
        pwg.decode_step_weights(cs.desc)
        torch.cuda.synchronize()
        eager.append((int(cs.desc.token_out.cpu()[0]), cs.h_final.clone()))
    cs.desc.token_in.fill_(t0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pwg.decode_step_weights(cs.desc, stream=s)
    torch.cuda.synchronize()
    for tok, h in eager:
        g.replay()
        torch.cuda.synchronize()
        pwg.step_status(cs.desc)
        assert int(cs.desc.token_out.cpu()[0]) == tok
        assert torch.equal(cs.h_final, h)


@pytest.mark.parametrize("schedule", SCHEDULES, ids=SCHED_IDS)
def test_chained_step_with_outlier_activations(schedule):
    """RMSNorm gains with massive entries (+-3e3 and +-1e4 at several places,
    and outliers among gains near 1e-3) put the same outliers into every
    formed level input and into h: every level, the logits and the token
    still meet the stated criteria, teacher-forced and end to end."""
    n_layers = 2
    wl = build_step(n_layers=n_layers, shapes=CHAIN_SMALL, vocab=3000, hidden=512, with_logits=True,
                    schedule=pwg.SCHEDULE_LEVELS)
    cs = make_chained(wl, schedule=schedule)
    d = cs.desc
    gains = []
    for layer in range(n_layers):
        ga = synth.outlier_vector(512, 60 + 2 * layer)
        gm = synth.outlier_vector(512, 61 + 2 * layer)
        d.levels[4 * layer][6].gamma.copy_(torch.from_numpy(ga))
        d.levels[4 * layer + 2][6].gamma.copy_(torch.from_numpy(gm))
        gains.append((ga, gm))
    cs.gains[:] = gains
    cs.g_final[:] = synth.outlier_vector(512, 70)
    d.h_in.gamma.copy_(torch.from_numpy(cs.g_final))
    d._c = None
    torch.cuda.synchronize()
    weights = level_weights(wl, CHAIN_SMALL, n_layers)
    shape = ch.ChainShape(512, 1536, 4, 1, 128)
    run(cs)
    tok = check_teacher_forced(wl, cs, wl.token0, weights)
    r = oracle_chain(wl, cs, weights, shape, wl.token0)
    h = cs.h_final.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(h - r["h_final"]) / np.linalg.norm(r["h_final"])
    assert rel <= CHAIN_REL_L2, f"final residual rel L2 {rel}"
    assert token_ok(tok, r["logits"])
