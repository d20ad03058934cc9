"""Pins of the chained-step oracle (oracle/chain.py) against facts that do
not come from it: hand-worked values, closed forms of softmax attention with
one key, identities of SiLU and RMSNorm, a scalar-loop brute force of whole
tiny steps, and the zero-matrix special case that reduces a step to the
pinned output projection.  A swapped gate/up, a dropped residual, a wrong
head mapping or a norm over the wrong length fails at least one."""
import math

import numpy as np
import pytest

from oracle import chain as ch
from oracle import reference as ref

RNG = np.random.default_rng(4321)


def test_rms_norm_hand_worked():
    # [1, 2, 3, 4]: mean square 30/4 = 7.5
    x = ch.rms_norm(np.array([1.0, 2.0, 3.0, 4.0]), np.ones(4), eps=0.0)
    assert np.allclose(x, np.array([1, 2, 3, 4]) / math.sqrt(7.5), rtol=1e-15, atol=0)
    # a constant vector normalises to its sign times the gain
    g = np.array([0.5, 2.0, -1.0])
    assert np.allclose(ch.rms_norm(np.full(3, -7.25), g, eps=0.0), -g, rtol=1e-15, atol=0)
    # eps enters under the root: h = [3, 4], mean square 12.5, eps 0.5 -> /sqrt(13)
    assert np.allclose(ch.rms_norm(np.array([3.0, 4.0]), np.ones(2), eps=0.5), np.array([3, 4]) / math.sqrt(13.0))


def test_rms_norm_scale_invariant_and_unit_rms():
    h = RNG.standard_normal(257)
    g = RNG.uniform(0.5, 1.5, 257)
    a = ch.rms_norm(h, g, eps=0.0)
    assert np.allclose(ch.rms_norm(1000.0 * h, g, eps=0.0), a, rtol=1e-13)
    assert math.isclose(float(np.sqrt(np.mean((a / g) ** 2))), 1.0, rel_tol=1e-13)


def test_silu_values_and_identity():
    assert ch.silu(np.array([0.0]))[0] == 0.0
    # sigmoid(ln 3) = 3 / 4
    assert math.isclose(float(ch.silu(np.array([math.log(3.0)]))[0]), 0.75 * math.log(3.0), rel_tol=1e-15)
    x = RNG.uniform(-30, 30, 1000)
    # x*s(x) - (-x)*s(-x) = x (s(x) + s(-x)) = x
    assert np.allclose(ch.silu(x) - ch.silu(-x), x, rtol=1e-12, atol=1e-12)
    # limits: very negative -> 0 from below, very positive -> x
    assert ch.silu(np.array([-800.0]))[0] == 0.0
    assert ch.silu(np.array([800.0]))[0] == 800.0


def _softmax_attention(q, keys, values, head_dim):
    """Textbook scaled-dot-product attention of one query over a cache."""
    s = np.array([float(np.dot(q, k)) / math.sqrt(head_dim) for k in keys])
    p = np.exp(s - s.max())
    p /= p.sum()
    return sum(pi * v for pi, v in zip(p, values))


@pytest.mark.parametrize("n_heads,n_kv,head_dim", [(32, 8, 128), (4, 4, 8), (6, 2, 1), (2, 1, 5)])
def test_one_position_attention_is_softmax_attention(n_heads, n_kv, head_dim):
    group = n_heads // n_kv
    q = RNG.standard_normal(n_heads * head_dim)
    k = RNG.standard_normal(n_kv * head_dim)
    v = RNG.standard_normal(n_kv * head_dim)
    got = ch.attention_one_position(v, n_heads, head_dim, group)
    for j in range(n_heads):
        kv = j // group
        sl, kvsl = slice(j * head_dim, (j + 1) * head_dim), slice(kv * head_dim, (kv + 1) * head_dim)
        one = _softmax_attention(q[sl], [k[kvsl]], [v[kvsl]], head_dim)
        # three identical cached positions: the same output
        three = _softmax_attention(q[sl], [k[kvsl]] * 3, [v[kvsl]] * 3, head_dim)
        assert np.allclose(got[sl], one, rtol=0, atol=0)
        assert np.allclose(got[sl], three, rtol=1e-15, atol=1e-15)
    if group == 1:
        assert np.array_equal(got, v)
    if head_dim == 1:
        assert np.array_equal(got, np.repeat(v, group))


def _tiny_problem(shape, n_layers, seed, zero_o_down=False):
    rng = np.random.default_rng(seed)
    hid, inter = shape.hidden, shape.inter
    rows = {"qkv": shape.q_rows + 2 * shape.kv_rows, "o": hid, "gate_up": 2 * inter, "down": hid}
    cols = {"qkv": hid, "o": shape.q_rows, "gate_up": hid, "down": inter}
    layers, gammas = [], []
    for _ in range(n_layers):
        mats = {}
        for m in ("qkv", "o", "gate_up", "down"):
            w = rng.integers(-1, 2, (rows[m], cols[m])).astype(np.int8)
            if zero_o_down and m in ("o", "down"):
                w[:] = 0
            mats[m] = (w, rng.uniform(0.01, 0.1, rows[m]).astype(np.float32))
        layers.append(mats)
        gammas.append((rng.uniform(0.5, 1.5, hid), rng.uniform(0.5, 1.5, hid)))
    vocab = 50
    out_t = rng.integers(-127, 128, (vocab, hid)).astype(np.int8)
    out_s = rng.uniform(0.001, 0.01, vocab).astype(np.float32)
    emb_t = rng.integers(-127, 128, (vocab, hid)).astype(np.int8)
    emb_s = rng.uniform(0.001, 0.01, vocab).astype(np.float32)
    g_final = rng.uniform(0.5, 1.5, hid)
    return layers, gammas, g_final, out_t, out_s, emb_t, emb_s


def _brute_step(layers, gammas, g_final, shape, out_t, out_s, emb_t, emb_s, token, eps):
    """The chained step in scalar loops with math.fsum, written out from the
    decoder layer's definition without the oracle's helpers."""
    hid, inter, hd = shape.hidden, shape.inter, shape.head_dim

    def matvec(w, s, x):
        return [float(s[r]) * math.fsum(int(w[r, k]) * x[k] for k in range(w.shape[1])) for r in range(w.shape[0])]

    def norm(h, g):
        ms = math.fsum(v * v for v in h) / len(h)
        return [float(g[i]) * h[i] / math.sqrt(ms + eps) for i in range(len(h))]

    h = [float(np.float32(int(emb_t[token, i])) * np.float32(emb_s[token])) for i in range(hid)]
    for mats, (ga, gm) in zip(layers, gammas):
        qkv = matvec(*mats["qkv"], norm(h, ga))
        v0 = shape.q_rows + shape.kv_rows
        a = []
        for head in range(shape.n_heads):
            kvh = head * shape.n_kv // shape.n_heads
            a.extend(qkv[v0 + kvh * hd:v0 + (kvh + 1) * hd])
        o = matvec(*mats["o"], a)
        h = [h[i] + o[i] for i in range(hid)]
        gu = matvec(*mats["gate_up"], norm(h, gm))
        m = [gu[i] / (1.0 + math.exp(-gu[i])) * gu[inter + i] for i in range(inter)]
        d = matvec(*mats["down"], m)
        h = [h[i] + d[i] for i in range(hid)]
    logits = [float(out_s[r]) * math.fsum(int(out_t[r, k]) * v for k, v in enumerate(norm(h, g_final)))
              for r in range(out_t.shape[0])]
    return h, logits


@pytest.mark.parametrize("shape", [ch.ChainShape(16, 24, 4, 2, 4), ch.ChainShape(12, 8, 3, 1, 4),
                                   ch.ChainShape(8, 16, 2, 2, 4)])
def test_chained_step_matches_scalar_brute_force(shape):
    prob = _tiny_problem(shape, 3, seed=shape.hidden * 7 + shape.inter)
    token = 17
    r = ch.chained_step(prob[0], prob[1], prob[2], shape, *prob[3:], token_in=token, eps=1e-6)
    h, logits = _brute_step(*prob[:3], shape, *prob[3:], token, 1e-6)
    assert np.allclose(r["h_final"], h, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["logits"], logits, rtol=1e-12, atol=1e-12)
    assert r["token"] == int(np.argmax(logits))


def test_zero_o_and_down_keep_the_embedding_row():
    shape = ch.ChainShape(16, 24, 4, 2, 4)
    layers, gammas, g_final, out_t, out_s, emb_t, emb_s = _tiny_problem(shape, 4, seed=99, zero_o_down=True)
    token = 3
    r = ch.chained_step(layers, gammas, g_final, shape, out_t, out_s, emb_t, emb_s, token_in=token)
    h0 = emb_t[token].astype(np.float32) * emb_s[token]
    for lay in r["layers"]:
        assert np.array_equal(lay["h_mid"], h0.astype(np.float64))
        assert np.array_equal(lay["h_out"], h0.astype(np.float64))
    # the step reduces to the (separately pinned) output projection of the
    # normalised embedding row
    ms = float(np.mean(h0.astype(np.float64) ** 2))
    x = g_final * h0.astype(np.float64) / math.sqrt(ms + ch.EPS)
    assert np.allclose(r["logits"], ref.int8_logits(out_t, out_s, x), rtol=1e-14, atol=0)


def test_zero_up_rows_silence_the_feed_forward_block():
    """silu(gate) * up with up = 0 is 0 whatever gate is; with gate = 0 the
    same (silu(0) = 0).  Only the attention branch then moves h."""
    shape = ch.ChainShape(16, 24, 4, 2, 4)
    layers, gammas, g_final, out_t, out_s, emb_t, emb_s = _tiny_problem(shape, 1, seed=5)
    w, s = layers[0]["gate_up"]
    w = w.copy()
    w[shape.inter:] = 0  # up rows
    layers[0]["gate_up"] = (w, s)
    lay = ch.chained_step(layers, gammas, g_final, shape, out_t, out_s, emb_t, emb_s, token_in=0)["layers"][0]
    assert np.any(lay["y"][2][:shape.inter] != 0)
    assert np.array_equal(lay["y"][3], np.zeros(shape.hidden))
    assert np.array_equal(lay["h_out"], lay["h_mid"])
