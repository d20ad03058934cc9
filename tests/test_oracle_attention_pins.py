"""Pins of the decode-attention oracle (oracle/attention.py) against facts
that do not come from it: hand-made bfloat16 patterns, the one-position
closed form, identical keys, a dominant score, invariance to a constant
score shift and to position order, and a scalar-loop brute force.  A wrong
head mapping, a missing scale, a transposed cache or a softmax over the
wrong axis fails at least one."""
import math

import numpy as np
import pytest

from oracle import attention as at
from oracle import chain as ch

RNG = np.random.default_rng(777)


def to_bf16(x):
    """Round-to-nearest-even float32 -> bfloat16 bits (test input helper)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def test_bf16_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x3FC0, 0x4049, 0x7F80], np.uint16)
    vals = at.bf16_to_f64(bits)
    assert vals[:6].tolist() == [1.0, -1.0, 2.0, 0.0, -0.0, 1.5]
    assert vals[6] == 3.140625 and math.isinf(vals[7])


@pytest.mark.parametrize("n_heads,n_kv,head_dim", [(32, 8, 128), (4, 2, 16), (3, 3, 8)])
def test_one_position_is_the_value_vector(n_heads, n_kv, head_dim):
    q = RNG.standard_normal(n_heads * head_dim).astype(np.float32)
    k = to_bf16(RNG.standard_normal((1, n_kv, head_dim)))
    v = to_bf16(RNG.standard_normal((1, n_kv, head_dim)))
    out = at.gqa_decode(q, k, v, n_heads, n_kv, head_dim, 1 / math.sqrt(head_dim))
    ref = ch.attention_one_position(at.bf16_to_f64(v).reshape(-1), n_heads, head_dim, n_heads // n_kv)
    assert np.array_equal(out, ref)


def test_identical_keys_average_the_values():
    n_heads, n_kv, hd, ctx = 8, 2, 16, 37
    k1 = to_bf16(RNG.standard_normal((1, n_kv, hd)))
    k = np.repeat(k1, ctx, axis=0)
    v = to_bf16(RNG.standard_normal((ctx, n_kv, hd)))
    out = at.gqa_decode(RNG.standard_normal(n_heads * hd), k, v, n_heads, n_kv, hd, 0.25).reshape(n_heads, hd)
    mean = at.bf16_to_f64(v).mean(axis=0)
    for j in range(n_heads):
        assert np.allclose(out[j], mean[j // (n_heads // n_kv)], rtol=1e-13, atol=1e-15)


def test_dominant_score_selects_its_value():
    n_heads, n_kv, hd, ctx = 4, 1, 8, 50
    q = np.zeros(n_heads * hd, np.float32)
    q[::hd] = 1.0                               # every head reads dimension 0 of the key
    kf = np.zeros((ctx, n_kv, hd), np.float32)
    kf[23, 0, 0] = 64.0                         # score 64 * scale for position 23, 0 elsewhere
    v = to_bf16(RNG.standard_normal((ctx, n_kv, hd)))
    out = at.gqa_decode(q, to_bf16(kf), v, n_heads, n_kv, hd, 1.0).reshape(n_heads, hd)
    assert np.allclose(out, at.bf16_to_f64(v)[23, 0], rtol=1e-20, atol=1e-25)


def test_score_shift_and_position_order_do_not_matter():
    n_heads, n_kv, hd, ctx = 8, 4, 16, 29
    q = RNG.standard_normal(n_heads * hd).astype(np.float32)
    k = to_bf16(RNG.standard_normal((ctx, n_kv, hd)))
    v = to_bf16(RNG.standard_normal((ctx, n_kv, hd)))
    base = at.gqa_decode(q, k, v, n_heads, n_kv, hd, 0.3)
    perm = RNG.permutation(ctx)
    assert np.allclose(at.gqa_decode(q, k[perm], v[perm], n_heads, n_kv, hd, 0.3), base, rtol=1e-12, atol=1e-14)
    # a key component along a dimension where q is 0 for every head changes no score
    q2 = q.reshape(n_heads, hd).copy()
    q2[:, 5] = 0
    kf = at.bf16_to_f64(k).astype(np.float32)
    kf2 = kf.copy()
    kf2[:, :, 5] = 100.0
    a = at.gqa_decode(q2.reshape(-1), to_bf16(kf), v, n_heads, n_kv, hd, 0.3)
    b = at.gqa_decode(q2.reshape(-1), to_bf16(kf2), v, n_heads, n_kv, hd, 0.3)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_scalar_loop_brute_force():
    n_heads, n_kv, hd, ctx = 6, 2, 5, 11
    q = RNG.standard_normal(n_heads * hd).astype(np.float32)
    k = to_bf16(RNG.standard_normal((ctx, n_kv, hd)))
    v = to_bf16(RNG.standard_normal((ctx, n_kv, hd)))
    kf, vf = at.bf16_to_f64(k), at.bf16_to_f64(v)
    scale = 0.7
    out = at.gqa_decode(q, k, v, n_heads, n_kv, hd, scale)
    for j in range(n_heads):
        kv = j * n_kv // n_heads
        scores = [scale * math.fsum(float(q[j * hd + d]) * kf[t, kv, d] for d in range(hd)) for t in range(ctx)]
        w = [math.exp(sc) for sc in scores]
        z = math.fsum(w)
        for d in range(hd):
            assert math.isclose(out[j * hd + d], math.fsum(w[t] * vf[t, kv, d] for t in range(ctx)) / z,
                                rel_tol=1e-12, abs_tol=1e-14)
