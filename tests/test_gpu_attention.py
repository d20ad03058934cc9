"""Grouped-query decode attention on the GPU against the oracle
(oracle/attention.py) through the C ABI.

Bound: the relative L2 error of the output is at most 1e-5, and every
element is within 1e-4 of its oracle value relative to that value or within
1e-6 * max(1, S_j) of its magnitude sum_t p_t |v_t| (the same attention over
|V|), where S_j = max_t scale * sum_d |q_jd k_td| bounds head j's scores:
tests/parity.py's GEMV criterion with the softmax weights in place of row
scales, widened by the score size because a float32 score carries an
absolute error of ~1e-7 * S_j, which becomes a relative error of each
weight p_t (peaked softmaxes have S_j in the hundreds).  float32
accumulation over up to 32,768 positions with online rescaling stays far
inside it."""
import math

import numpy as np
import pytest

import synth
from oracle import attention as at
from tests.parity import assert_gemv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import packed_weight_gemv_amd as pwg  # noqa: E402


def device_inputs(q, k, v):
    dev = torch.device("cuda:0")
    return (torch.from_numpy(q).to(dev), torch.from_numpy(k.view(np.int16)).to(dev),
            torch.from_numpy(v.view(np.int16)).to(dev))


def score_bound(q, k, n_heads, n_kv, hd, scale):
    """max(1, S_j) per output element, S_j = max_t scale * sum_d |q_jd k_td|."""
    kf = np.abs(at.bf16_to_f64(k).reshape(-1, n_kv, hd))
    qa = np.abs(np.asarray(q, np.float64).reshape(n_heads, hd))
    group = n_heads // n_kv
    sj = np.array([(kf[:, j // group, :] @ qa[j]).max() * scale for j in range(n_heads)])
    return np.repeat(np.maximum(1.0, sj), hd)


def check(out_gpu, q, k, v, n_heads, n_kv, hd, scale, what):
    ref = at.gqa_decode(q, k, v, n_heads, n_kv, hd, scale)
    mag = at.gqa_decode(q, k, v & np.uint16(0x7FFF), n_heads, n_kv, hd, scale)
    return assert_gemv(out_gpu, ref, mag * score_bound(q, k, n_heads, n_kv, hd, scale), what)


def inputs(ctx, n_heads, n_kv, hd, seed):
    rng = synth.rng_for(synth.W_ATTN, 1000 + seed, ctx)
    q = rng.standard_normal(n_heads * hd).astype(np.float32)
    k = synth.bf16_bits(rng.standard_normal((ctx, n_kv, hd)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((ctx, n_kv, hd)).astype(np.float32))
    return q, k, v


@pytest.mark.parametrize("n_heads,n_kv,hd,ctx", [
    (32, 8, 128, 1), (32, 8, 128, 37), (32, 8, 128, 4096), (32, 8, 128, 5001), (16, 8, 128, 300),
    (8, 8, 128, 129), (8, 8, 64, 1000), (8, 4, 64, 129), (16, 4, 64, 2047), (4, 1, 128, 77)])
def test_matches_oracle(n_heads, n_kv, hd, ctx):
    q, k, v = inputs(ctx, n_heads, n_kv, hd, 0)
    scale = 1 / math.sqrt(hd)
    qd, kd, vd = device_inputs(q, k, v)
    out = pwg.gqa_decode_attention(kd, vd, qd, n_heads, n_kv, hd, scale)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), q, k, v, n_heads, n_kv, hd, scale, f"{n_heads}/{n_kv}/{hd}/{ctx}")


def test_8b_layer_at_32k_context():
    """One layer of the 8B shape (32 query heads over 8 key/value heads of
    128) at 32,768 cached positions: 268 MB of bfloat16 keys and values."""
    ctx = 32768
    q, k, v = synth.kv_cache(0, ctx)
    qd, kd, vd = device_inputs(q, k, v)
    out = pwg.gqa_decode_attention(kd, vd, qd, 32, 8, 128, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    check(out.cpu().numpy(), q, k, v, 32, 8, 128, 1 / math.sqrt(128), "8B layer, 32K positions")


def test_peaked_scores_and_workspace_reuse():
    """Large scores (a near one-hot softmax) and two calls on one workspace,
    the second over a shorter cache."""
    n_heads, n_kv, hd = 32, 8, 128
    q, k, v = inputs(3000, n_heads, n_kv, hd, 1)
    q = (q * 40).astype(np.float32)
    ws = torch.zeros(pwg.attention_workspace_bytes(n_heads, n_kv, hd, 3000), dtype=torch.uint8, device="cuda:0")
    for ctx in (3000, 700):
        qd, kd, vd = device_inputs(q, k[:ctx].copy(), v[:ctx].copy())
        out = pwg.gqa_decode_attention(kd, vd, qd, n_heads, n_kv, hd, 0.1, workspace=ws)
        torch.cuda.synchronize()
        check(out.cpu().numpy(), q, k[:ctx], v[:ctx], n_heads, n_kv, hd, 0.1, f"ctx {ctx}")


def test_graph_replay_matches_eager():
    n_heads, n_kv, hd, ctx = 32, 8, 128, 2500
    q, k, v = inputs(ctx, n_heads, n_kv, hd, 2)
    qd, kd, vd = device_inputs(q, k, v)
    ws = torch.zeros(pwg.attention_workspace_bytes(n_heads, n_kv, hd, ctx), dtype=torch.uint8, device="cuda:0")
    out = torch.empty(n_heads * hd, dtype=torch.float32, device="cuda:0")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        pwg.gqa_decode_attention(kd, vd, qd, n_heads, n_kv, hd, 0.09, out=out, workspace=ws, stream=s)
        s.synchronize()
        eager = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            pwg.gqa_decode_attention(kd, vd, qd, n_heads, n_kv, hd, 0.09, out=out, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    check(eager.cpu().numpy(), q, k, v, n_heads, n_kv, hd, 0.09, "graph")
