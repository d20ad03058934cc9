"""pwg_int8_gemv_argmax_noalloc (scratch in the library's fixed device array,
no workspace, no allocation) against pwg_int8_gemv_argmax with a workspace:
the same tokens and logits bit for bit, on two calls in a row, the second
with a smaller input; a request beyond the array's size is refused."""
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


def both(tab, h):
    q, t, hd = dev(tab.q), dev(tab.scale), dev(h)
    rows = tab.q.shape[0]
    shape = (h.shape[0], rows) if h.ndim == 2 else (rows,)
    lo_ref = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    lo_na = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    tok_ref = pwg.int8_gemv_argmax(q, t, hd, logits_out=lo_ref)
    tok_na = torch.full((h.shape[0] if h.ndim == 2 else 1,), -1, dtype=torch.int32, device=DEV)
    pwg.int8_gemv_argmax_noalloc(q, t, hd, token_out=tok_na, logits_out=lo_na)
    torch.cuda.synchronize()
    return tok_ref.cpu().numpy(), lo_ref.cpu().numpy(), tok_na.cpu().numpy(), lo_na.cpu().numpy()


@pytest.mark.parametrize("batch", [1, 8])
def test_noalloc_matches_the_workspace_entry_point(batch):
    # first call: a larger table; second call: a smaller one (the array keeps
    # the first call's contents)
    for rows, cols, seed in ((20000, 4096, 0), (777, 1024, 1)):
        tab = synth.int8_table((160, seed), rows, cols)
        h = synth.batch_inputs(batch, cols, 160 + seed) if batch > 1 else synth.normal_f32(synth.rng_for(160, seed), cols)
        tr, lr, tn, ln = both(tab, h)
        assert np.array_equal(tn, tr), (rows, cols, batch)
        assert np.array_equal(ln.view(np.uint32), lr.view(np.uint32)), (rows, cols, batch)
        lo = ref.int8_logits(tab.q, tab.scale, h)
        for b in range(batch):
            lb = lo if batch == 1 else lo[b]
            hb = h if batch == 1 else h[b]
            got = ln if batch == 1 else ln[b]
            assert token_ok(int(tn[b]), lb)
            assert_gemv(got, lb, ref.int8_logits_magnitude(tab.q, tab.scale, hb), f"{rows}x{cols} vector {b}")


def test_noalloc_refuses_requests_beyond_its_array():
    rows, cols, batch = 151936, 4096, 16    # 1.05 MB of scratch > 1 MiB
    q = torch.zeros((rows, cols), dtype=torch.int8, device=DEV)
    t = torch.ones(rows, dtype=torch.float32, device=DEV)
    h = torch.zeros((batch, cols), dtype=torch.float32, device=DEV)
    with pytest.raises(pwg.PwgError, match="scratch"):
        pwg.int8_gemv_argmax_noalloc(q, t, h, token_out=torch.empty(batch, dtype=torch.int32, device=DEV))
