"""Device-side acceptance of drafted tokens (pwg_verify_accept) against the
oracle's rule (oracle/verify.py), exactly: planted agreement prefixes for
every draft count, and a verify step captured in one graph: the batched
int8 output projection over 8 vectors produces the large model's greedy
tokens, the acceptance kernel reads them on the device."""
import numpy as np
import pytest

import synth
from oracle import reference as ref
from oracle import verify

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import packed_weight_gemv_amd as pwg  # noqa: E402

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("n_drafts", [0, 1, 2, 3, 7, 15])
def test_planted_prefixes(n_drafts):
    rng = np.random.default_rng(100 + n_drafts)
    for k_true in range(n_drafts + 1):
        targets = rng.integers(0, 151936, 16).astype(np.int32)
        tokens = rng.integers(0, 151936, 16).astype(np.int32)
        tokens[1:k_true + 1] = targets[:k_true]
        if k_true < n_drafts:
            tokens[k_true + 1] = (targets[k_true] + 1) % 151936      # first disagreement
        tokens[k_true + 2:] = targets[k_true + 1:15]                  # later agreement must not count
        acc, nxt = pwg.verify_accept(torch.from_numpy(tokens).to(DEV), torch.from_numpy(targets).to(DEV), n_drafts)
        torch.cuda.synchronize()
        assert (int(acc[0]), int(nxt[0])) == verify.accept(tokens, targets, n_drafts) == (k_true, int(targets[k_true]))


def test_verify_step_in_one_graph():
    vocab, hidden, batch = 3000, 1024, 8
    tab = synth.int8_table((synth.W_BATCH, 9, 0), vocab, hidden)
    h = synth.batch_inputs(batch, hidden, 9)
    targets_ref = [ref.greedy_token(ref.int8_logits(tab.q, tab.scale, h[b]))[0] for b in range(batch)]
    qt = pwg.tile_rows(torch.from_numpy(tab.q).to(DEV), vocab, hidden)
    scale, hd = torch.from_numpy(tab.scale).to(DEV), torch.from_numpy(h).to(DEV)
    ws = torch.zeros(max(1, pwg.argmax_workspace_bytes(vocab, batch)), dtype=torch.uint8, device=DEV)
    targets = torch.empty(batch, dtype=torch.int32, device=DEV)
    # 5 drafts: the first three agree with the large model, the fourth does not
    tokens = np.array([7] + targets_ref[:3] + [(targets_ref[3] + 1) % vocab, 0, 0, 0], dtype=np.int32)
    tokens_d = torch.from_numpy(tokens).to(DEV)
    acc = torch.empty(4, dtype=torch.int32, device=DEV)
    nxt = torch.empty(4, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            pwg.int8_gemv_argmax_tiled(qt, scale, vocab, hidden, hd, workspace=ws, token_out=targets, stream=s)
            pwg.verify_accept(tokens_d, targets, 5, accepted=acc, next_token=nxt, stream=s)
    torch.cuda.synchronize()
    for _ in range(3):
        acc.fill_(-1)
        nxt.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert targets.cpu().tolist() == targets_ref
        assert (int(acc[0]), int(nxt[0])) == verify.accept(tokens, targets_ref, 5) == (3, targets_ref[3])
