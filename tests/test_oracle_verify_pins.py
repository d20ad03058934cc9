"""Pins of the verify-step acceptance rule (oracle/verify.py): the edge
cases, and the property that defines it: a draft-and-verify loop emits
exactly the tokens of plain greedy decoding with the large model, whatever
the drafts are (a toy deterministic next-token function stands in for the
model)."""
import numpy as np

from oracle import verify


def test_edge_cases():
    assert verify.accept([5, 1, 2, 3], [1, 2, 3, 9], 3) == (3, 9)       # all accepted, bonus token
    assert verify.accept([5, 1, 2, 3], [7, 2, 3, 9], 3) == (0, 7)       # first draft rejected
    assert verify.accept([5, 1, 2, 3], [1, 8, 3, 9], 3) == (1, 8)       # later agreement does not count
    assert verify.accept([5], [4], 0) == (0, 4)                         # no drafts: one greedy token
    assert verify.accept([5, 1, 2, 3, 0, 0, 0, 0], [1, 2, 6, 6, 6, 6, 6, 6], 3) == (2, 6)  # padding ignored


def test_draft_and_verify_equals_greedy():
    rng = np.random.default_rng(11)
    V = 50
    table = rng.integers(0, V, size=(V, V))         # next token from the last two tokens

    def big(prev2, prev1):
        return int(table[prev2, prev1])

    for trial in range(40):
        seq = [1, 2]
        greedy = [1, 2]
        for _ in range(30):
            greedy.append(big(greedy[-2], greedy[-1]))
        drafted_ok = rng.uniform()
        while len(seq) < len(greedy):
            n = int(rng.integers(0, 8))
            drafts, ctx = [], list(seq)
            for _ in range(n):  # a draft model right with probability drafted_ok
                t = big(ctx[-2], ctx[-1]) if rng.uniform() < drafted_ok else int(rng.integers(0, V))
                drafts.append(t)
                ctx.append(t)
            tokens_in = [seq[-1]] + drafts
            full = seq[:-1] + tokens_in
            targets = [big(full[len(seq) - 2 + i], full[len(seq) - 1 + i]) for i in range(n + 1)]
            k, nxt = verify.accept(tokens_in, targets, n)
            seq.extend(drafts[:k] + [nxt])
        assert seq[:len(greedy)] == greedy[:len(seq)]
