"""Plain reference of the speculative verify step's acceptance rule.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Source: the page "The Neutrino Engine" (fermionresearch.com), section "The
0.6B model does not get to decide": a small model drafts tokens, the large
model scores them in one batched forward pass and keeps the drafted tokens
only while its own greedy choice agrees, so the output is exactly what the
large model alone would have produced.

Reading (the pages give no interface): the pass runs on positions 0..n,
position 0 fed the last accepted token and position i >= 1 fed draft i; the
large model's greedy token after position i is target[i].  Draft i + 1 is
accepted while target[i] == draft[i + 1] for every earlier i; with k drafts
accepted, the step emits drafts 1..k and then target[k] (the large model's
own next token), k + 1 tokens in all.

Pins (tests marked "not gpu"): every draft accepted, none accepted, a
mismatch in the middle (later agreement does not count), no drafts; and
the identity with plain greedy decoding on a toy deterministic model.
"""
from __future__ import annotations


def accept(tokens_in, targets, n_drafts: int):
    """tokens_in[0] = last accepted token, tokens_in[1..n_drafts] = drafts;
    targets[i] = the large model's greedy token after position i.
    Returns (k accepted drafts, next token = targets[k])."""
    k = 0
    while k < n_drafts and int(targets[k]) == int(tokens_in[k + 1]):
        k += 1
    return k, int(targets[k])
