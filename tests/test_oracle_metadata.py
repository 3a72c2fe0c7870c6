"""Pins of the metadata reference (oracle/kda_metadata.py): a hand-derived
batch, and on random batches a token-by-token brute force of what the tables
mean (every token of a prefill request falls in its own run of 64-token
chunks, every chunk holds 1..64 consecutive tokens of one request)."""
import json
import os

import numpy as np
import pytest

from oracle.kda_metadata import CHUNK, build_metadata

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_derived_batch():
    ex = json.load(open(os.path.join(GOLDEN, "kda_metadata_example.json")))
    cu, slot_idx, chunk_start, counts, error = build_metadata(ex["num_tokens"], ex["req_slot"], ex["n_slots"])
    e = ex["expected"]
    assert cu == e["cu_seqlens"]
    assert slot_idx == e["slot_idx"]
    assert chunk_start == e["chunk_start"]
    assert counts == e["counts"]
    assert error == e["error"]


@pytest.mark.parametrize("seed", range(6))
def test_tables_by_brute_force(seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(1, 300))
    n_slots = 50
    num_tokens = g.choice([0, 1, 1, 2, 63, 64, 65, 128, 200, -1], size=n)
    req_slot = g.integers(-2, n_slots + 3, size=n)
    cu, slot_idx, chunk_start, counts, error = build_metadata(num_tokens, req_slot, n_slots)
    # walk the packed token axis one token at a time
    owner, chunk_of = [], {}
    for r in range(n):
        for j in range(max(int(num_tokens[r]), 0)):
            owner.append(r)
    assert cu[-1] == len(owner)
    for tok, r in enumerate(owner):
        assert cu[r] <= tok < cu[r + 1]
        if slot_idx[r] >= 0 and num_tokens[r] >= 2:
            c = chunk_start[r] + (tok - cu[r]) // CHUNK
            assert chunk_start[r] <= c < chunk_start[r + 1]
            chunk_of.setdefault(c, []).append(tok)
    # chunks: 0 .. total - 1, each 1..64 consecutive tokens of one request
    assert sorted(chunk_of) == list(range(counts[3]))
    for c, toks in chunk_of.items():
        assert 1 <= len(toks) <= CHUNK and toks == list(range(toks[0], toks[0] + len(toks)))
        assert len({owner[t] for t in toks}) == 1
    for r in range(n):
        has = num_tokens[r] > 0 and 0 <= req_slot[r] < n_slots
        assert slot_idx[r] == (req_slot[r] if has else -1)
    assert counts[1] == sum(1 for r in range(n) if slot_idx[r] >= 0 and num_tokens[r] == 1)
    assert counts[2] == sum(1 for r in range(n) if slot_idx[r] >= 0 and num_tokens[r] >= 2)
    bad = any(t < 0 for t in num_tokens) or any(s < -1 or s >= n_slots for s in req_slot)
    assert error == int(bad)
