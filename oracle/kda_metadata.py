"""Plain CPU reference of the per-step batch metadata (integer work).

TEST INFRASTRUCTURE ONLY (tests and the smoke check); never part of the
product path.

"vLLM Kimi K3 support", section "Fused kernels and metadata optimisation"
(metadata builder bullet), names a dedicated KDA metadata builder: the
per-step tables the KDA kernels read are built in one fused launch instead
of a chain of eager tensor operations.  The pages do not list the tables.
The ones built here are exactly the ones this library's calls take or derive,
from two per-request arrays of the scheduler (tokens scheduled this step and
the request's state slot):

  cu_seqlens[r]   start of request r's tokens in the packed token axis
                  (exclusive prefix sum of the token counts, counts below
                  zero taken as 0), cu_seqlens[n] = total tokens;
  slot_idx[r]     the request's slot when it has tokens and its slot is in
                  [0, n_slots); -1 (a padding row) when it has no tokens or
                  its slot is -1 or out of range;
  chunk_start[r]  first 64-token chunk of request r in the chunk axis of the
                  chunked prefill: requests of two or more tokens with a
                  valid slot take ceil(len / 64) chunks, all others none;
                  chunk_start[n] = total chunks;
  counts          [total tokens, one-token requests with a slot (the decode
                  rows of a mixed batch), requests of two or more tokens with
                  a slot (the prefill sequences), total chunks];
  error           1 when any count is negative or any slot is outside
                  [-1, n_slots), else 0.

Everything is a plain loop over the requests in order.
"""
from __future__ import annotations

CHUNK = 64


def build_metadata(num_tokens, req_slot, n_slots):
    """Returns (cu_seqlens, slot_idx, chunk_start, counts, error) as Python
    lists / int."""
    n = len(num_tokens)
    assert len(req_slot) == n
    cu = [0] * (n + 1)
    slot_idx = [-1] * n
    chunk_start = [0] * (n + 1)
    ones = prefills = 0
    error = 0
    for r in range(n):
        t = int(num_tokens[r])
        s = int(req_slot[r])
        if t < 0:
            error = 1
            t = 0
        valid = 0 <= s < n_slots
        if not valid and s != -1:
            error = 1
        cu[r + 1] = cu[r] + t
        chunks = 0
        if t > 0 and valid:
            slot_idx[r] = s
            if t == 1:
                ones += 1
            else:
                prefills += 1
                chunks = (t + CHUNK - 1) // CHUNK
        chunk_start[r + 1] = chunk_start[r] + chunks
    counts = [cu[n], ones, prefills, chunk_start[n]]
    return cu, slot_idx, chunk_start, counts, error
