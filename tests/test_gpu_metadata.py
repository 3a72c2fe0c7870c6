"""GPU check of kda_build_metadata: bit-exact against the plain reference
(oracle/kda_metadata.py) on the hand-derived batch and on random batches of
1 to 3000 requests (several 1024-request passes), and a step driven by the
built tables: kda_chunk_prefill with the device-built cu_seqlens and slot
table gives bitwise the results of the same call with host-built ones."""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import DEV, layer_pair, new_cache, to_dev
from linear_attention_recurrent_kda_amd import api, synth
from oracle.kda_metadata import build_metadata

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def device_build(num_tokens, req_slot, n_slots):
    n = len(num_tokens)
    i32 = lambda a: torch.tensor(np.asarray(a, np.int32), dtype=torch.int32, device=DEV)
    cu = torch.full((n + 1,), -7, dtype=torch.int32, device=DEV)
    si = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    cs = torch.full((n + 1,), -7, dtype=torch.int32, device=DEV)
    ct = torch.full((4,), -7, dtype=torch.int32, device=DEV)
    ef = torch.zeros(1, dtype=torch.int32, device=DEV)
    api.kda_build_metadata(i32(num_tokens), i32(req_slot), n_slots, cu, si, cs, ct, ef)
    torch.cuda.synchronize()
    return cu.tolist(), si.tolist(), cs.tolist(), ct.tolist(), int(ef.item())


def test_hand_derived_batch():
    ex = json.load(open(os.path.join(GOLDEN, "kda_metadata_example.json")))
    got = device_build(ex["num_tokens"], ex["req_slot"], ex["n_slots"])
    e = ex["expected"]
    assert got == (e["cu_seqlens"], e["slot_idx"], e["chunk_start"], e["counts"], e["error"])


@pytest.mark.parametrize("n", [0, 1, 7, 64, 1000, 1024, 1025, 3000])
def test_random_batches_bit_exact(n):
    g = np.random.default_rng(2000 + n)
    n_slots = 4096
    num_tokens = g.choice([0, 1, 1, 1, 2, 17, 64, 65, 300, 4096], size=n).astype(np.int32)
    req_slot = g.permutation(n_slots)[:n].astype(np.int32)
    if n > 4:
        req_slot[g.integers(0, n, size=n // 5)] = -1
    ref = build_metadata(num_tokens.tolist(), req_slot.tolist(), n_slots)
    got = device_build(num_tokens, req_slot, n_slots)
    assert got == tuple(ref)


def test_errors_flagged_bit_exact():
    g = np.random.default_rng(7)
    n, n_slots = 1500, 100
    num_tokens = g.integers(-2, 70, size=n).astype(np.int32)
    req_slot = g.integers(-3, n_slots + 5, size=n).astype(np.int32)
    ref = build_metadata(num_tokens.tolist(), req_slot.tolist(), n_slots)
    assert ref[4] == 1
    assert device_build(num_tokens, req_slot, n_slots) == tuple(ref)


def test_built_tables_drive_a_mixed_prefill_step():
    g = synth.rng(2100)
    H, dk, dv, n_slots = 4, 128, 128, 12
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    num_tokens = np.array([1, 150, 0, 1, 64, 3, 1], np.int32)
    req_slot = np.array([5, 2, 7, 11, 0, -1, 9], np.int32)
    ref = build_metadata(num_tokens.tolist(), req_slot.tolist(), n_slots)
    total = ref[3][0]
    inp = synth.token_inputs(g, (total,), H, dk, dv, "bf16")
    I = api.Inputs(*(to_dev(inp[k], torch.bfloat16) for k in ("x_q", "x_k", "x_v", "g", "b", "z")))
    n = len(num_tokens)
    cu = torch.empty(n + 1, dtype=torch.int32, device=DEV)
    si = torch.empty(n, dtype=torch.int32, device=DEV)
    cs = torch.empty(n + 1, dtype=torch.int32, device=DEV)
    ct = torch.empty(4, dtype=torch.int32, device=DEV)
    api.kda_build_metadata(torch.from_numpy(num_tokens).to(DEV), torch.from_numpy(req_slot).to(DEV), n_slots,
                           cu, si, cs, ct)
    outs = []
    for tables in ((cu, si), (torch.tensor(ref[0], dtype=torch.int32, device=DEV),
                              torch.tensor(ref[1], dtype=torch.int32, device=DEV))):
        cache = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=31)
        y = torch.full((total, H, dv), 3.0, device=DEV)
        api.kda_chunk_prefill(dl, cache, tables[1], tables[0], I, y)
        torch.cuda.synchronize()
        outs.append((y, cache.state, cache.conv_state, cache.err_flag.item()))
    assert outs[0][3] == 0 and outs[1][3] == 0
    for a, b in zip(outs[0][:3], outs[1][:3]):
        assert torch.equal(a, b)
