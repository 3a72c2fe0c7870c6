"""KDA_CHECK=1 debug validation: slot tables copied to the host and checked
for aliasing (two rows on one slot, snapshot or checkpoint slots on live
slots or on each other) and out-of-range entries before anything launches;
valid calls give the same results as without the check."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, inputs_dev, layer_pair, new_cache
from linear_attention_recurrent_kda_amd import api, synth

pytestmark = pytest.mark.gpu

ALIAS, SHAPE = 8, 2


def _case(B=3, T=2, H=2, dk=64, dv=64, n_slots=12):
    g = synth.rng(1600)
    dl, _ = layer_pair(synth.layer_params(g, H, dk, dv))
    inp1 = synth.token_inputs(g, (B,), H, dk, dv, "bf16")
    inpT = synth.token_inputs(g, (B, T), H, dk, dv, "bf16")
    cache = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=16)
    return dl, inp1, inpT, cache


def _code(fn):
    try:
        fn()
    except api.KdaError as e:
        return e.code
    return 0


def test_check_decode_and_verify(monkeypatch):
    dl, inp1, inpT, cache = _case()
    t = lambda a: torch.tensor(a, dtype=torch.int32, device=DEV)
    y = torch.empty((3, dl.H, dl.d_v), device=DEV)
    yT = torch.empty((3, 2, dl.H, dl.d_v), device=DEV)
    # reference result of a valid call, without the check
    ref = api.Cache(cache.state.clone(), cache.conv_state.clone(), torch.zeros_like(cache.err_flag))
    yr = torch.empty_like(y)
    api.kda_decode(dl, ref, t([4, 7, 1]), inputs_dev(inp1, "bf16"), yr)
    monkeypatch.setenv("KDA_CHECK", "1")
    before = cache.state.clone()
    assert _code(lambda: api.kda_decode(dl, cache, t([4, 7, 4]), inputs_dev(inp1, "bf16"), y)) == ALIAS
    assert _code(lambda: api.kda_decode(dl, cache, t([4, 7, 12]), inputs_dev(inp1, "bf16"), y)) == SHAPE
    torch.cuda.synchronize()
    assert torch.equal(cache.state, before)                 # nothing launched
    assert _code(lambda: api.kda_decode(dl, cache, t([4, 7, 1]), inputs_dev(inp1, "bf16"), y)) == 0
    assert _code(lambda: api.kda_decode(dl, cache, t([4, -1, -1]), inputs_dev(inp1, "bf16"), y)) == 0
    torch.cuda.synchronize()
    # padding rows repeat -1 without aliasing; the valid call matches the unchecked one
    api.kda_decode(dl, ref, t([4, -1, -1]), inputs_dev(inp1, "bf16"), yr)
    torch.cuda.synchronize()
    assert torch.equal(cache.state, ref.state)
    # verify: a snapshot slot on a live slot, or two snapshots on one slot
    snaps = lambda a: torch.tensor(a, dtype=torch.int32, device=DEV).reshape(3, 2)
    I = inputs_dev(inpT, "bf16")
    assert _code(lambda: api.kda_spec_verify(dl, cache, t([0, 1, 2]), snaps([3, 4, 5, 6, 7, 1]), I, yT)) == ALIAS
    assert _code(lambda: api.kda_spec_verify(dl, cache, t([0, 1, 2]), snaps([3, 4, 5, 6, 7, 3]), I, yT)) == ALIAS
    assert _code(lambda: api.kda_spec_verify(dl, cache, t([0, 1, 2]), snaps([3, 4, 5, 6, 7, -1]), I, yT)) == 0
    acc = t([1, 2, 0])
    assert _code(lambda: api.kda_spec_commit(dl, cache, t([0, 1, 2]), snaps([3, 4, 5, 6, 2, 8]), acc)) == ALIAS
    assert _code(lambda: api.kda_spec_commit(dl, cache, t([0, 1, 2]), snaps([3, 4, 5, 6, 7, -1]), acc)) == 0
    delta = api.new_spec_delta(dl, 3, 2, torch.bfloat16, DEV)
    assert _code(lambda: api.kda_spec_verify_delta(dl, cache, t([0, 0, 2]), I, yT, delta)) == ALIAS
    assert _code(lambda: api.kda_spec_commit_delta(dl, cache, t([5, 6, 5]), delta, acc)) == ALIAS
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 0


def test_check_prefill(monkeypatch):
    dl, inp1, inpT, cache = _case()
    g = synth.rng(1601)
    inp = synth.token_inputs(g, (130,), dl.H, dl.d_k, dl.d_v, "bf16")
    I = inputs_dev(inp, "bf16")
    y = torch.empty((130, dl.H, dl.d_v), device=DEV)
    cu = torch.tensor([0, 65, 130], dtype=torch.int32, device=DEV)
    t = lambda a: torch.tensor(a, dtype=torch.int32, device=DEV)
    monkeypatch.setenv("KDA_CHECK", "1")
    assert _code(lambda: api.kda_chunk_prefill(dl, cache, t([3, 3]), cu, I, y)) == ALIAS
    assert _code(lambda: api.kda_chunk_prefill_ckpt(dl, cache, t([3, 4]), cu, I, y, t([[5], [3]]), 64)) == ALIAS
    assert _code(lambda: api.kda_chunk_prefill_ckpt(dl, cache, t([3, 4]), cu, I, y, t([[5], [5]]), 64)) == ALIAS
    assert _code(lambda: api.kda_chunk_prefill_ckpt(dl, cache, t([3, 4]), cu, I, y, t([[5], [6]]), 64)) == 0
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 0
