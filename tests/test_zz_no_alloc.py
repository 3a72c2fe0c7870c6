"""kda_chunk_prefill_static (no allocation: the workspace is the library's
static device array) against kda_chunk_prefill with a caller workspace:
bitwise the same outputs, states and windows, on two calls in a row, the
second one smaller, through the C ABI."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, layer_pair, new_cache, to_dev
from linear_attention_recurrent_kda_amd import _lib, api, synth

pytestmark = pytest.mark.gpu

KEYS = ("x_q", "x_k", "x_v", "g", "b", "z")


def one_call(dl, lens, slots, inp, n_slots, H, dk, dv):
    I = api.Inputs(*(to_dev(inp[k], torch.bfloat16) for k in KEYS))
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(DEV)
    sl = torch.from_numpy(np.asarray(slots, np.int32)).to(DEV)
    total = int(sum(lens))
    outs = []
    for static in (True, False):
        cache = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=41)
        y = torch.full((total, H, dv), 5.0, device=DEV)
        if static:
            api.kda_chunk_prefill_static(dl, cache, sl, cu, I, y)
        else:
            ws = torch.empty(api.kda_chunk_prefill_workspace_bytes(dl, total, len(lens)), dtype=torch.uint8,
                             device=DEV)
            api.kda_chunk_prefill(dl, cache, sl, cu, I, y, ws)
        torch.cuda.synchronize()
        outs.append((y, cache.state, cache.conv_state, cache.err_flag.item()))
    assert outs[0][3] == 0 and outs[1][3] == 0
    for a, b in zip(outs[0][:3], outs[1][:3]):
        assert torch.equal(a, b)


def test_static_prefill_equals_workspace_prefill_twice():
    g = synth.rng(3100)
    H, dk, dv, n_slots = 32, 128, 128, 8
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    # first call: three prompts and a one-token row (1341 tokens)
    lens = [700, 1, 513, 127]
    one_call(dl, lens, [3, 0, 6, 1], synth.token_inputs(g, (sum(lens),), H, dk, dv, "bf16"), n_slots, H, dk, dv)
    # second call, smaller: one prompt
    one_call(dl, [90], [5], synth.token_inputs(g, (90,), H, dk, dv, "bf16"), n_slots, H, dk, dv)


def test_static_prefill_rejects_calls_beyond_the_array():
    g = synth.rng(3101)
    H, dk, dv = 32, 128, 128
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    T = 4096   # at H = 32, d = 128 this needs more than the static array
    assert api.kda_chunk_prefill_workspace_bytes(dl, T, 1) > _lib.KDA_STATIC_WORKSPACE_BYTES
    inp = synth.token_inputs(g, (T,), H, dk, dv, "bf16")
    cache = new_cache(2, H, dk, dv, "bf16")
    y = torch.empty((T, H, dv), device=DEV)
    with pytest.raises(api.KdaError) as e:
        api.kda_chunk_prefill_static(dl, cache, torch.zeros(1, dtype=torch.int32, device=DEV),
                                     torch.tensor([0, T], dtype=torch.int32, device=DEV),
                                     api.Inputs(*(to_dev(inp[k], torch.bfloat16) for k in KEYS)), y)
    assert e.value.status == "KDA_ERR_WORKSPACE"
