"""api.prepared(): a call checked and marshalled once, then re-issued, gives
bitwise the results of the same direct calls (spec-verify with replay records
and its commit, repeated; chunked prefill with a workspace the binding
allocates, which the prepared call must keep alive)."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, inputs_dev, layer_pair, new_cache
from linear_attention_recurrent_kda_amd import api, synth

pytestmark = pytest.mark.gpu


def test_prepared_spec_delta_equals_direct_calls():
    B, T, H, dk, dv = 6, 4, 4, 128, 128
    g = synth.rng(4100)
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    inp = [synth.token_inputs(g, (B, T), H, dk, dv, "bf16") for _ in range(3)]
    acc = torch.from_numpy(g.integers(0, T + 1, size=B).astype(np.int32)).to(DEV)
    live = torch.arange(B, dtype=torch.int32, device=DEV)
    results = []
    for use_prepared in (False, True):
        cache = new_cache(B, H, dk, dv, "bf16", fill_seed=41)
        delta = api.new_spec_delta(dl, B, T, torch.bfloat16, DEV)
        y = torch.empty((B, T, H, dv), device=DEV)
        ys = []
        I = inputs_dev(inp[0], "bf16")
        if use_prepared:
            verify = api.prepared(api.kda_spec_verify_delta, dl, cache, live, I, y, delta)
            commit = api.prepared(api.kda_spec_commit_delta, dl, cache, live, delta, acc)
        for step in range(3):
            # new inputs copied into the buffers the prepared calls captured
            src = inputs_dev(inp[step], "bf16")
            for k in ("x_q", "x_k", "x_v", "g", "b", "z"):
                getattr(I, k).copy_(getattr(src, k))
            if use_prepared:
                verify()
                commit()
            else:
                api.kda_spec_verify_delta(dl, cache, live, I, y, delta)
                api.kda_spec_commit_delta(dl, cache, live, delta, acc)
            ys.append(y.clone())
        torch.cuda.synchronize()
        results.append((ys, cache.state.clone(), cache.conv_state.clone()))
    (ya, sa, wa), (yb, sb, wb) = results
    for a, b in zip(ya, yb):
        assert torch.equal(a, b)
    assert torch.equal(sa, sb) and torch.equal(wa, wb)


def test_prepared_prefill_keeps_its_workspace():
    H, dk, dv, T = 4, 64, 64, 200
    g = synth.rng(4200)
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    inp = synth.token_inputs(g, (T,), H, dk, dv, "bf16")
    cu = torch.tensor([0, 70, T], dtype=torch.int32, device=DEV)
    sl = torch.tensor([1, 0], dtype=torch.int32, device=DEV)
    out = []
    for use_prepared in (False, True):
        cache = new_cache(2, H, dk, dv, "bf16", fill_seed=42)
        y = torch.empty((T, H, dv), device=DEV)
        I = inputs_dev(inp, "bf16")
        if use_prepared:
            run = api.prepared(api.kda_chunk_prefill, dl, cache, sl, cu, I, y)   # workspace allocated inside
            torch.cuda.synchronize()
            # had the workspace been freed, this allocation could take its
            # memory and the runs would overwrite it
            junk = torch.full((1 << 22,), 7, dtype=torch.uint8, device=DEV)
            run()
            run()
            torch.cuda.synchronize()
            assert bool((junk == 7).all())
        else:
            api.kda_chunk_prefill(dl, cache, sl, cu, I, y)
            api.kda_chunk_prefill(dl, cache, sl, cu, I, y)
        torch.cuda.synchronize()
        out.append((y.clone(), cache.state.clone(), cache.conv_state.clone()))
    for a, b in zip(*out):
        assert torch.equal(a, b)
