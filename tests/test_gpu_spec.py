"""GPU parity of kda_spec_verify / kda_spec_commit: against the oracle (outputs
and per-token snapshots) and, bit for bit, against decode launches."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, TOL, host, inputs_dev, layer_pair, new_cache, parity_error, state_rel_err
from linear_attention_recurrent_kda_amd import api, synth
from oracle import kda_oracle

pytestmark = pytest.mark.gpu


def setup_case(B, T, H=32, dk=128, dv=128, seed=None, dtype="bf16"):
    cfg = synth.WORKLOADS["spec_verify_b16_t8"]
    g = synth.rng(cfg["seed"] if seed is None else seed)
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    # live slots [0, B), snapshot slots [B, B + B*T), a seeded permutation of them
    n_slots = B + B * T + 3
    perm = g.permutation(n_slots - 3).astype(np.int32)
    live = perm[:B].copy()
    snaps = perm[B:].reshape(B, T).copy()
    s0 = synth.random_state(g, (B, H, dk, dv), 0.2)
    w0 = synth.window_inputs(g, (B,), H, dk, dv, dtype)
    inp = synth.token_inputs(g, (B, T), H, dk, dv, dtype)
    cache = new_cache(n_slots, H, dk, dv, dtype, fill_seed=21)
    lt = torch.from_numpy(live).to(DEV)
    cache.state[lt.long()] = torch.from_numpy(s0).to(DEV)
    cache.conv_state[lt.long()] = torch.from_numpy(w0).to(DEV).to(cache.conv_state.dtype)
    return dl, ol, cache, live, snaps, s0, w0, inp, g


def test_verify_matches_oracle_outputs_and_snapshots():
    B, T = 16, 8
    dl, ol, cache, live, snaps, s0, w0, inp, g = setup_case(B, T)
    lens = synth.accepted_lengths(g, B, T)
    lens[0], lens[1] = T, 1
    live_before = cache.state[torch.from_numpy(live).long().to(DEV)].clone()
    y = torch.full((B, T, dl.H, dl.d_v), 9.0, device=DEV)
    api.kda_spec_verify(dl, cache, torch.from_numpy(live).to(DEV), torch.from_numpy(snaps).to(DEV),
                        inputs_dev(inp, "bf16"), y, draft_len=torch.from_numpy(lens).to(DEV))
    torch.cuda.synchronize()
    orc = kda_oracle.run(ol, s0, w0, inp["x_q"], inp["x_k"], inp["x_v"], inp["g"], inp["b"], inp["z"],
                         lens=lens, snapshots=True)
    yg = host(y)
    worst = 0.0
    for t in range(T):
        rows = np.nonzero(lens > t)[0]
        worst = max(worst, parity_error(yg[rows, t], orc["y"][rows, t]))
        for bi in np.nonzero(lens <= t)[0]:
            assert np.all(yg[bi, t] == 0.0)
        sg = host(cache.state[torch.from_numpy(snaps[rows, t]).long().to(DEV)])
        assert state_rel_err(sg, orc["snap_state"][rows, t]) < 1e-4
        wg = host(cache.conv_state[torch.from_numpy(snaps[rows, t]).long().to(DEV)])
        assert np.array_equal(wg, orc["snap_window"][rows, t])
    print(f"  verify parity max|d|/RMS = {worst:.3e}", flush=True)
    assert worst <= TOL
    # the live slots are not modified
    assert torch.equal(cache.state[torch.from_numpy(live).long().to(DEV)], live_before)
    assert cache.err_flag.item() == 0


@pytest.mark.parametrize("T", [8, 3, 16])
def test_verify_commit_equals_decode_bitwise(T):
    B = 12
    dl, _, cache, live, snaps, s0, w0, inp, g = setup_case(B, T, H=8, seed=800 + T)
    acc = g.integers(0, T + 1, size=B).astype(np.int32)
    acc[0], acc[1] = 0, T
    ref = api.Cache(cache.state.clone(), cache.conv_state.clone(), torch.zeros_like(cache.err_flag))
    lt = torch.from_numpy(live).to(DEV)
    y = torch.empty((B, T, dl.H, dl.d_v), device=DEV)
    api.kda_spec_verify(dl, cache, lt, torch.from_numpy(snaps).to(DEV), inputs_dev(inp, "bf16"), y)
    api.kda_spec_commit(dl, cache, lt, torch.from_numpy(snaps).to(DEV), torch.from_numpy(acc).to(DEV))
    # reference: decode launches, sequence b stopping after acc[b] tokens
    yd = torch.zeros_like(y)
    for t in range(T):
        rows = np.nonzero(acc > t)[0]
        if len(rows) == 0:
            continue
        sub = {k: v[rows, t] for k, v in inp.items()}
        yt = torch.empty((len(rows), dl.H, dl.d_v), device=DEV)
        api.kda_decode(dl, ref, torch.from_numpy(live[rows].copy()).to(DEV), inputs_dev(sub, "bf16"), yt)
        yd[torch.from_numpy(rows).long().to(DEV), t] = yt
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 0
    ll = lt.long()
    assert torch.equal(cache.state[ll], ref.state[ll])
    assert torch.equal(cache.conv_state[ll], ref.conv_state[ll])
    for bi in range(B):
        assert torch.equal(y[bi, :acc[bi]], yd[bi, :acc[bi]])


def test_commit_errors_and_padding():
    B, T = 4, 4
    dl, _, cache, live, snaps, s0, w0, inp, g = setup_case(B, T, H=4, seed=830)
    snaps[2, 1] = -1                       # snapshot of token 1 not kept
    y = torch.empty((B, T, dl.H, dl.d_v), device=DEV)
    lt = torch.from_numpy(live).to(DEV)
    st = torch.from_numpy(snaps).to(DEV)
    api.kda_spec_verify(dl, cache, lt, st, inputs_dev(inp, "bf16"), y)
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 0
    before = cache.state.clone()
    live_pad = live.copy()
    live_pad[3] = -1                       # padding row: nothing happens
    acc = np.array([T + 1, 0, 2, 2], dtype=np.int32)   # row 0: bad length; row 2: needs the -1 snapshot
    api.kda_spec_commit(dl, cache, torch.from_numpy(live_pad).to(DEV), st, torch.from_numpy(acc).to(DEV))
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 1
    assert torch.equal(cache.state, before)


def test_verify_bad_snapshot_slot_flags_error():
    B, T = 2, 3
    dl, _, cache, live, snaps, s0, w0, inp, g = setup_case(B, T, H=2, seed=840)
    snaps[1, 2] = cache.n_slots + 5
    y = torch.empty((B, T, dl.H, dl.d_v), device=DEV)
    api.kda_spec_verify(dl, cache, torch.from_numpy(live).to(DEV), torch.from_numpy(snaps).to(DEV),
                        inputs_dev(inp, "bf16"), y)
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 1
