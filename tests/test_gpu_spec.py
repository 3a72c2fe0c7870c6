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


@pytest.mark.parametrize("B,H", [(12, 8), (40, 32)])
@pytest.mark.parametrize("T", [8, 3, 16])
def test_verify_commit_equals_decode_bitwise(T, B, H):
    dl, _, cache, live, snaps, s0, w0, inp, g = setup_case(B, T, H=H, seed=800 + T + B)
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


# ---------------------------------------------------------------------------
# replayable-delta verification (kda_spec_verify_delta / kda_spec_commit_delta)
# ---------------------------------------------------------------------------
def _records(delta, dk, dv, dtype="bf16"):
    """Split a uint8 record buffer [B, T, H, rec] into (alpha, khat, d, x)."""
    raw = delta.cpu()
    nf = 2 * dk + dv
    f = raw[..., :4 * nf].contiguous().view(torch.float32).numpy().astype(np.float64)
    xb = raw[..., 4 * nf:].contiguous()
    x = xb.view(torch.bfloat16 if dtype == "bf16" else torch.float32).float().numpy().astype(np.float64)
    return f[..., :dk], f[..., dk:2 * dk], f[..., 2 * dk:], x


def test_verify_delta_matches_oracle_and_records():
    """Outputs equal the snapshot verification's bit for bit and match the
    oracle; every record holds the oracle's alpha, k^, beta (v - u) and the
    raw inputs; the commit reaches the oracle's state after L tokens."""
    from oracle.kda_oracle_np import core_sequential, preprocess
    B, T = 16, 8
    dl, ol, cache, live, snaps, s0, w0, inp, g = setup_case(B, T)
    lens = synth.accepted_lengths(g, B, T)
    lens[0], lens[1] = T, 1
    dlen = np.full(B, T, dtype=np.int32)
    dlen[2] = 5                                   # a shorter draft
    lens[2] = min(lens[2], 5)
    lt = torch.from_numpy(live).to(DEV)
    live_before = cache.state[lt.long()].clone()
    I = inputs_dev(inp, "bf16")
    ys = torch.empty((B, T, dl.H, dl.d_v), device=DEV)
    api.kda_spec_verify(dl, cache, lt, torch.from_numpy(snaps).to(DEV), I, ys,
                        draft_len=torch.from_numpy(dlen).to(DEV))
    delta = api.new_spec_delta(dl, B, T, torch.bfloat16, DEV).zero_()
    yd = torch.full((B, T, dl.H, dl.d_v), 7.0, device=DEV)
    api.kda_spec_verify_delta(dl, cache, lt, I, yd, delta, draft_len=torch.from_numpy(dlen).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(yd, ys)
    assert torch.equal(cache.state[lt.long()], live_before)
    orc = kda_oracle.run(ol, s0, w0, inp["x_q"], inp["x_k"], inp["x_v"], inp["g"], inp["b"], inp["z"],
                         lens=dlen, snapshots=True)
    yg = host(yd)
    worst = 0.0
    for t in range(T):
        rows = np.nonzero(dlen > t)[0]
        worst = max(worst, parity_error(yg[rows, t], orc["y"][rows, t]))
        assert np.all(yg[dlen <= t, t] == 0.0)
    print(f"  verify-delta parity max|d|/RMS = {worst:.3e}", flush=True)
    assert worst <= TOL
    # record contents against the oracle's per-token quantities
    qn, kn, v, log_alpha, beta, _ = preprocess(ol, w0, inp["x_q"], inp["x_k"], inp["x_v"], inp["g"], inp["b"])
    _, _, snap = core_sequential(qn, kn, v, log_alpha, beta, s0, snapshots=True)
    ra, rk, rd, rx = _records(delta, dl.d_k, dl.d_v)
    prev = np.concatenate([s0[:, None], snap[:, :-1]], axis=1)        # state before token t
    alpha = np.exp(log_alpha)
    u = np.einsum('bthij,bthi->bthj', alpha[..., None] * prev, kn)
    d_ref = beta[..., None] * (v - u)
    xin = np.concatenate([inp["x_q"], inp["x_k"], inp["x_v"]], axis=-1)
    for b in range(B):
        n = dlen[b]
        assert np.max(np.abs(ra[b, :n] - alpha[b, :n]) / alpha[b, :n]) < 1e-5
        assert np.max(np.abs(rk[b, :n] - kn[b, :n])) < 1e-5
        scale = np.sqrt(np.mean(d_ref[b, :n] ** 2))
        assert np.max(np.abs(rd[b, :n] - d_ref[b, :n])) < 1e-3 * scale
        assert np.array_equal(rx[b, :n], xin[b, :n])
    # commit the accepted prefixes: the oracle's state and window after L tokens
    api.kda_spec_commit_delta(dl, cache, lt, delta, torch.from_numpy(lens).to(DEV))
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 0
    for b in range(B):
        L = lens[b]
        sg = host(cache.state[int(live[b])])
        assert state_rel_err(sg[None], orc["snap_state"][b, L - 1][None]) < 1e-4
        assert np.array_equal(host(cache.conv_state[int(live[b])]), orc["snap_window"][b, L - 1])


# (12, 8): a grid within one round (lane-ordered token rows for T <= 8);
# (40, 32): 1280 workgroups, more than one round (per-row reads)
@pytest.mark.parametrize("B,H", [(12, 8), (40, 32)])
@pytest.mark.parametrize("T", [8, 3, 16])
@pytest.mark.parametrize("stream_state", [False, True])
def test_verify_delta_commit_equals_decode_bitwise(T, stream_state, B, H):
    dl, _, cache, live, snaps, s0, w0, inp, g = setup_case(B, T, H=H, seed=900 + T + B)
    dl.stream_state = stream_state
    acc = g.integers(0, T + 1, size=B).astype(np.int32)
    acc[0], acc[1] = 0, T
    ref = api.Cache(cache.state.clone(), cache.conv_state.clone(), torch.zeros_like(cache.err_flag))
    snap_c = api.Cache(cache.state.clone(), cache.conv_state.clone(), torch.zeros_like(cache.err_flag))
    lt = torch.from_numpy(live).to(DEV)
    st = torch.from_numpy(snaps).to(DEV)
    at = torch.from_numpy(acc).to(DEV)
    delta = api.new_spec_delta(dl, B, T, torch.bfloat16, DEV)
    y = torch.empty((B, T, dl.H, dl.d_v), device=DEV)
    api.kda_spec_verify_delta(dl, cache, lt, inputs_dev(inp, "bf16"), y, delta)
    api.kda_spec_commit_delta(dl, cache, lt, delta, at)
    # the snapshot form on a copy of the pools
    y2 = torch.empty_like(y)
    api.kda_spec_verify(dl, snap_c, lt, st, inputs_dev(inp, "bf16"), y2)
    api.kda_spec_commit(dl, snap_c, lt, st, at)
    # decode launches, sequence b stopping after acc[b] tokens
    for t in range(T):
        rows = np.nonzero(acc > t)[0]
        if len(rows) == 0:
            continue
        sub = {k: v[rows, t] for k, v in inp.items()}
        yt = torch.empty((len(rows), dl.H, dl.d_v), device=DEV)
        api.kda_decode(dl, ref, torch.from_numpy(live[rows].copy()).to(DEV), inputs_dev(sub, "bf16"), yt)
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 0
    assert torch.equal(y, y2)
    ll = lt.long()
    assert torch.equal(cache.state[ll], ref.state[ll])
    assert torch.equal(cache.conv_state[ll], ref.conv_state[ll])
    assert torch.equal(cache.state[ll], snap_c.state[ll])
    # nothing but the live slots changed
    others = torch.ones(cache.n_slots, dtype=torch.bool, device=DEV)
    others[ll] = False
    assert torch.equal(cache.state[others], ref.state[others])


def test_verify_delta_fp32_inputs_small_heads():
    """fp32 inputs and windows, d_k = 64, d_v = 128: commit equals decode bitwise."""
    B, T, H, dk, dv = 5, 4, 3, 64, 128
    g = synth.rng(960)
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    n_slots = 2 * B
    live = g.permutation(n_slots)[:B].astype(np.int32)
    s0 = synth.random_state(g, (B, H, dk, dv), 0.2)
    w0 = synth.window_inputs(g, (B,), H, dk, dv, "f32")
    inp = synth.token_inputs(g, (B, T), H, dk, dv, "f32")
    cache = new_cache(n_slots, H, dk, dv, "f32", fill_seed=22)
    lt = torch.from_numpy(live).to(DEV)
    cache.state[lt.long()] = torch.from_numpy(s0).to(DEV)
    cache.conv_state[lt.long()] = torch.from_numpy(w0).to(DEV)
    ref = api.Cache(cache.state.clone(), cache.conv_state.clone(), torch.zeros_like(cache.err_flag))
    acc = np.array([4, 0, 1, 2, 3], dtype=np.int32)
    delta = api.new_spec_delta(dl, B, T, torch.float32, DEV)
    y = torch.empty((B, T, H, dv), device=DEV)
    api.kda_spec_verify_delta(dl, cache, lt, inputs_dev(inp, "f32"), y, delta)
    api.kda_spec_commit_delta(dl, cache, lt, delta, torch.from_numpy(acc).to(DEV))
    for t in range(T):
        rows = np.nonzero(acc > t)[0]
        sub = {k: v[rows, t] for k, v in inp.items()}
        yt = torch.empty((len(rows), H, dv), device=DEV)
        api.kda_decode(dl, ref, torch.from_numpy(live[rows].copy()).to(DEV), inputs_dev(sub, "f32"), yt)
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 0
    assert torch.equal(cache.state, ref.state)
    assert torch.equal(cache.conv_state, ref.conv_state)


def test_commit_delta_errors_and_padding():
    B, T = 4, 4
    dl, _, cache, live, snaps, s0, w0, inp, g = setup_case(B, T, H=4, seed=930)
    lt = torch.from_numpy(live).to(DEV)
    delta = api.new_spec_delta(dl, B, T, torch.bfloat16, DEV)
    y = torch.empty((B, T, dl.H, dl.d_v), device=DEV)
    live_pad = live.copy()
    live_pad[3] = -1                       # padding row: zero outputs, nothing else
    api.kda_spec_verify_delta(dl, cache, torch.from_numpy(live_pad).to(DEV), inputs_dev(inp, "bf16"), y, delta)
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 0
    assert torch.all(y[3] == 0)
    before_s, before_w = cache.state.clone(), cache.conv_state.clone()
    acc = np.array([T + 1, 0, -1, 2], dtype=np.int32)  # rows 0, 2: bad lengths; row 1: no-op; row 3: padding
    api.kda_spec_commit_delta(dl, cache, torch.from_numpy(live_pad).to(DEV), delta, torch.from_numpy(acc).to(DEV))
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 1
    assert torch.equal(cache.state, before_s)
    assert torch.equal(cache.conv_state, before_w)
    # a sequence with no draft tokens: zero outputs, and its commit (L = 0) is a no-op
    dlen = np.array([0, T, 2, T], dtype=np.int32)
    y.fill_(5.0)
    api.kda_spec_verify_delta(dl, cache, lt, inputs_dev(inp, "bf16"), y, delta,
                              draft_len=torch.from_numpy(dlen).to(DEV))
    api.kda_spec_commit_delta(dl, cache, lt, delta, torch.from_numpy(np.array([0, 1, 2, 0], np.int32)).to(DEV))
    torch.cuda.synchronize()
    assert torch.all(y[0] == 0) and torch.all(y[2, 2:] == 0) and not torch.any(y[1] == 5.0)
    assert torch.equal(cache.state[int(live[0])], before_s[int(live[0])])
    assert torch.equal(cache.conv_state[int(live[3])], before_w[int(live[3])])
    assert cache.err_flag.item() == 1            # still set from the bad lengths above
    # a bad live slot in the verification flags and zeroes that row
    cache.err_flag.zero_()
    bad = live.copy()
    bad[0] = cache.n_slots + 3
    api.kda_spec_verify_delta(dl, cache, torch.from_numpy(bad).to(DEV), inputs_dev(inp, "bf16"), y, delta)
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 1
    assert torch.all(y[0] == 0)
