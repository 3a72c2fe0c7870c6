"""GPU parity of kda_decode against the fp64 oracle, slot-table exactness,
padding and error rows, invariants through the full pipeline, determinism.

Tolerance: max |GPU - oracle| <= 2e-3 * RMS(oracle output), checked at every
step (RMS over that step's whole output tensor)."""
import numpy as np
import pytest
import torch

from gpu_util import (DEV, TOL, host, inputs_dev, layer_pair, new_cache, parity_error,
                      state_rel_err, tdt, to_dev)
from linear_attention_recurrent_kda_amd import api, synth
from oracle import kda_oracle

pytestmark = pytest.mark.gpu


def run_decode_steps(dl, cache, slots_t, inp, dtype, steps, B):
    """`steps` decode launches; inp arrays are [steps, B, H, .]. Returns y [steps, B, H, d_v]."""
    dev_inp = {k: to_dev(inp[k], tdt(dtype)) for k in ("x_q", "x_k", "x_v", "g", "b", "z")}
    ys = torch.empty((steps, B, dl.H, dl.d_v), dtype=torch.float32, device=DEV)
    for t in range(steps):
        I = api.Inputs(*(dev_inp[k][t] for k in ("x_q", "x_k", "x_v", "g", "b", "z")))
        api.kda_decode(dl, cache, slots_t, I, ys[t])
    torch.cuda.synchronize()
    return host(ys)


def oracle_steps(ol, state0, win0, inp, steps):
    """Oracle over `steps` tokens for inputs laid out [steps, B, ...]."""
    tb = {k: np.swapaxes(inp[k][:steps], 0, 1) for k in inp}     # -> [B, steps, ...]
    out = kda_oracle.run(ol, state0, win0, tb["x_q"], tb["x_k"], tb["x_v"], tb["g"], tb["b"], tb["z"])
    return np.swapaxes(out["y"], 0, 1), out["state"], out["window"]


def assert_per_step(y_gpu, y_orc, tol=TOL):
    errs = [parity_error(y_gpu[t], y_orc[t]) for t in range(y_gpu.shape[0])]
    worst = int(np.argmax(errs))
    print(f"  parity: worst step {worst} max|d|/RMS = {errs[worst]:.3e} (tol {tol})", flush=True)
    assert errs[worst] <= tol, f"step {worst}: {errs[worst]:.3e} > {tol}"


def test_tiny_recurrence_1000_steps():
    """B=1, H=4, d_k=d_v=64, fp32 inputs, 1000 steps from a zero state."""
    cfg = synth.WORKLOADS["tiny_recurrence"]
    g = synth.rng(cfg["seed"])
    H, dk, dv, steps = cfg["H"], cfg["d_k"], cfg["d_v"], 1000
    params = synth.layer_params(g, H, dk, dv)
    inp = synth.token_inputs(g, (steps, 1), H, dk, dv, "f32")
    dl, ol = layer_pair(params)
    cache = new_cache(4, H, dk, dv, "f32")
    slots = torch.tensor([2], dtype=torch.int32, device=DEV)
    y = run_decode_steps(dl, cache, slots, inp, "f32", steps, 1)
    yo, so, wo = oracle_steps(ol, np.zeros((1, H, dk, dv)), np.zeros((1, H, 3, 2 * dk + dv)), inp, steps)
    assert_per_step(y, yo)
    assert state_rel_err(host(cache.state[2:3]), so) < 1e-3
    assert np.array_equal(host(cache.conv_state[2:3]), wo)
    assert cache.err_flag.item() == 0


def test_decode_b1_from_warm_state():
    """B=1, H=32, d=128, bf16 inputs, a 256-slot pool, state warmed up by 512
    oracle steps and rounded to fp32, then 200 decode steps."""
    cfg = synth.WORKLOADS["decode_b1"]
    g = synth.rng(cfg["seed"])
    H, dk, dv, n_slots = cfg["H"], cfg["d_k"], cfg["d_v"], cfg["n_slots"]
    params = synth.layer_params(g, H, dk, dv)
    slot = int(synth.slot_table(g, 1, n_slots)[0])
    warm = synth.token_inputs(g, (1, cfg["warmup"]), H, dk, dv, "bf16")
    dl, ol = layer_pair(params)
    w = kda_oracle.run(ol, np.zeros((1, H, dk, dv)), np.zeros((1, H, 3, 2 * dk + dv)),
                       warm["x_q"], warm["x_k"], warm["x_v"], warm["g"], warm["b"], warm["z"],
                       y_tokens=0)
    s32 = w["state"].astype(np.float32)
    cache = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=7)
    cache.state[slot] = to_dev(s32[0])
    cache.conv_state[slot] = to_dev(w["window"][0], torch.bfloat16)
    steps = 200
    inp = synth.token_inputs(g, (steps, 1), H, dk, dv, "bf16")
    slots = torch.tensor([slot], dtype=torch.int32, device=DEV)
    y = run_decode_steps(dl, cache, slots, inp, "bf16", steps, 1)
    yo, so, wo = oracle_steps(ol, s32.astype(np.float64), w["window"], inp, steps)
    assert_per_step(y, yo)
    assert state_rel_err(host(cache.state[slot:slot + 1]), so) < 1e-3
    assert np.array_equal(host(cache.conv_state[slot:slot + 1]), wo)


def _b64_setup(seed_offset=0):
    cfg = synth.WORKLOADS["decode_b64"]
    g = synth.rng(cfg["seed"] + seed_offset)
    H, dk, dv, B, n_slots = cfg["H"], cfg["d_k"], cfg["d_v"], cfg["B"], cfg["n_slots"]
    params = synth.layer_params(g, H, dk, dv)
    slots = synth.slot_table(g, B, n_slots)
    return cfg, g, params, slots


def test_decode_b64_100_steps_all_sequences():
    """B=64 in a 1024-slot pool addressed by a random slot table: 10 GPU warm-up
    steps from zero, then 100 steps compared with the oracle started from the
    GPU's fp32 state."""
    cfg, g, params, slots = _b64_setup()
    H, dk, dv, B, n_slots = cfg["H"], cfg["d_k"], cfg["d_v"], cfg["B"], cfg["n_slots"]
    dl, ol = layer_pair(params)
    cache = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=11)
    st = torch.from_numpy(slots).to(DEV)
    cache.state[st.long()] = 0.0
    cache.conv_state[st.long()] = 0
    warm = synth.token_inputs(g, (10, B), H, dk, dv, "bf16")
    run_decode_steps(dl, cache, st, warm, "bf16", 10, B)
    s0 = host(cache.state[st.long()])
    w0 = host(cache.conv_state[st.long()])
    steps = 100
    inp = synth.token_inputs(g, (steps, B), H, dk, dv, "bf16")
    y = run_decode_steps(dl, cache, st, inp, "bf16", steps, B)
    yo, so, wo = oracle_steps(ol, s0, w0, inp, steps)
    assert_per_step(y, yo)
    assert state_rel_err(host(cache.state[st.long()]), so) < 1e-3
    assert np.array_equal(host(cache.conv_state[st.long()]), wo)
    assert cache.err_flag.item() == 0


def test_decode_b64_1000_steps_four_sequences():
    """The 1000-step horizon at the batched shape: all 64 sequences run on the
    GPU from zero, 4 of them are checked against the oracle at every step."""
    cfg, g, params, slots = _b64_setup(1000)
    H, dk, dv, B, n_slots = cfg["H"], cfg["d_k"], cfg["d_v"], cfg["B"], cfg["n_slots"]
    dl, ol = layer_pair(params)
    cache = new_cache(n_slots, H, dk, dv, "bf16")
    st = torch.from_numpy(slots).to(DEV)
    steps = 1000
    inp = synth.token_inputs(g, (steps, B), H, dk, dv, "bf16")
    y = run_decode_steps(dl, cache, st, inp, "bf16", steps, B)
    pick = [0, 17, 42, 63]
    sub = {k: v[:, pick] for k, v in inp.items()}
    yo, so, _ = oracle_steps(ol, np.zeros((4, H, dk, dv)), np.zeros((4, H, 3, 2 * dk + dv)), sub, steps)
    assert_per_step(y[:, pick], yo)
    assert state_rel_err(host(cache.state[st[pick].long()]), so) < 1e-3


@pytest.mark.parametrize("dk,dv,dtype", [(64, 128, "bf16"), (128, 64, "f32"), (64, 64, "bf16")])
def test_other_head_sizes(dk, dv, dtype):
    g = synth.rng(500 + dk + dv)
    H, B, steps = 3, 5, 40
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    cache = new_cache(8, H, dk, dv, dtype)
    slots = np.array([6, 1, 3, 0, 7], dtype=np.int32)
    st = torch.from_numpy(slots).to(DEV)
    inp = synth.token_inputs(g, (steps, B), H, dk, dv, dtype)
    y = run_decode_steps(dl, cache, st, inp, dtype, steps, B)
    yo, so, wo = oracle_steps(ol, np.zeros((B, H, dk, dv)), np.zeros((B, H, 3, 2 * dk + dv)), inp, steps)
    assert_per_step(y, yo)
    assert state_rel_err(host(cache.state[st.long()]), so) < 1e-3
    assert np.array_equal(host(cache.conv_state[st.long()]), wo)


@pytest.mark.parametrize("silu,q_scale,rms_eps", [(False, None, 1e-6), (True, 0.3, 0.05)])
def test_layer_options(silu, q_scale, rms_eps):
    g = synth.rng(600)
    H, dk, dv, B, steps = 2, 128, 128, 3, 30
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params, q_scale=q_scale, rms_eps=rms_eps, silu=silu)
    cache = new_cache(3, H, dk, dv, "bf16")
    st = torch.tensor([2, 0, 1], dtype=torch.int32, device=DEV)
    inp = synth.token_inputs(g, (steps, B), H, dk, dv, "bf16")
    y = run_decode_steps(dl, cache, st, inp, "bf16", steps, B)
    yo, _, _ = oracle_steps(ol, np.zeros((B, H, dk, dv)), np.zeros((B, H, 3, 2 * dk + dv)), inp, steps)
    assert_per_step(y, yo)


# ---------------------------------------------------------------------------
# slots: bit-exact indexing, padding, errors
# ---------------------------------------------------------------------------
def _slot_case(B=8, n_slots=32, H=4, dk=128, dv=128, seed=700):
    g = synth.rng(seed)
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    inp = synth.token_inputs(g, (B,), H, dk, dv, "bf16")
    slots = synth.slot_table(g, B, n_slots)
    return dl, ol, inp, slots


def test_untouched_slots_bitwise_identical():
    dl, _, inp, slots = _slot_case()
    cache = new_cache(32, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=3)
    before_s, before_w = cache.state.clone(), cache.conv_state.clone()
    y = torch.empty((8, dl.H, dl.d_v), device=DEV)
    api.kda_decode(dl, cache, torch.from_numpy(slots).to(DEV), inputs_dev(inp, "bf16"), y)
    torch.cuda.synchronize()
    touched = np.zeros(32, bool)
    touched[slots] = True
    for s in range(32):
        same_s = torch.equal(cache.state[s], before_s[s])
        same_w = torch.equal(cache.conv_state[s], before_w[s])
        assert (same_s and same_w) != touched[s], f"slot {s}"


def test_permuted_batch_permutes_results_bitwise():
    dl, _, inp, slots = _slot_case()
    c1 = new_cache(32, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=4)
    c2 = new_cache(32, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=4)
    y1 = torch.empty((8, dl.H, dl.d_v), device=DEV)
    y2 = torch.empty_like(y1)
    api.kda_decode(dl, c1, torch.from_numpy(slots).to(DEV), inputs_dev(inp, "bf16"), y1)
    perm = np.random.default_rng(1).permutation(8)
    pinp = {k: v[perm] for k, v in inp.items()}
    api.kda_decode(dl, c2, torch.from_numpy(slots[perm].copy()).to(DEV), inputs_dev(pinp, "bf16"), y2)
    torch.cuda.synchronize()
    assert torch.equal(y2, y1[torch.from_numpy(perm).to(DEV)])
    assert torch.equal(c1.state, c2.state) and torch.equal(c1.conv_state, c2.conv_state)


def test_sequence_result_independent_of_batch():
    dl, _, inp, slots = _slot_case()
    c1 = new_cache(32, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=5)
    c2 = new_cache(32, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=5)
    y1 = torch.empty((8, dl.H, dl.d_v), device=DEV)
    api.kda_decode(dl, c1, torch.from_numpy(slots).to(DEV), inputs_dev(inp, "bf16"), y1)
    b = 5
    y2 = torch.empty((1, dl.H, dl.d_v), device=DEV)
    api.kda_decode(dl, c2, torch.from_numpy(slots[b:b + 1].copy()).to(DEV),
                   inputs_dev(inp, "bf16", slice(b, b + 1)), y2)
    torch.cuda.synchronize()
    s = int(slots[b])
    assert torch.equal(y2[0], y1[b])
    assert torch.equal(c2.state[s], c1.state[s]) and torch.equal(c2.conv_state[s], c1.conv_state[s])


def test_padding_and_out_of_range_rows():
    dl, ol, inp, slots = _slot_case()
    cache = new_cache(32, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=6)
    ref = new_cache(32, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=6)
    bad = slots.copy()
    bad[1] = -1          # padding
    bad[4] = 32          # out of range (== n_slots)
    bad[6] = -7          # out of range (negative)
    y = torch.full((8, dl.H, dl.d_v), 123.0, device=DEV)
    api.kda_decode(dl, cache, torch.from_numpy(bad).to(DEV), inputs_dev(inp, "bf16"), y)
    keep = [0, 2, 3, 5, 7]
    yr = torch.empty((5, dl.H, dl.d_v), device=DEV)
    api.kda_decode(dl, ref, torch.from_numpy(slots[keep].copy()).to(DEV),
                   inputs_dev(inp, "bf16", keep), yr)
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 1
    assert ref.err_flag.item() == 0
    for r in (1, 4, 6):
        assert torch.count_nonzero(y[r]) == 0
    assert torch.equal(y[keep], yr)
    assert torch.equal(cache.state, ref.state) and torch.equal(cache.conv_state, ref.conv_state)


def test_zero_batch_is_noop():
    dl, _, inp, _ = _slot_case(B=1)
    cache = new_cache(4, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=8)
    before = cache.state.clone()
    empty = {k: v[:0] for k, v in inp.items()}
    api.kda_decode(dl, cache, torch.empty(0, dtype=torch.int32, device=DEV),
                   inputs_dev(empty, "bf16"), torch.empty((0, dl.H, dl.d_v), device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(cache.state, before)


# ---------------------------------------------------------------------------
# invariants through the whole pipeline
# ---------------------------------------------------------------------------
def test_beta_zero_alpha_one_state_bitwise():
    """b = -inf (beta = 0) and g = -inf (softplus 0, alpha = 1): the state is
    bitwise unchanged (bf16 infinities)."""
    dl, _, inp, slots = _slot_case(seed=710)
    inp = dict(inp, b=np.full_like(inp["b"], -np.inf), g=np.full_like(inp["g"], -np.inf))
    cache = new_cache(32, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=9)
    before = cache.state.clone()
    y = torch.empty((8, dl.H, dl.d_v), device=DEV)
    api.kda_decode(dl, cache, torch.from_numpy(slots).to(DEV), inputs_dev(inp, "bf16"), y)
    torch.cuda.synchronize()
    assert torch.equal(cache.state, before)


def test_q_equals_k_beta_one_reads_back_value():
    """beta = 1, same q and k inputs and taps, scale 1, eps 0: o = S^T k^ = v
    after the update, so y = RMSNorm(v) * sigmoid(z).  Checked against the
    oracle, which pins the same identity."""
    g = synth.rng(720)
    H, dk, dv, B = 4, 128, 128, 6
    params = synth.layer_params(g, H, dk, dv)
    params["conv_wt"][:, dk:2 * dk] = params["conv_wt"][:, :dk]
    dl, ol = layer_pair(params, q_scale=1.0, l2_eps=0.0)
    inp = synth.token_inputs(g, (1, B), H, dk, dv, "bf16")
    inp["x_k"] = inp["x_q"].copy()
    inp["b"] = np.full_like(inp["b"], np.inf)
    cache = new_cache(B, H, dk, dv, "bf16")
    st = torch.arange(B, dtype=torch.int32, device=DEV)
    y = run_decode_steps(dl, cache, st, inp, "bf16", 1, B)
    yo, _, _ = oracle_steps(ol, np.zeros((B, H, dk, dv)), np.zeros((B, H, 3, 2 * dk + dv)), inp, 1)
    assert_per_step(y, yo)


def test_repeated_runs_bitwise_identical():
    dl, _, inp, slots = _slot_case(seed=730)
    outs = []
    for _ in range(2):
        cache = new_cache(32, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=10)
        y = torch.empty((8, dl.H, dl.d_v), device=DEV)
        for _ in range(3):
            api.kda_decode(dl, cache, torch.from_numpy(slots).to(DEV), inputs_dev(inp, "bf16"), y)
        torch.cuda.synchronize()
        outs.append((y.clone(), cache.state.clone(), cache.conv_state.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_cache_policy_flags_are_bitwise_identical(dk, dv):
    """The cache-policy flags change only how state traffic is cached: decode
    (streaming by default, cached under KDA_STATE_RESIDENT) and verify
    (cached by default, streaming under KDA_STREAM_STATE) give bitwise the
    same results under every setting, for every supported head size."""
    g = synth.rng(740 + dk + 2 * dv)
    H, B, T = 4, 6, 5
    params = synth.layer_params(g, H, dk, dv)
    layers = []
    for stream, resident in ((False, False), (True, False), (False, True), (True, True)):
        layer, _ = layer_pair(params)
        layer.stream_state, layer.state_resident = stream, resident
        layers.append(layer)
    inp = synth.token_inputs(g, (B,), H, dk, dv, "bf16")
    vin = synth.token_inputs(g, (B, T), H, dk, dv, "bf16")
    outs = []
    for layer in layers:
        cache = new_cache(B + B * T, H, dk, dv, "bf16", fill_seed=12)
        live = torch.arange(B, dtype=torch.int32, device=DEV)
        snaps = torch.arange(B, B + B * T, dtype=torch.int32, device=DEV).reshape(B, T)
        y = torch.empty((B, H, dv), device=DEV)
        api.kda_decode(layer, cache, live, inputs_dev(inp, "bf16"), y)
        yv = torch.empty((B, T, H, dv), device=DEV)
        api.kda_spec_verify(layer, cache, live, snaps, inputs_dev(vin, "bf16"), yv)
        torch.cuda.synchronize()
        outs.append((y, yv, cache.state.clone(), cache.conv_state.clone()))
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a, b)


def test_decode_in_a_hip_graph_matches_eager():
    """One decode step captured in a HIP graph (torch.cuda.CUDAGraph on the
    capture stream) and replayed step after step, with the next step's inputs
    copied into the captured buffers eagerly between replays: every replay's
    output and the final state and window equal the eager launches bitwise."""
    B, H, dk, dv, steps = 4, 4, 128, 128, 6
    g = synth.rng(1500)
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    inp = synth.token_inputs(g, (steps, B), H, dk, dv, "bf16")
    slots = torch.from_numpy(g.permutation(8)[:B].astype(np.int32)).to(DEV)
    eager = new_cache(8, H, dk, dv, "bf16", fill_seed=3)
    graphed = api.Cache(eager.state.clone(), eager.conv_state.clone(), torch.zeros_like(eager.err_flag))
    ye = []
    for t in range(steps):
        y = torch.empty((B, H, dv), device=DEV)
        api.kda_decode(dl, eager, slots, inputs_dev(inp, "bf16", sl=t), y)
        ye.append(y)
    static = inputs_dev(inp, "bf16", sl=0)
    ys = torch.empty((B, H, dv), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        api.kda_decode(dl, graphed, slots, static, ys)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture does not run the kernel: the graphed pools still hold the start state
    assert not torch.equal(graphed.state, eager.state)
    for t in range(steps):
        src = inputs_dev(inp, "bf16", sl=t)
        for name in ("x_q", "x_k", "x_v", "g", "b", "z"):
            getattr(static, name).copy_(getattr(src, name))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, ye[t]), t
    assert torch.equal(graphed.state, eager.state)
    assert torch.equal(graphed.conv_state, eager.conv_state)
    assert graphed.err_flag.item() == 0


def test_alpha_zero_forgets_the_state():
    """g = +inf (bf16 infinity): alpha = exp(-e^A * inf) = 0 exactly, so the
    old state is wiped and, from any state, S_1 = beta k^ v^T and
    o = beta (k^.q^) v as from a zero state; GPU state and outputs match the
    oracle run from the same (non-zero) start."""
    dl, ol, inp, slots = _slot_case(seed=720)
    inp = dict(inp, g=np.full_like(inp["g"], np.inf))
    cache = new_cache(32, dl.H, dl.d_k, dl.d_v, "bf16", fill_seed=11)
    st = torch.from_numpy(slots).to(DEV).long()
    s0, w0 = host(cache.state[st]), host(cache.conv_state[st])
    y = torch.empty((8, dl.H, dl.d_v), device=DEV)
    api.kda_decode(dl, cache, torch.from_numpy(slots).to(DEV), inputs_dev(inp, "bf16"), y)
    torch.cuda.synchronize()
    o = kda_oracle.run(ol, s0, w0, *(inp[k][:, None] for k in ("x_q", "x_k", "x_v", "g", "b", "z")))
    z = kda_oracle.run(ol, np.zeros_like(s0), w0, *(inp[k][:, None] for k in ("x_q", "x_k", "x_v", "g", "b", "z")))
    assert np.array_equal(o["state"], z["state"])            # the oracle forgets S0 as well
    assert parity_error(host(y), o["y"][:, 0]) <= TOL
    assert state_rel_err(host(cache.state[st]), o["state"]) < 1e-5
    assert cache.err_flag.item() == 0


def test_large_batch_sampled_sequences():
    """B = 512 sequences (16384 workgroups, many rounds) over a 2048-slot
    pool: 6 sampled sequences against the oracle over 3 steps, every slot
    outside the table bitwise untouched."""
    B, H, dk, dv, n_slots, steps = 512, 32, 128, 128, 2048, 3
    g = synth.rng(730)
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    inp = synth.token_inputs(g, (steps, B), H, dk, dv, "bf16")
    slots = synth.slot_table(g, B, n_slots)
    cache = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=12)
    before_s, before_w = cache.state.clone(), cache.conv_state.clone()
    pick = np.array([0, 1, 137, 255, 256, 511])
    s0 = host(cache.state[torch.from_numpy(slots[pick]).long().to(DEV)])
    w0 = host(cache.conv_state[torch.from_numpy(slots[pick]).long().to(DEV)])
    y = run_decode_steps(dl, cache, torch.from_numpy(slots).to(DEV), inp, "bf16", steps, B)
    sub = {k: v[:, pick] for k, v in inp.items()}
    yo, so, wo = oracle_steps(ol, s0, w0, sub, steps)
    assert_per_step(y[:, pick], yo)
    got = host(cache.state[torch.from_numpy(slots[pick]).long().to(DEV)])
    assert state_rel_err(got, so) < 1e-5
    assert np.array_equal(host(cache.conv_state[torch.from_numpy(slots[pick]).long().to(DEV)]), wo)
    untouched = torch.ones(n_slots, dtype=torch.bool, device=DEV)
    untouched[torch.from_numpy(slots).long().to(DEV)] = False
    assert torch.equal(cache.state[untouched], before_s[untouched])
    assert torch.equal(cache.conv_state[untouched], before_w[untouched])
    assert cache.err_flag.item() == 0


@pytest.mark.parametrize("resident", [False, True])
def test_multi_round_batch_equals_small_batches_bitwise(resident):
    """A batch of more (sequence, head) items than the GPU holds at once
    (here 2560 workgroups, several rounds) gives bitwise the results of the
    same rows decoded 16 sequences at a time, with padding and bad rows,
    under both cache policies."""
    g = synth.rng(1500 + int(resident))
    B, H, dk, dv, n_slots = 80, 32, 128, 128, 200
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    dl.state_resident = resident
    inp = synth.token_inputs(g, (B,), H, dk, dv, "bf16")
    slots = synth.slot_table(g, B, n_slots)
    slots[3] = -1        # padding
    slots[41] = n_slots  # out of range
    big = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=21)
    small = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=21)
    yb = torch.full((B, H, dv), 9.0, device=DEV)
    api.kda_decode(dl, big, torch.from_numpy(slots).to(DEV), inputs_dev(inp, "bf16"), yb)
    ys = torch.full((B, H, dv), 9.0, device=DEV)
    for a in range(0, B, 16):
        sl = slice(a, a + 16)
        api.kda_decode(dl, small, torch.from_numpy(slots[sl].copy()).to(DEV), inputs_dev(inp, "bf16", sl),
                       ys[a:a + 16])
    torch.cuda.synchronize()
    assert big.err_flag.item() == 1 and small.err_flag.item() == 1
    assert torch.count_nonzero(yb[3]) == 0 and torch.count_nonzero(yb[41]) == 0
    assert torch.equal(yb, ys)
    assert torch.equal(big.state, small.state) and torch.equal(big.conv_state, small.conv_state)
