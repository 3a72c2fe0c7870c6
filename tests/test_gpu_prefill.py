"""GPU parity of kda_chunk_prefill against the token-by-token fp64 oracle:
brute force on small sizes (chunk boundaries, partial chunks, T = 1), several
packed sequences with their own start states and windows, prefill followed
by decode, the full 32768-token workload on every head, error handling."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, TOL, host, layer_pair, new_cache, parity_error, state_rel_err, tdt, to_dev
from linear_attention_recurrent_kda_amd import api, synth
from oracle import kda_oracle

pytestmark = pytest.mark.gpu

KEYS = ("x_q", "x_k", "x_v", "g", "b", "z")


def dev_inputs(inp, dtype):
    return api.Inputs(*(to_dev(inp[k], tdt(dtype)) for k in KEYS))


def run_prefill(dl, cache, slots, lens, inp, dtype):
    """inp arrays are packed [total_T, H, .]; lens per sequence."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    y = torch.full((total, dl.H, dl.d_v), 7.0, device=DEV)
    api.kda_chunk_prefill(dl, cache, torch.from_numpy(np.asarray(slots, np.int32)).to(DEV),
                          torch.from_numpy(cu).to(DEV), dev_inputs(inp, dtype), y)
    torch.cuda.synchronize()
    return host(y), cu


def oracle_seq(ol, s0, w0, inp, a, b, y_tokens=None):
    """Oracle over packed tokens [a, b) as one sequence."""
    sub = {k: v[None, a:b] for k, v in inp.items()}
    return kda_oracle.run(ol, s0[None], w0[None], sub["x_q"], sub["x_k"], sub["x_v"], sub["g"],
                          sub["b"], sub["z"], y_tokens=y_tokens)


def check_tokens(y_gpu, y_orc):
    """Per-token check: max |d| over the token's H x d_v outputs <= TOL x RMS."""
    errs = [parity_error(y_gpu[t], y_orc[t]) for t in range(y_gpu.shape[0])]
    if not errs:
        return 0.0
    worst = int(np.argmax(errs))
    print(f"  prefill parity: worst token {worst} max|d|/RMS = {errs[worst]:.3e}", flush=True)
    assert errs[worst] <= TOL, f"token {worst}: {errs[worst]:.3e}"
    return errs[worst]


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 130, 257])
def test_single_sequence_brute_force(T):
    g = synth.rng(900 + T)
    H, dk, dv = 4, 128, 128
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    inp = synth.token_inputs(g, (T,), H, dk, dv, "bf16")
    s0 = synth.random_state(g, (H, dk, dv), 0.2)
    w0 = synth.window_inputs(g, (), H, dk, dv, "bf16")
    cache = new_cache(3, H, dk, dv, "bf16", fill_seed=1)
    cache.state[1] = torch.from_numpy(s0).to(DEV)
    cache.conv_state[1] = to_dev(w0, torch.bfloat16)
    other = cache.state[[0, 2]].clone()
    y, _ = run_prefill(dl, cache, [1], [T], inp, "bf16")
    o = oracle_seq(ol, s0, w0, inp, 0, T)
    check_tokens(y, o["y"][0])
    assert state_rel_err(host(cache.state[1:2]), o["state"]) < 1e-4
    assert np.array_equal(host(cache.conv_state[1:2]), o["window"])
    assert torch.equal(cache.state[[0, 2]], other)
    assert cache.err_flag.item() == 0


@pytest.mark.parametrize("dk,dv,dtype", [(64, 64, "f32"), (64, 128, "bf16"), (128, 64, "bf16")])
def test_other_head_sizes(dk, dv, dtype):
    g = synth.rng(950 + dk + dv)
    H, T = 2, 150
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    inp = synth.token_inputs(g, (T,), H, dk, dv, dtype)
    cache = new_cache(2, H, dk, dv, dtype)
    y, _ = run_prefill(dl, cache, [1], [T], inp, dtype)
    o = oracle_seq(ol, np.zeros((H, dk, dv)), np.zeros((H, 3, 2 * dk + dv)), inp, 0, T)
    check_tokens(y, o["y"][0])
    assert state_rel_err(host(cache.state[1:2]), o["state"]) < 1e-4


def test_strong_decay_direct_diagonal_tiles():
    """Decay strong enough that some 16-token blocks span more than 2^60 of
    decay (their diagonal Gram tiles take the direct path), mixed with weak
    blocks, and one token whose decay hits the log2(alpha) floor."""
    g = synth.rng(960)
    H, dk, dv, T = 2, 128, 128, 200
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    inp = synth.token_inputs(g, (T,), H, dk, dv, "f32")
    pos = np.arange(T) % 64
    strong = ((pos // 16) % 2 == 1)[:, None, None]          # blocks 1 and 3 of every chunk
    inp["g"] = np.where(strong, inp["g"] + 8.0, inp["g"]).astype(np.float32)
    inp["g"][77] = 1000.0
    cache = new_cache(1, H, dk, dv, "f32")
    y, _ = run_prefill(dl, cache, [0], [T], inp, "f32")
    o = oracle_seq(ol, np.zeros((H, dk, dv)), np.zeros((H, 3, 2 * dk + dv)), inp, 0, T)
    check_tokens(y, o["y"][0])
    assert state_rel_err(host(cache.state), o["state"]) < 1e-4


def test_packed_sequences_with_padding():
    """Four packed sequences (lengths 70, 0, 2, 129) with their own start
    states and windows, one padding row (-1), slots in permuted order."""
    g = synth.rng(970)
    H, dk, dv = 3, 128, 128
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    lens = [70, 0, 2, 129, 5]
    slots = [4, 0, 2, 1, -1]
    total = sum(lens)
    inp = synth.token_inputs(g, (total,), H, dk, dv, "bf16")
    cache = new_cache(6, H, dk, dv, "bf16", fill_seed=2)
    s_before = host(cache.state)
    w_before = host(cache.conv_state)
    y, cu = run_prefill(dl, cache, slots, lens, inp, "bf16")
    assert cache.err_flag.item() == 0
    for i, (sl, ln) in enumerate(zip(slots, lens)):
        a, b = cu[i], cu[i + 1]
        if sl < 0:
            assert np.all(y[a:b] == 0.0)
            continue
        o = oracle_seq(ol, s_before[sl], w_before[sl], inp, a, b)
        check_tokens(y[a:b], o["y"][0])
        assert state_rel_err(host(cache.state[sl:sl + 1]), o["state"]) < 1e-4
        assert np.array_equal(host(cache.conv_state[sl:sl + 1]), o["window"])
    # slots nobody named are untouched
    assert np.array_equal(host(cache.state[[3, 5]]), s_before[[3, 5]])


def test_many_sequences_mixed_lengths():
    """41 packed sequences with seeded lengths from 0 to 200 (chunk-aligned,
    one-token and empty ones included), three padding rows, slots in random
    order: every output, final state and window against the oracle."""
    g = synth.rng(975)
    H, dk, dv = 2, 64, 64
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    lens = [int(x) for x in g.integers(0, 201, size=41)]
    lens[:6] = [0, 1, 64, 128, 3, 65]
    n_slots = 48
    slots = [int(x) for x in g.permutation(n_slots)[:41]]
    for i in (7, 19, 33):
        slots[i] = -1
    total = sum(lens)
    inp = synth.token_inputs(g, (total,), H, dk, dv, "bf16")
    cache = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=4)
    s_before = host(cache.state)
    w_before = host(cache.conv_state)
    y, cu = run_prefill(dl, cache, slots, lens, inp, "bf16")
    assert cache.err_flag.item() == 0
    worst = 0.0
    for i, (sl, ln) in enumerate(zip(slots, lens)):
        a, b = cu[i], cu[i + 1]
        if sl < 0:
            assert np.all(y[a:b] == 0.0)
            continue
        o = oracle_seq(ol, s_before[sl], w_before[sl], inp, a, b)
        if ln:
            errs = [parity_error(y[t], o["y"][0][t - a]) for t in range(a, b)]
            worst = max(worst, max(errs))
        assert state_rel_err(host(cache.state[sl:sl + 1]), o["state"]) < 1e-4
        assert np.array_equal(host(cache.conv_state[sl:sl + 1]), o["window"])
    print(f"  prefill parity over {len(lens)} sequences: worst max|d|/RMS = {worst:.3e}", flush=True)
    assert worst <= TOL


def test_many_sequences_wide_scan_blocks():
    """40 packed sequences x 8 heads at d = 128: enough workgroups that the
    scan takes 64-column blocks.  Every output, final state and window against
    the oracle, and the outputs bitwise equal to the same sequences run alone
    (16-column blocks)."""
    g = synth.rng(976)
    H, dk, dv = 8, 128, 128
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    lens = [int(x) for x in g.integers(200, 601, size=40)]   # ~16K tokens: four chunks per row on average
    lens[:5] = [0, 1, 64, 200, 129]
    n_slots = 44
    slots = [int(x) for x in g.permutation(n_slots)[:40]]
    slots[11] = -1
    total = sum(lens)
    inp = synth.token_inputs(g, (total,), H, dk, dv, "bf16")
    cache = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=5)
    s_before = host(cache.state)
    w_before = host(cache.conv_state)
    y, cu = run_prefill(dl, cache, slots, lens, inp, "bf16")
    assert cache.err_flag.item() == 0
    worst = 0.0
    for i, (sl, ln) in enumerate(zip(slots, lens)):
        a, b = cu[i], cu[i + 1]
        if sl < 0:
            assert np.all(y[a:b] == 0.0)
            continue
        o = oracle_seq(ol, s_before[sl], w_before[sl], inp, a, b)
        if ln:
            errs = [parity_error(y[t], o["y"][0][t - a]) for t in range(a, b)]
            worst = max(worst, max(errs))
        assert state_rel_err(host(cache.state[sl:sl + 1]), o["state"]) < 1e-4
        assert np.array_equal(host(cache.conv_state[sl:sl + 1]), o["window"])
    print(f"  prefill parity over {len(lens)} sequences x {H} heads: worst max|d|/RMS = {worst:.3e}", flush=True)
    assert worst <= TOL
    # sequence 3 (200 tokens) alone: one sequence, 16-column scan blocks
    i = 3
    a, b = cu[i], cu[i + 1]
    one = {k: v[a:b] for k, v in inp.items()}
    c1 = new_cache(n_slots, H, dk, dv, "bf16")
    c1.state.copy_(torch.from_numpy(s_before).to(DEV))
    c1.conv_state.copy_(torch.from_numpy(w_before).to(DEV).to(torch.bfloat16))
    y1, _ = run_prefill(dl, c1, [slots[i]], [lens[i]], one, "bf16")
    assert np.array_equal(y1, y[a:b])
    assert np.array_equal(host(c1.state[slots[i]]), host(cache.state[slots[i]]))


def test_head_count_not_a_multiple_of_8_many_rounds():
    """12 heads (padded to 16 in the scan's item order) x 6 sequences at
    d = 64: more 16-column scan items than workgroups, so the groups of
    column workgroups that exchange row sums come in several rounds, beside
    items of padded heads that only exit.  Every output, final state and
    window against the oracle."""
    g = synth.rng(977)
    H, dk, dv = 12, 64, 64
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    lens = [130, 64, 257, 2, 1, 190]
    n_slots = 8
    slots = [5, 0, 7, 2, 3, 6]
    total = sum(lens)
    inp = synth.token_inputs(g, (total,), H, dk, dv, "bf16")
    cache = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=6)
    s_before = host(cache.state)
    w_before = host(cache.conv_state)
    y, cu = run_prefill(dl, cache, slots, lens, inp, "bf16")
    assert cache.err_flag.item() == 0
    worst = 0.0
    for i, (sl, ln) in enumerate(zip(slots, lens)):
        a, b = cu[i], cu[i + 1]
        o = oracle_seq(ol, s_before[sl], w_before[sl], inp, a, b)
        errs = [parity_error(y[t], o["y"][0][t - a]) for t in range(a, b)]
        worst = max(worst, max(errs))
        assert state_rel_err(host(cache.state[sl:sl + 1]), o["state"]) < 1e-4
        assert np.array_equal(host(cache.conv_state[sl:sl + 1]), o["window"])
    print(f"  prefill parity over {len(lens)} sequences x {H} heads: worst max|d|/RMS = {worst:.3e}", flush=True)
    assert worst <= TOL


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (64, 64, "f32")])
def test_rows_left_for_the_repair_kernel(dk, dv, dtype, monkeypatch):
    """The 16-column scan normalises O rows with row sums that other
    workgroups publish.  A row whose sums do not arrive within the wait
    bound is stored unnormalised and marked, and a kernel after the scan
    normalises it with the same arithmetic.  KDA_XP_SPIN bounds the wait
    (a negative value: no row is taken as in time, so every row goes the
    repair way; 0: one poll).  Both give bitwise the outputs and states of
    the ordinary call, with no error flag, and match the oracle."""
    g = synth.rng(981 + dk)
    H = 8
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    lens = [300, 1, 129, 64]
    slots = [2, 0, 3, 1]
    inp = synth.token_inputs(g, (sum(lens),), H, dk, dv, dtype)
    runs = {}
    for spin in (None, "-1", "0"):
        if spin is None:
            monkeypatch.delenv("KDA_XP_SPIN", raising=False)
        else:
            monkeypatch.setenv("KDA_XP_SPIN", spin)
        cache = new_cache(4, H, dk, dv, dtype, fill_seed=9)
        if spin is None:
            s_before, w_before = host(cache.state), host(cache.conv_state)
        y, cu = run_prefill(dl, cache, slots, lens, inp, dtype)
        assert cache.err_flag.item() == 0
        runs[spin] = (y, host(cache.state), host(cache.conv_state))
    monkeypatch.delenv("KDA_XP_SPIN", raising=False)
    for spin in ("-1", "0"):
        for a, b in zip(runs[None], runs[spin]):
            assert np.array_equal(a, b), f"KDA_XP_SPIN={spin}"
    y = runs["-1"][0]
    for i, (sl, ln) in enumerate(zip(slots, lens)):
        o = oracle_seq(ol, s_before[sl], w_before[sl], inp, cu[i], cu[i + 1])
        check_tokens(y[cu[i]:cu[i + 1]], o["y"][0])


def test_two_calls_at_once_on_two_streams(monkeypatch):
    """Two prefill calls launched on two streams at once, each with its own
    cache and (allocated) workspace: the column workgroups of one call can
    find compute units held by the other's, so some waits for row sums may
    run out (the bound is cut to 4096 polls to keep such waits short) and
    those rows take the repair kernel.  Outputs and states are bitwise those
    of the same calls run one after the other."""
    monkeypatch.setenv("KDA_XP_SPIN", "4096")
    g = synth.rng(986)
    H, dk, dv, T = 32, 128, 128, 2048
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    inps = [dev_inputs(synth.token_inputs(g, (T,), H, dk, dv, "bf16"), "bf16") for _ in range(2)]
    sl = torch.zeros(1, dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, T], dtype=torch.int32, device=DEV)

    def fresh():
        return [new_cache(1, H, dk, dv, "bf16", fill_seed=11 + i) for i in range(2)], \
               [torch.full((T, H, dv), 7.0, device=DEV) for _ in range(2)]

    caches, ys = fresh()
    for i in range(2):
        api.kda_chunk_prefill(dl, caches[i], sl, cu, inps[i], ys[i])
    torch.cuda.synchronize()
    want = [(host(ys[i]), host(caches[i].state)) for i in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        caches, ys = fresh()
        torch.cuda.synchronize()
        for i in range(2):
            api.kda_chunk_prefill(dl, caches[i], sl, cu, inps[i], ys[i], stream=streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert caches[i].err_flag.item() == 0
            assert np.array_equal(host(ys[i]), want[i][0])
            assert np.array_equal(host(caches[i].state), want[i][1])


@pytest.mark.parametrize("static", [False, True])
def test_prefill_in_a_hip_graph_matches_eager(static):
    """A mixed batch (prompts and one-token rows: the metadata, decode, intra,
    scan and repair launches) captured in a HIP graph, with a caller
    workspace or in the library's static array, and replayed three times;
    before each replay the start states and windows are copied back eagerly,
    and an eager call on other buffers runs between replays.  Every replay's
    outputs, states and windows equal the eager call's bitwise."""
    g = synth.rng(991)
    H, dk, dv = 8, 128, 128
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    lens, slots = [300, 1, 130, 1], [2, 0, 3, 1]
    total = sum(lens)
    inp = dev_inputs(synth.token_inputs(g, (total,), H, dk, dv, "bf16"), "bf16")
    sl = torch.from_numpy(np.asarray(slots, np.int32)).to(DEV)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(DEV)
    ws = torch.empty(api.kda_chunk_prefill_workspace_bytes(dl, total, len(lens)), dtype=torch.uint8, device=DEV)

    def call(cache, y):
        if static:
            api.kda_chunk_prefill_static(dl, cache, sl, cu, inp, y)
        else:
            api.kda_chunk_prefill(dl, cache, sl, cu, inp, y, ws)

    cache = new_cache(4, H, dk, dv, "bf16", fill_seed=31)
    s0, w0 = cache.state.clone(), cache.conv_state.clone()
    y = torch.full((total, H, dv), 7.0, device=DEV)
    call(cache, y)
    torch.cuda.synchronize()
    want = (y.clone(), cache.state.clone(), cache.conv_state.clone())
    other = new_cache(4, H, dk, dv, "bf16", fill_seed=32)
    y_other = torch.empty_like(y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(cache, y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        cache.state.copy_(s0)
        cache.conv_state.copy_(w0)
        y.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want[0]), r
        assert torch.equal(cache.state, want[1]), r
        assert torch.equal(cache.conv_state, want[2]), r
        assert cache.err_flag.item() == 0
        call(other, y_other)   # eager work between replays
        torch.cuda.synchronize()


def test_prefill_then_decode_continues_the_sequence():
    g = synth.rng(980)
    H, dk, dv, T, D = 4, 128, 128, 100, 20
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    inp = synth.token_inputs(g, (T + D,), H, dk, dv, "bf16")
    cache = new_cache(2, H, dk, dv, "bf16")
    pre = {k: v[:T] for k, v in inp.items()}
    y_pre, _ = run_prefill(dl, cache, [1], [T], pre, "bf16")
    slot = torch.tensor([1], dtype=torch.int32, device=DEV)
    ys = []
    for t in range(T, T + D):
        I = api.Inputs(*(to_dev(inp[k][t:t + 1], torch.bfloat16) for k in KEYS))
        y = torch.empty((1, H, dv), device=DEV)
        api.kda_decode(dl, cache, slot, I, y)
        ys.append(host(y)[0])
    o = oracle_seq(ol, np.zeros((H, dk, dv)), np.zeros((H, 3, 2 * dk + dv)), inp, 0, T + D)
    check_tokens(y_pre, o["y"][0, :T])
    check_tokens(np.stack(ys), o["y"][0, T:])


def test_full_length_32k_all_heads():
    """The long-prompt workload at full size: B=1, T=32768, H=32, d=128,
    every head checked against the sequential oracle: outputs of the first
    2048 tokens and of the last chunk, each 8192-token checkpoint (state and
    window) and the final state.  The same call with a checkpoint every 8192
    tokens gives bitwise the same outputs and final state."""
    cfg = synth.WORKLOADS["prefill_t32k"]
    g = synth.rng(cfg["seed"])
    H, dk, dv, T = cfg["H"], cfg["d_k"], cfg["d_v"], cfg["T"]
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    inp = synth.token_inputs(g, (T,), H, dk, dv, "bf16")
    cache = new_cache(1, H, dk, dv, "bf16")
    print("  running prefill on the GPU", flush=True)
    y, _ = run_prefill(dl, cache, [0], [T], inp, "bf16")
    # the same call keeping a checkpoint every 8192 tokens (slots 1..4)
    print("  running prefill with checkpoints on the GPU", flush=True)
    ckc = new_cache(5, H, dk, dv, "bf16")
    yc = torch.empty((T, H, dv), device=DEV)
    api.kda_chunk_prefill_ckpt(dl, ckc, torch.zeros(1, dtype=torch.int32, device=DEV),
                               torch.tensor([0, T], dtype=torch.int32, device=DEV), dev_inputs(inp, "bf16"),
                               yc, torch.arange(1, 5, dtype=torch.int32, device=DEV).reshape(1, 4), 8192)
    torch.cuda.synchronize()
    assert ckc.err_flag.item() == 0
    assert np.array_equal(host(yc), y)
    assert torch.equal(ckc.state[0], cache.state[0])
    print("  oracle: all heads, first 2048 tokens", flush=True)
    st, win = np.zeros((H, dk, dv)), np.zeros((H, 3, 2 * dk + dv))
    o = oracle_seq(ol, st, win, inp, 0, 2048)
    check_tokens(y[:2048], o["y"][0])
    for j in range(4):
        print(f"  oracle: all heads, tokens {8192 * j} .. {8192 * (j + 1)}", flush=True)
        o2 = oracle_seq(ol, st, win, inp, 8192 * j, 8192 * (j + 1), y_tokens=8192 if j == 3 else 0)
        st, win = o2["state"][0], o2["window"][0]
        err = state_rel_err(host(ckc.state[j + 1:j + 2]), o2["state"])
        print(f"  checkpoint {j} state rel err (all {H} heads) {err:.3e}", flush=True)
        assert err < 1e-3
        assert np.array_equal(host(ckc.conv_state[j + 1]), o2["window"][0])
    check_tokens(y[-64:], o2["y"][0, -64:])
    err = state_rel_err(host(cache.state[0:1]), o2["state"])
    print(f"  final state rel err (all {H} heads) {err:.3e}", flush=True)
    assert err < 1e-3
    assert np.array_equal(host(cache.conv_state[0]), o2["window"][0])
    assert torch.equal(ckc.state[4], ckc.state[0])


def test_all_sequences_empty():
    """total_T = 0: nothing to compute; states and windows stay bitwise."""
    g = synth.rng(985)
    H, dk, dv = 2, 128, 128
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    inp = synth.token_inputs(g, (0,), H, dk, dv, "bf16")
    cache = new_cache(3, H, dk, dv, "bf16", fill_seed=5)
    s_before, w_before = cache.state.clone(), cache.conv_state.clone()
    y, _ = run_prefill(dl, cache, [2, 0, 1], [0, 0, 0], inp, "bf16")
    assert y.shape == (0, H, dv)
    assert torch.equal(cache.state, s_before) and torch.equal(cache.conv_state, w_before)
    assert cache.err_flag.item() == 0


def test_invalid_cu_seqlens_flags_and_leaves_state():
    g = synth.rng(990)
    H, dk, dv = 2, 64, 64
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    inp = synth.token_inputs(g, (10,), H, dk, dv, "bf16")
    cache = new_cache(3, H, dk, dv, "bf16", fill_seed=3)
    before = cache.state.clone()
    y = torch.full((10, H, dv), 5.0, device=DEV)
    bad_cu = torch.tensor([0, 7, 4, 10], dtype=torch.int32, device=DEV)
    api.kda_chunk_prefill(dl, cache, torch.tensor([0, 1, 2], dtype=torch.int32, device=DEV),
                          bad_cu, dev_inputs(inp, "bf16"), y)
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 1
    assert torch.equal(cache.state, before)
    assert torch.count_nonzero(y) == 0


def test_prefill_deterministic():
    g = synth.rng(995)
    H, dk, dv, T = 4, 128, 128, 200
    params = synth.layer_params(g, H, dk, dv)
    dl, _ = layer_pair(params)
    inp = synth.token_inputs(g, (T,), H, dk, dv, "bf16")
    outs = []
    for _ in range(2):
        cache = new_cache(1, H, dk, dv, "bf16")
        y, _ = run_prefill(dl, cache, [0], [T], inp, "bf16")
        outs.append((y, host(cache.state)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


# ---------------------------------------------------------------------------
# interval checkpoints (kda_chunk_prefill_ckpt)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("interval", [64, 128])
def test_prefill_checkpoints_match_oracle(interval):
    """Each checkpoint equals the oracle's state and window after that many
    tokens; outputs and final states are bitwise those of kda_chunk_prefill;
    slots the call must not touch stay as they were."""
    g = synth.rng(1200 + interval)
    H, dk, dv = 4, 128, 128
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    lens = [300, 128, 70, 0, 63]
    per = 4
    total = sum(lens)
    inp = synth.token_inputs(g, (total,), H, dk, dv, "bf16")
    N = len(lens)
    n_slots = N + N * per + 2
    perm = g.permutation(n_slots).astype(np.int32)
    live = perm[:N].copy()
    ck = perm[N:N + N * per].reshape(N, per).copy()
    ck[2, 0] = -1                       # sequence 2's only checkpoint is not kept
    s0 = synth.random_state(g, (N, H, dk, dv), 0.2)
    w0 = synth.window_inputs(g, (N,), H, dk, dv, "bf16")
    cache = new_cache(n_slots, H, dk, dv, "bf16", fill_seed=5)
    lt = torch.from_numpy(live).to(DEV).long()
    cache.state[lt] = torch.from_numpy(s0).to(DEV)
    cache.conv_state[lt] = to_dev(w0, torch.bfloat16)
    plain = api.Cache(cache.state.clone(), cache.conv_state.clone(), torch.zeros_like(cache.err_flag))
    before = api.Cache(cache.state.clone(), cache.conv_state.clone(), None)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cut = torch.from_numpy(cu).to(DEV)
    y = torch.full((total, H, dv), 7.0, device=DEV)
    api.kda_chunk_prefill_ckpt(dl, cache, lt.int(), cut, dev_inputs(inp, "bf16"), y,
                               torch.from_numpy(ck).to(DEV), interval)
    y2 = torch.full_like(y, 7.0)
    api.kda_chunk_prefill(dl, plain, lt.int(), cut, dev_inputs(inp, "bf16"), y2)
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 0
    assert torch.equal(y, y2)
    assert torch.equal(cache.state[lt], plain.state[lt])
    assert torch.equal(cache.conv_state[lt], plain.conv_state[lt])
    written = set()
    for s in range(N):
        n_ck = min(per, lens[s] // interval)
        if n_ck == 0:
            continue
        sub = {k: v[None, cu[s]:cu[s + 1]] for k, v in inp.items()}
        o = kda_oracle.run(ol, s0[s][None], w0[s][None], sub["x_q"], sub["x_k"], sub["x_v"], sub["g"],
                           sub["b"], sub["z"], y_tokens=0, snapshots=True)
        for j in range(n_ck):
            if ck[s, j] == -1:
                continue
            pos = (j + 1) * interval
            slot = int(ck[s, j])
            written.add(slot)
            err = state_rel_err(host(cache.state[slot:slot + 1]), o["snap_state"][:, pos - 1])
            assert err < 1e-4, (s, j, err)
            assert np.array_equal(host(cache.conv_state[slot]), o["snap_window"][0, pos - 1]), (s, j)
    # a checkpoint at the last token equals the final state bit for bit
    if lens[0] % interval == 0 or lens[1] % interval == 0:
        s = 0 if lens[0] % interval == 0 else 1
        j = lens[s] // interval - 1
        if j < per:
            assert torch.equal(cache.state[int(ck[s, j])], cache.state[int(live[s])])
    untouched = [i for i in range(n_slots) if i not in written and i not in set(live.tolist())]
    ut = torch.tensor(untouched, device=DEV).long()
    assert torch.equal(cache.state[ut], before.state[ut])
    assert torch.equal(cache.conv_state[ut], before.conv_state[ut])
    assert len(written) == sum(int(ck[s, j] != -1) for s in range(N) for j in range(min(per, lens[s] // interval)))


def test_prefill_checkpoint_bad_slot_flags_error():
    g = synth.rng(1300)
    H, dk, dv = 2, 64, 64
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    T = 192
    inp = synth.token_inputs(g, (T,), H, dk, dv, "bf16")
    cache = new_cache(4, H, dk, dv, "bf16")
    ck = np.array([[2, cache.n_slots + 9, 3]], dtype=np.int32)
    y = torch.empty((T, H, dv), device=DEV)
    api.kda_chunk_prefill_ckpt(dl, cache, torch.tensor([0], dtype=torch.int32, device=DEV),
                               torch.tensor([0, T], dtype=torch.int32, device=DEV), dev_inputs(inp, "bf16"),
                               y, torch.from_numpy(ck).to(DEV), 64)
    torch.cuda.synchronize()
    assert cache.err_flag.item() == 1
    o = oracle_seq(ol, np.zeros((H, dk, dv)), np.zeros((H, 3, 2 * dk + dv)), inp, 0, T, y_tokens=T)
    check_tokens(host(y), o["y"][0])
    assert state_rel_err(host(cache.state[0:1]), o["state"]) < 1e-4
    # the good checkpoints (64 and 192 tokens) were still written
    o2 = kda_oracle.run(ol, np.zeros((1, H, dk, dv)), np.zeros((1, H, 3, 2 * dk + dv)),
                        *(inp[k][None] for k in KEYS), y_tokens=0, snapshots=True)
    assert state_rel_err(host(cache.state[2:3]), o2["snap_state"][:, 63]) < 1e-4
    assert state_rel_err(host(cache.state[3:4]), o2["snap_state"][:, 191]) < 1e-4


def test_mixed_batch_one_token_rows_equal_decode_bitwise():
    """A packed batch mixing prompts and one-token (decode) rows: the
    one-token sequences take the decode kernel inside kda_chunk_prefill, so
    their outputs, states and windows equal a kda_decode call on the same
    rows bit for bit; the longer sequences match the oracle."""
    g = synth.rng(1400)
    H, dk, dv = 4, 128, 128
    params = synth.layer_params(g, H, dk, dv)
    dl, ol = layer_pair(params)
    lens = [300, 1, 1, 5, 0, 1, 70]
    N, total = len(lens), sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    inp = synth.token_inputs(g, (total,), H, dk, dv, "bf16")
    slots = g.permutation(2 * N)[:N].astype(np.int32)
    cache = new_cache(2 * N, H, dk, dv, "bf16", fill_seed=14)
    ref = api.Cache(cache.state.clone(), cache.conv_state.clone(), torch.zeros_like(cache.err_flag))
    s0, w0 = host(cache.state[torch.from_numpy(slots).long().to(DEV)]), host(cache.conv_state[torch.from_numpy(slots).long().to(DEV)])
    y, _ = run_prefill(dl, cache, slots, lens, inp, "bf16")
    assert cache.err_flag.item() == 0
    one = [s for s in range(N) if lens[s] == 1]
    rows = cu[one]
    yd = torch.empty((len(one), H, dv), device=DEV)
    api.kda_decode(dl, ref, torch.from_numpy(slots[one]).to(DEV), dev_inputs({k: v[rows] for k, v in inp.items()}, "bf16"), yd)
    torch.cuda.synchronize()
    assert np.array_equal(y[rows], host(yd))
    st = torch.from_numpy(slots[one]).long().to(DEV)
    assert torch.equal(cache.state[st], ref.state[st])
    assert torch.equal(cache.conv_state[st], ref.conv_state[st])
    for s in (0, 3, 6):
        o = oracle_seq(ol, s0[s], w0[s], inp, cu[s], cu[s + 1])
        check_tokens(y[cu[s]:cu[s + 1]], o["y"][0])
        assert state_rel_err(host(cache.state[int(slots[s]):int(slots[s]) + 1]), o["state"]) < 1e-4
    # the empty sequence's slot is untouched
    e = int(slots[4])
    assert torch.equal(cache.state[e], ref.state[e])
