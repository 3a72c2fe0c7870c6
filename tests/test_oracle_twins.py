"""The two oracle implementations agree with each other, and the chunked
(WY/UT) form of the core agrees with the token-by-token recurrence, by brute
force on small inputs (chunk boundaries, partial last chunks, T = 1)."""
import numpy as np
import pytest

from linear_attention_recurrent_kda_amd import synth
from oracle import kda_oracle_np as onp
from oracle.kda_oracle_np import Layer


def random_case(seed, B, T, H, dk, dv, dtype="f32", state_scale=0.3):
    g = synth.rng(seed)
    p = synth.layer_params(g, H, dk, dv)
    layer = Layer(p["A"], p["conv_wt"], p["norm_w"])
    inp = synth.token_inputs(g, (B, T), H, dk, dv, dtype)
    state = synth.random_state(g, (B, H, dk, dv), state_scale)
    window = synth.window_inputs(g, (B,), H, dk, dv, dtype)
    return layer, state, window, inp


def run_np(layer, state, window, inp, **kw):
    return onp.run(layer, state, window, inp["x_q"], inp["x_k"], inp["x_v"], inp["g"],
                   inp["b"], inp["z"], **kw)


def run_c(oc, layer, state, window, inp, **kw):
    return oc.run(layer, state, window, inp["x_q"], inp["x_k"], inp["x_v"], inp["g"],
                  inp["b"], inp["z"], **kw)


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("dk,dv", [(8, 12), (12, 8), (16, 16)])
def test_c_matches_numpy(oracle_c, dk, dv):
    layer, state, window, inp = random_case(21, 3, 40, 3, dk, dv)
    a = run_c(oracle_c, layer, state, window, inp, snapshots=True)
    b = run_np(layer, state, window, inp, snapshots=True)
    assert rel(a["y"], b["y"]) < 1e-12
    assert rel(a["state"], b["state"]) < 1e-12
    assert rel(a["snap_state"], b["snap_state"]) < 1e-12
    assert np.array_equal(a["window"], b["window"])


def test_c_matches_numpy_bf16_inputs_and_lengths(oracle_c):
    layer, state, window, inp = random_case(22, 4, 9, 2, 16, 16, dtype="bf16")
    lens = np.array([9, 0, 4, 1], dtype=np.int32)
    a = run_c(oracle_c, layer, state, window, inp, lens=lens)
    b = run_np(layer, state, window, inp, lens=lens)
    for bi, n in enumerate(lens):
        if n:
            assert rel(a["y"][bi, :n], b["y"][bi, :n]) < 1e-12
    assert rel(a["state"], b["state"]) < 1e-12
    assert np.array_equal(a["window"], b["window"])
    # a shortened sequence equals the same sequence run for only its length
    for bi, n in enumerate(lens):
        sub = {k: v[bi:bi + 1, :n] for k, v in inp.items()}
        c = run_c(oracle_c, layer, state[bi:bi + 1], window[bi:bi + 1], sub)
        assert np.array_equal(c["state"][0], a["state"][bi])
        assert np.array_equal(c["window"][0], a["window"][bi])


def test_sequences_independent_of_batch(oracle_c):
    layer, state, window, inp = random_case(23, 5, 6, 2, 8, 8)
    full = run_c(oracle_c, layer, state, window, inp)
    for bi in (0, 3):
        sub = {k: v[bi:bi + 1] for k, v in inp.items()}
        one = run_c(oracle_c, layer, state[bi:bi + 1], window[bi:bi + 1], sub)
        assert np.array_equal(one["y"][0], full["y"][bi])
        assert np.array_equal(one["state"][0], full["state"][bi])


def test_snapshots_are_prefix_states(oracle_c):
    layer, state, window, inp = random_case(24, 2, 5, 2, 8, 8)
    full = run_c(oracle_c, layer, state, window, inp, snapshots=True)
    for t in range(5):
        sub = {k: v[:, :t + 1] for k, v in inp.items()}
        pre = run_c(oracle_c, layer, state, window, sub)
        assert np.array_equal(full["snap_state"][:, t], pre["state"])
        assert np.array_equal(full["snap_window"][:, t], pre["window"])


def test_heads_are_independent(oracle_c):
    layer, state, window, inp = random_case(25, 1, 7, 4, 8, 8)
    full = run_c(oracle_c, layer, state, window, inp)
    idx = [2, 0]
    sub = {k: v[:, :, idx] for k, v in inp.items()}
    part = run_c(oracle_c, layer.heads(idx), state[:, idx], window[:, idx], sub)
    assert np.array_equal(part["y"], full["y"][:, :, idx])
    assert np.array_equal(part["state"], full["state"][:, idx])


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 130])
@pytest.mark.parametrize("chunk", [16, 64])
def test_chunked_equals_sequential(oracle_c, T, chunk):
    layer, state, window, inp = random_case(30 + T, 1, T, 2, 8, 6)
    seq = run_c(oracle_c, layer, state, window, inp)
    chk = run_np(layer, state, window, inp, chunk=chunk)
    assert rel(chk["y"], seq["y"]) < 1e-12
    assert rel(chk["state"], seq["state"]) < 1e-12


def test_chunked_equals_sequential_strong_decay(oracle_c):
    """Large g drives alpha towards 0 inside a chunk (cumulative log-decay far
    below fp32/fp64 range if factorised naively); the difference form stays exact."""
    layer, state, window, inp = random_case(40, 1, 130, 2, 8, 8)
    inp = dict(inp, g=inp["g"] * 6.0 + 4.0)
    seq = run_c(oracle_c, layer, state, window, inp)
    chk = run_np(layer, state, window, inp, chunk=64)
    assert rel(chk["y"], seq["y"]) < 1e-11
    assert rel(chk["state"], seq["state"]) < 1e-11
