"""Helpers for the GPU tests: move seeded synthetic arrays to the device in
the layouts the C ABI expects, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

from linear_attention_recurrent_kda_amd import api, synth
from oracle.kda_oracle_np import Layer as OracleLayer

DEV = "cuda:0"
TOL = 2e-3   # max |GPU - oracle| <= TOL * RMS(oracle output), per step


def tdt(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a, dtype=torch.float32):
    """float32 numpy (holding values exact in `dtype`) -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype).contiguous()


def layer_pair(params, q_scale=None, l2_eps=1e-6, rms_eps=1e-6, silu=True):
    """(device api.Layer, oracle Layer) from synth.layer_params output."""
    dl = api.Layer(to_dev(params["A"]), to_dev(params["conv_wt"]), to_dev(params["norm_w"]),
                   q_scale, l2_eps, rms_eps, silu)
    ol = OracleLayer(params["A"], params["conv_wt"], params["norm_w"], q_scale, l2_eps, rms_eps, silu)
    return dl, ol


def inputs_dev(inp: dict, dtype: str, sl=None) -> api.Inputs:
    """Device inputs from a synth.token_inputs dict; `sl` indexes the leading axes."""
    dt = tdt(dtype)
    pick = (lambda a: a) if sl is None else (lambda a: a[sl])
    return api.Inputs(*(to_dev(pick(inp[k]), dt) for k in ("x_q", "x_k", "x_v", "g", "b", "z")))


def new_cache(n_slots, H, dk, dv, dtype: str, fill_seed=None, W=4):
    """A cache pool; with fill_seed every slot holds seeded sentinel values."""
    if fill_seed is None:
        state = torch.zeros((n_slots, H, dk, dv), dtype=torch.float32, device=DEV)
        win = torch.zeros((n_slots, H, W - 1, 2 * dk + dv), dtype=tdt(dtype), device=DEV)
    else:
        gen = torch.Generator(device=DEV)
        gen.manual_seed(fill_seed)
        state = torch.randn((n_slots, H, dk, dv), generator=gen, device=DEV) * 0.05
        win = torch.randn((n_slots, H, W - 1, 2 * dk + dv), generator=gen, device=DEV).to(tdt(dtype))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    return api.Cache(state, win, err)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def parity_error(y_gpu, y_orc):
    """max |Δ| / RMS(oracle) over one step's output tensor."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_orc = np.asarray(y_orc, dtype=np.float64)
    rms = np.sqrt(np.mean(y_orc ** 2))
    return float(np.max(np.abs(y_gpu - y_orc)) / rms)


def state_rel_err(s_gpu, s_orc):
    """Largest per-head relative Frobenius error of a state tensor [..., d_k, d_v]."""
    d = np.sqrt(np.sum((np.asarray(s_gpu) - s_orc) ** 2, axis=(-1, -2)))
    n = np.sqrt(np.sum(np.asarray(s_orc) ** 2, axis=(-1, -2)))
    return float(np.max(d / np.maximum(n, 1e-30)))
