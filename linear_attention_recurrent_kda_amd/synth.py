"""Seeded synthetic inputs for the KDA recurrent-state path.

This module holds data generation only (random draws, dtype rounding, the
workload shapes); none of the method's arithmetic.  Both the HIP path's tests
and benchmark and the oracle's tests draw their inputs from here, so the two
sides always see the same values.

Distributions (the workload descriptions that accompany the pages' KDA
decode/prefill discussion): q/k/v, decay logits g, beta logits b and output
gate z ~ N(0, 1); conv weights ~ N(0, 0.5^2) (read as standard deviation 0.5);
decay log-rate A ~ U(-1, 0) per (head, key channel); RMSNorm weight 1.
Generator: NumPy PCG64 seeded per workload; bf16 values are float32 draws
rounded to nearest-even and kept as float32 that hold them exactly.
"""
from __future__ import annotations

import numpy as np

CONV_W = 4

# Named workloads.  Shapes follow the decode / verify / prefill workloads the
# pages' serving numbers are quoted on: batch 1 and batch 64 decode, 8 draft
# tokens per verification, long chunked prefill.
WORKLOADS = {
    "tiny_recurrence": dict(B=1, H=4, d_k=64, d_v=64, T=256, dtype="f32", seed=101),
    "decode_b1": dict(B=1, H=32, d_k=128, d_v=128, n_slots=256, warmup=512, dtype="bf16", seed=102),
    "decode_b64": dict(B=64, H=32, d_k=128, d_v=128, n_slots=1024, steps=100, dtype="bf16", seed=103),
    "spec_verify_b16_t8": dict(B=16, T=8, H=32, d_k=128, d_v=128, dtype="bf16", seed=104),
    "prefill_t32k": dict(B=1, T=32768, H=32, d_k=128, d_v=128, chunk=64, dtype="bf16", seed=105),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); the result
    is float32 holding the bf16 value exactly.  Infinities pass through."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32)
    return np.where(np.isinf(f), f, out).astype(np.float32)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of float32 values that already hold bf16 values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def to_dtype(x, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def layer_params(g: np.random.Generator, H: int, d_k: int, d_v: int, conv_w: int = CONV_W):
    """A [H, d_k], conv_wt [H, 2 d_k + d_v, conv_w], norm_w [H, d_v]; fp32."""
    A = g.uniform(-1.0, 0.0, size=(H, d_k)).astype(np.float32)
    conv_wt = (0.5 * g.standard_normal((H, 2 * d_k + d_v, conv_w))).astype(np.float32)
    norm_w = np.ones((H, d_v), dtype=np.float32)
    return dict(A=A, conv_wt=conv_wt, norm_w=norm_w)


def token_inputs(g: np.random.Generator, lead: tuple, H: int, d_k: int, d_v: int, dtype: str):
    """Per-token inputs with leading shape ``lead`` (e.g. (B,) or (B, T)):
    x_q, x_k, g [*lead, H, d_k]; x_v, z [*lead, H, d_v]; b [*lead, H]."""
    lead = tuple(lead)
    out = {}
    for name, shape in (("x_q", (H, d_k)), ("x_k", (H, d_k)), ("x_v", (H, d_v)),
                        ("g", (H, d_k)), ("b", (H,)), ("z", (H, d_v))):
        out[name] = to_dtype(g.standard_normal(lead + shape, dtype=np.float32), dtype)
    return out


def random_state(g: np.random.Generator, shape, scale: float = 0.1) -> np.ndarray:
    """A dense fp32 state of modest magnitude (for parity cases that start
    from a non-zero state without running a warm-up)."""
    return (scale * g.standard_normal(shape, dtype=np.float32)).astype(np.float32)


def window_inputs(g: np.random.Generator, lead: tuple, H: int, d_k: int, d_v: int,
                  dtype: str, conv_w: int = CONV_W) -> np.ndarray:
    """A conv window [*lead, H, conv_w-1, 2 d_k + d_v] of raw past inputs."""
    x = g.standard_normal(tuple(lead) + (H, conv_w - 1, 2 * d_k + d_v), dtype=np.float32)
    return to_dtype(x, dtype)


def slot_table(g: np.random.Generator, B: int, n_slots: int) -> np.ndarray:
    """B distinct slots drawn from a pool of n_slots (a random permutation's
    first B entries), int32."""
    return g.permutation(n_slots)[:B].astype(np.int32)


def accepted_lengths(g: np.random.Generator, B: int, T: int) -> np.ndarray:
    """Accepted draft lengths ~ U{1..T}, int32."""
    return g.integers(1, T + 1, size=B).astype(np.int32)
