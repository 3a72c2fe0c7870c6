"""Python binding of libkda.so: the entry points of include/kda.h under the
same names, taking torch tensors.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity (the C ABI sees bare pointers and cannot check sizes), their device
pointers and torch's current HIP stream are passed through, and a non-OK
status raises ``KdaError``.  All computation happens in the HIP kernels.
"""
from __future__ import annotations

import ctypes
import threading
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib


class KdaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        self.status = _lib.STATUS.get(code, str(code))
        super().__init__(f"{fn}: {self.status} ({kda_status_string(code)})")


@dataclass
class Layer:
    """Parameters of one KDA layer: A [H, d_k], conv_wt [H, 2 d_k + d_v, 4],
    norm_w [H, d_v], all fp32 device tensors."""
    A: torch.Tensor
    conv_wt: torch.Tensor
    norm_w: torch.Tensor
    q_scale: Optional[float] = None     # default d_k ** -0.5
    l2_eps: float = 1e-6
    rms_eps: float = 1e-6
    conv_silu: bool = True
    stream_state: bool = False          # non-temporal state traffic (KDA_STREAM_STATE)
    state_resident: bool = False        # decode: states stay cache-resident (KDA_STATE_RESIDENT)

    @property
    def H(self):
        return self.A.shape[0]

    @property
    def d_k(self):
        return self.A.shape[1]

    @property
    def d_v(self):
        return self.norm_w.shape[1]

    @property
    def conv_w(self):
        return self.conv_wt.shape[2]

    def c_struct(self) -> _lib.KdaLayer:
        for name in ("A", "conv_wt", "norm_w"):
            _check(getattr(self, name), name, torch.float32)
        H, dk, dv = self.H, self.d_k, self.d_v
        if self.conv_wt.dim() != 3 or tuple(self.conv_wt.shape[:2]) != (H, 2 * dk + dv) \
                or tuple(self.norm_w.shape) != (H, dv):
            raise ValueError("layer parameter shapes disagree")
        qs = dk ** -0.5 if self.q_scale is None else self.q_scale
        return _lib.KdaLayer(H, dk, dv, self.conv_w, self.A.data_ptr(), self.conv_wt.data_ptr(),
                             self.norm_w.data_ptr(), qs, self.l2_eps, self.rms_eps,
                             (_lib.KDA_CONV_SILU if self.conv_silu else 0)
                             | (_lib.KDA_STREAM_STATE if self.stream_state else 0)
                             | (_lib.KDA_STATE_RESIDENT if self.state_resident else 0))


@dataclass
class Cache:
    """State pool [n_slots, H, d_k, d_v] fp32 and conv-window pool
    [n_slots, H, conv_w - 1, 2 d_k + d_v] of the input dtype; optional int32
    error flag (one element)."""
    state: torch.Tensor
    conv_state: torch.Tensor
    err_flag: Optional[torch.Tensor] = None

    @property
    def n_slots(self):
        return self.state.shape[0]

    def c_struct(self, layer: Layer) -> _lib.KdaCache:
        _check(self.state, "state", torch.float32)
        _check(self.conv_state, "conv_state")
        if self.conv_state.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError(f"conv_state must be float32 or bfloat16, not {self.conv_state.dtype}")
        H, dk, dv, W = layer.H, layer.d_k, layer.d_v, layer.conv_w
        if tuple(self.state.shape) != (self.n_slots, H, dk, dv):
            raise ValueError(f"state shape {tuple(self.state.shape)} != [n_slots, {H}, {dk}, {dv}]")
        if tuple(self.conv_state.shape) != (self.n_slots, H, W - 1, 2 * dk + dv):
            raise ValueError("conv_state shape must be [n_slots, H, conv_w-1, 2 d_k + d_v]")
        ef = None
        if self.err_flag is not None:
            _check(self.err_flag, "err_flag", torch.int32)
            ef = self.err_flag.data_ptr()
        return _lib.KdaCache(self.state.data_ptr(), self.conv_state.data_ptr(), self.n_slots, ef)


@dataclass
class Inputs:
    """Per-token inputs, fp32 or bf16 device tensors: x_q, x_k, g [..., H, d_k];
    x_v, z [..., H, d_v]; b [..., H]."""
    x_q: torch.Tensor
    x_k: torch.Tensor
    x_v: torch.Tensor
    g: torch.Tensor
    b: torch.Tensor
    z: torch.Tensor

    @property
    def dtype(self):
        return self.x_q.dtype

    def c_struct(self, layer: Layer, lead: tuple) -> _lib.KdaInputs:
        dt = self.x_q.dtype
        if dt not in (torch.float32, torch.bfloat16):
            raise TypeError(f"inputs must be float32 or bfloat16, not {dt}")
        H, dk, dv = layer.H, layer.d_k, layer.d_v
        want = dict(x_q=(H, dk), x_k=(H, dk), g=(H, dk), x_v=(H, dv), z=(H, dv), b=(H,))
        for name, tail in want.items():
            t = getattr(self, name)
            _check(t, name, dt)
            if tuple(t.shape) != tuple(lead) + tail:
                raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(lead) + tail}")
        code = _lib.KDA_BF16 if dt == torch.bfloat16 else _lib.KDA_F32
        return _lib.KdaInputs(self.x_q.data_ptr(), self.x_k.data_ptr(), self.x_v.data_ptr(),
                              self.g.data_ptr(), self.b.data_ptr(), self.z.data_ptr(), code)


def _check(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _raise(fn: str, code: int):
    if code != 0:
        raise KdaError(fn, code)


# While prepared() runs an entry point on a thread, the marshalled C call is
# recorded here (per thread) instead of being issued.
_tls = threading.local()


def _call(name: str, *args, keep=None) -> None:
    """Issue C entry point `name` with marshalled arguments (or record it;
    `keep` holds objects the recorded call needs alive, e.g. a workspace
    allocated here)."""
    rec = getattr(_tls, "recording", None)
    if rec is not None:
        rec.append((name, args, keep))
        return
    _raise(name, getattr(_lib.load(), name)(*args))


def prepared(entry, *args, **kwargs):
    """Check and marshal one call of a launching entry point of this module
    (kda_decode, kda_spec_verify, kda_spec_commit, kda_spec_verify_delta,
    kda_spec_commit_delta, kda_chunk_prefill, kda_chunk_prefill_ckpt,
    kda_chunk_prefill_static, kda_build_metadata) once,
    without launching it; return a zero-argument callable that issues exactly
    that C call again each time (for launch loops where per-call Python
    overhead would leave the GPU idle).  The callable keeps the arguments
    alive and raises KdaError on a non-OK status.  The stream is fixed at
    preparation (the current stream unless `stream=` is given)."""
    if getattr(_tls, "recording", None) is not None:
        raise RuntimeError("prepared() does not nest")
    rec = _tls.recording = []
    try:
        entry(*args, **kwargs)
    finally:
        _tls.recording = None
    if len(rec) != 1:
        raise ValueError(f"{getattr(entry, '__name__', entry)} does not issue exactly one C call")
    name, cargs, held = rec[0]
    fn = getattr(_lib.load(), name)

    def call():
        rc = fn(*cargs)
        if rc:
            raise KdaError(name, rc)
    call.keep = (args, kwargs, cargs, held)
    return call


def kda_decode(layer: Layer, cache: Cache, slot_idx: torch.Tensor, inputs: Inputs,
               y: torch.Tensor, stream=None) -> None:
    """One token per sequence; slot_idx [B] int32, inputs [B, H, .], y [B, H, d_v]."""
    _check(slot_idx, "slot_idx", torch.int32)
    B = slot_idx.numel()
    _check(y, "y", torch.float32)
    if tuple(y.shape) != (B, layer.H, layer.d_v):
        raise ValueError("y must be [B, H, d_v]")
    L, C, I = layer.c_struct(), cache.c_struct(layer), inputs.c_struct(layer, (B,))
    if cache.conv_state.dtype != inputs.dtype:
        raise TypeError("conv_state dtype must equal the input dtype")
    _call("kda_decode", ctypes.byref(L), ctypes.byref(C), slot_idx.data_ptr(),
          B, ctypes.byref(I), y.data_ptr(), _stream(stream))


def kda_decode_prepared(layer: Layer, cache: Cache, slot_idx: torch.Tensor, inputs: Inputs,
                        y: torch.Tensor, stream=None):
    """prepared(kda_decode, ...): a zero-argument callable issuing this call."""
    return prepared(kda_decode, layer, cache, slot_idx, inputs, y, stream=stream)


def kda_spec_verify(layer: Layer, cache: Cache, slot_idx: torch.Tensor, snap_slots: torch.Tensor,
                    inputs: Inputs, y: torch.Tensor, draft_len: Optional[torch.Tensor] = None,
                    stream=None) -> None:
    """T draft tokens per sequence: snap_slots [B, T] int32, inputs [B, T, H, .],
    y [B, T, H, d_v]; draft_len [B] int32 or None."""
    _check(slot_idx, "slot_idx", torch.int32)
    _check(snap_slots, "snap_slots", torch.int32)
    B = slot_idx.numel()
    if snap_slots.dim() != 2 or snap_slots.shape[0] != B:
        raise ValueError("snap_slots must be [B, T]")
    T = snap_slots.shape[1]
    _check(y, "y", torch.float32)
    if tuple(y.shape) != (B, T, layer.H, layer.d_v):
        raise ValueError("y must be [B, T, H, d_v]")
    dl = None
    if draft_len is not None:
        _check(draft_len, "draft_len", torch.int32)
        if draft_len.numel() != B:
            raise ValueError("draft_len must be [B]")
        dl = draft_len.data_ptr()
    L, C, I = layer.c_struct(), cache.c_struct(layer), inputs.c_struct(layer, (B, T))
    if cache.conv_state.dtype != inputs.dtype:
        raise TypeError("conv_state dtype must equal the input dtype")
    _call("kda_spec_verify",
          ctypes.byref(L), ctypes.byref(C), slot_idx.data_ptr(), snap_slots.data_ptr(), B, T, dl,
          ctypes.byref(I), y.data_ptr(), _stream(stream))


def kda_spec_commit(layer: Layer, cache: Cache, slot_idx: torch.Tensor, snap_slots: torch.Tensor,
                    accepted_len: torch.Tensor, stream=None) -> None:
    """Copy snapshot accepted_len[b]-1 of each sequence into its live slot."""
    _check(slot_idx, "slot_idx", torch.int32)
    _check(snap_slots, "snap_slots", torch.int32)
    _check(accepted_len, "accepted_len", torch.int32)
    B = slot_idx.numel()
    if snap_slots.dim() != 2 or snap_slots.shape[0] != B or accepted_len.numel() != B:
        raise ValueError("snap_slots must be [B, T] and accepted_len [B]")
    T = snap_slots.shape[1]
    L, C = layer.c_struct(), cache.c_struct(layer)
    wdt = _dtype_code(cache.conv_state.dtype)
    _call("kda_spec_commit",
          ctypes.byref(L), ctypes.byref(C), slot_idx.data_ptr(), snap_slots.data_ptr(),
          accepted_len.data_ptr(), B, T, wdt, _stream(stream))


def _dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return _lib.KDA_BF16
    if dt == torch.float32:
        return _lib.KDA_F32
    raise TypeError(f"inputs must be float32 or bfloat16, not {dt}")


def kda_spec_delta_bytes(layer: Layer, B: int, T: int, dtype=torch.bfloat16) -> int:
    """Bytes of the replay-record buffer of B sequences x T draft tokens."""
    L = layer.c_struct()
    return int(_lib.load().kda_spec_delta_bytes(ctypes.byref(L), B, T, _dtype_code(dtype)))


def new_spec_delta(layer: Layer, B: int, T: int, dtype=torch.bfloat16, device="cuda") -> torch.Tensor:
    """An uninitialised record buffer, uint8 [B, T, H, record_bytes]."""
    n = kda_spec_delta_bytes(layer, B, T, dtype)
    if n == 0 and B > 0:
        raise ValueError("invalid sizes for a record buffer")
    rec = n // max(B * T * layer.H, 1)
    return torch.empty((B, T, layer.H, rec), dtype=torch.uint8, device=device)


def _delta_buf(delta: torch.Tensor, B: int):
    _check(delta, "delta", torch.uint8)
    if delta.dim() != 4 or delta.shape[0] != B:
        raise ValueError("delta must be a [B, T, H, record_bytes] uint8 buffer (new_spec_delta)")
    return delta.shape[1], delta.numel()


def kda_spec_verify_delta(layer: Layer, cache: Cache, slot_idx: torch.Tensor, inputs: Inputs,
                          y: torch.Tensor, delta: torch.Tensor, draft_len: Optional[torch.Tensor] = None,
                          stream=None) -> None:
    """Verification with replay records instead of snapshots: inputs
    [B, T, H, .], y [B, T, H, d_v], delta from new_spec_delta(layer, B, T)."""
    _check(slot_idx, "slot_idx", torch.int32)
    B = slot_idx.numel()
    T, nbytes = _delta_buf(delta, B)
    _check(y, "y", torch.float32)
    if tuple(y.shape) != (B, T, layer.H, layer.d_v):
        raise ValueError("y must be [B, T, H, d_v]")
    dl = None
    if draft_len is not None:
        _check(draft_len, "draft_len", torch.int32)
        if draft_len.numel() != B:
            raise ValueError("draft_len must be [B]")
        dl = draft_len.data_ptr()
    L, C, I = layer.c_struct(), cache.c_struct(layer), inputs.c_struct(layer, (B, T))
    if cache.conv_state.dtype != inputs.dtype:
        raise TypeError("conv_state dtype must equal the input dtype")
    _call("kda_spec_verify_delta",
          ctypes.byref(L), ctypes.byref(C), slot_idx.data_ptr(), B, T, dl, ctypes.byref(I),
          y.data_ptr(), delta.data_ptr(), nbytes, _stream(stream))


def kda_spec_commit_delta(layer: Layer, cache: Cache, slot_idx: torch.Tensor, delta: torch.Tensor,
                          accepted_len: torch.Tensor, stream=None) -> None:
    """Replay the first accepted_len[b] records of each sequence onto its live slot."""
    _check(slot_idx, "slot_idx", torch.int32)
    _check(accepted_len, "accepted_len", torch.int32)
    B = slot_idx.numel()
    if accepted_len.numel() != B:
        raise ValueError("accepted_len must be [B]")
    T, nbytes = _delta_buf(delta, B)
    L, C = layer.c_struct(), cache.c_struct(layer)
    _call("kda_spec_commit_delta",
          ctypes.byref(L), ctypes.byref(C), slot_idx.data_ptr(), delta.data_ptr(), nbytes,
          accepted_len.data_ptr(), B, T, _dtype_code(cache.conv_state.dtype), _stream(stream))


def kda_chunk_prefill_workspace_bytes(layer: Layer, total_T: int, N_seq: int, chunk: int = 64) -> int:
    L = layer.c_struct()
    return int(_lib.load().kda_chunk_prefill_workspace_bytes(ctypes.byref(L), total_T, N_seq, chunk))


def _prefill_args(layer, cache, slot_idx, cu_seqlens, inputs, y, workspace, chunk, stream):
    _check(slot_idx, "slot_idx", torch.int32)
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    N = slot_idx.numel()
    if cu_seqlens.numel() != N + 1:
        raise ValueError("cu_seqlens must be [N_seq + 1]")
    total_T = inputs.x_q.shape[0]
    _check(y, "y", torch.float32)
    if tuple(y.shape) != (total_T, layer.H, layer.d_v):
        raise ValueError("y must be [total_T, H, d_v]")
    L, C, I = layer.c_struct(), cache.c_struct(layer), inputs.c_struct(layer, (total_T,))
    if cache.conv_state.dtype != inputs.dtype:
        raise TypeError("conv_state dtype must equal the input dtype")
    need = int(_lib.load().kda_chunk_prefill_workspace_bytes(ctypes.byref(L), total_T, N, chunk))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=y.device)
        # allocated on the current stream, used on the launch stream: keep the
        # caching allocator from handing it out again before the call is done
        if stream is not None:
            workspace.record_stream(stream)
    wp, wb = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    return L, C, I, N, total_T, wp, wb, workspace


def kda_chunk_prefill(layer: Layer, cache: Cache, slot_idx: torch.Tensor, cu_seqlens: torch.Tensor,
                      inputs: Inputs, y: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                      chunk: int = 64, stream=None) -> None:
    """Chunked prefill of N_seq sequences packed along the token axis:
    slot_idx [N_seq], cu_seqlens [N_seq + 1] int32, inputs [total_T, H, .],
    y [total_T, H, d_v].  A workspace of the size query's bytes is allocated
    here (torch) when none is given."""
    L, C, I, N, total_T, wp, wb, keep = _prefill_args(layer, cache, slot_idx, cu_seqlens, inputs, y,
                                                      workspace, chunk, stream)
    _call("kda_chunk_prefill",
          ctypes.byref(L), ctypes.byref(C), slot_idx.data_ptr(), cu_seqlens.data_ptr(), N, total_T,
          chunk, ctypes.byref(I), y.data_ptr(), wp, wb, _stream(stream), keep=keep)


def kda_chunk_prefill_static(layer: Layer, cache: Cache, slot_idx: torch.Tensor, cu_seqlens: torch.Tensor,
                             inputs: Inputs, y: torch.Tensor, chunk: int = 64, stream=None) -> None:
    """kda_chunk_prefill in the library's static workspace: nothing is
    allocated (for callers under graph capture or that may not allocate);
    calls whose workspace exceeds KDA_STATIC_WORKSPACE_BYTES raise
    KdaError (KDA_ERR_WORKSPACE).  Calls overlapping on one GPU race."""
    _check(slot_idx, "slot_idx", torch.int32)
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    N = slot_idx.numel()
    if cu_seqlens.numel() != N + 1:
        raise ValueError("cu_seqlens must be [N_seq + 1]")
    total_T = inputs.x_q.shape[0]
    _check(y, "y", torch.float32)
    if tuple(y.shape) != (total_T, layer.H, layer.d_v):
        raise ValueError("y must be [total_T, H, d_v]")
    L, C, I = layer.c_struct(), cache.c_struct(layer), inputs.c_struct(layer, (total_T,))
    if cache.conv_state.dtype != inputs.dtype:
        raise TypeError("conv_state dtype must equal the input dtype")
    _call("kda_chunk_prefill_static",
          ctypes.byref(L), ctypes.byref(C), slot_idx.data_ptr(), cu_seqlens.data_ptr(), N, total_T,
          chunk, ctypes.byref(I), y.data_ptr(), _stream(stream))


def kda_chunk_prefill_ckpt(layer: Layer, cache: Cache, slot_idx: torch.Tensor, cu_seqlens: torch.Tensor,
                           inputs: Inputs, y: torch.Tensor, ckpt_slots: torch.Tensor, ckpt_interval: int,
                           workspace: Optional[torch.Tensor] = None, chunk: int = 64, stream=None) -> None:
    """kda_chunk_prefill plus interval checkpoints: ckpt_slots [N_seq, per_seq]
    int32; the state and window after (j+1)*ckpt_interval tokens of sequence
    s go to ckpt_slots[s, j] (-1: not kept)."""
    _check(ckpt_slots, "ckpt_slots", torch.int32)
    if ckpt_slots.dim() != 2 or ckpt_slots.shape[0] != slot_idx.numel():
        raise ValueError("ckpt_slots must be [N_seq, per_seq]")
    L, C, I, N, total_T, wp, wb, keep = _prefill_args(layer, cache, slot_idx, cu_seqlens, inputs, y,
                                                      workspace, chunk, stream)
    _call("kda_chunk_prefill_ckpt",
          ctypes.byref(L), ctypes.byref(C), slot_idx.data_ptr(), cu_seqlens.data_ptr(), N, total_T,
          chunk, ctypes.byref(I), y.data_ptr(), ckpt_slots.data_ptr(), int(ckpt_interval),
          int(ckpt_slots.shape[1]), wp, wb, _stream(stream), keep=keep)


def kda_build_metadata(num_tokens: torch.Tensor, req_slot: torch.Tensor, n_slots: int,
                       cu_seqlens: torch.Tensor, slot_idx: torch.Tensor, chunk_start: torch.Tensor,
                       counts: torch.Tensor, err_flag: Optional[torch.Tensor] = None, stream=None) -> None:
    """Per-step batch tables from per-request token counts and slots (all
    int32 device tensors): cu_seqlens [n + 1], slot_idx [n], chunk_start
    [n + 1], counts [4] (total tokens, one-token rows, prompts, chunks)."""
    for name, t in (("num_tokens", num_tokens), ("req_slot", req_slot), ("cu_seqlens", cu_seqlens),
                    ("slot_idx", slot_idx), ("chunk_start", chunk_start), ("counts", counts)):
        _check(t, name, torch.int32)
    n = num_tokens.numel()
    if req_slot.numel() != n or slot_idx.numel() != n or cu_seqlens.numel() != n + 1 \
            or chunk_start.numel() != n + 1 or counts.numel() != 4:
        raise ValueError("table sizes must be [n], [n], [n + 1], [n], [n + 1], [4]")
    ef = None
    if err_flag is not None:
        _check(err_flag, "err_flag", torch.int32)
        ef = err_flag.data_ptr()
    _call("kda_build_metadata", num_tokens.data_ptr(), req_slot.data_ptr(), n, int(n_slots),
          cu_seqlens.data_ptr(), slot_idx.data_ptr(), chunk_start.data_ptr(), counts.data_ptr(), ef,
          _stream(stream))


def kda_copy_probe(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    """dst[i] = src[i]; dst may be src itself (an in-place read and rewrite)."""
    _check(dst, "dst", torch.float32)
    _check(src, "src", torch.float32)
    if dst.numel() != src.numel():
        raise ValueError("dst and src sizes differ")
    _call("kda_copy_probe", dst.data_ptr(), src.data_ptr(), src.numel(), _stream(stream))


def kda_status_string(code: int) -> str:
    return _lib.load().kda_status_string(int(code)).decode()


def kda_abi_version() -> int:
    return int(_lib.load().kda_abi_version())
