"""ctypes front end of the C fp64 oracle (``kda_oracle.c``).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
benchmark)."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .kda_oracle_np import Layer  # parameter container only; no arithmetic used

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KDA_ORACLE_LIB", os.path.join(HERE, "libkda_oracle.so"))

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


class _CLayer(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int), ("d_k", ctypes.c_int), ("d_v", ctypes.c_int),
                ("conv_w", ctypes.c_int), ("A", _dp), ("conv_wt", _dp), ("norm_w", _dp),
                ("q_scale", ctypes.c_double), ("l2_eps", ctypes.c_double),
                ("rms_eps", ctypes.c_double), ("conv_silu", ctypes.c_int)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from .build import build
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        _lib.kda_oracle_run.restype = ctypes.c_int
        _lib.kda_oracle_run.argtypes = [ctypes.POINTER(_CLayer), ctypes.c_int, ctypes.c_int,
                                        _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _ip,
                                        _dp, ctypes.c_int, _dp, _dp, ctypes.c_int]
        _lib.kda_oracle_threads.restype = ctypes.c_int
        _lib.kda_oracle_threads.argtypes = [ctypes.c_int]
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def threads(n_threads: int = 0) -> int:
    return lib().kda_oracle_threads(n_threads)


def run(layer: Layer, state, window, x_q, x_k, x_v, g, b, z, lens=None,
        y_tokens=None, snapshots=False, n_threads: int = 0):
    """Run T tokens of B sequences through the C oracle.

    state [B,H,d_k,d_v]; window [B,H,W-1,C_h]; x_q,x_k,g [B,T,H,d_k];
    x_v,z [B,T,H,d_v]; b [B,T,H].  Returns a dict with y [B,y_tokens,H,d_v],
    the final state and window, and the per-token snapshots if asked."""
    st = _f64(state).copy()
    win = _f64(window).copy()
    xq, xk, xv, gg, bb, zz = (_f64(a) for a in (x_q, x_k, x_v, g, b, z))
    B, T = xq.shape[:2]
    H, dk, dv, W = layer.H, layer.d_k, layer.d_v, layer.conv_w
    Ch = 2 * dk + dv
    assert st.shape == (B, H, dk, dv) and win.shape == (B, H, W - 1, Ch)
    assert xq.shape == (B, T, H, dk) and xk.shape == xq.shape and gg.shape == xq.shape
    assert xv.shape == (B, T, H, dv) and zz.shape == xv.shape and bb.shape == (B, T, H)
    yt = T if y_tokens is None else int(y_tokens)
    y = np.zeros((B, yt, H, dv))
    ss = np.zeros((B, T, H, dk, dv)) if snapshots else None
    sw = np.zeros((B, T, H, W - 1, Ch)) if snapshots else None
    ln = None if lens is None else np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    cl = _CLayer(H, dk, dv, W, _p(layer.A), _p(layer.conv_wt), _p(layer.norm_w),
                 layer.q_scale, layer.l2_eps, layer.rms_eps, int(layer.conv_silu))
    rc = lib().kda_oracle_run(ctypes.byref(cl), B, T, _p(st), _p(win), _p(xq), _p(xk),
                              _p(xv), _p(gg), _p(bb), _p(zz),
                              None if ln is None else ln.ctypes.data_as(_ip),
                              _p(y), yt, _p(ss), _p(sw), int(n_threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_run failed ({rc})")
    return dict(y=y, state=st, window=win, snap_state=ss, snap_window=sw)
