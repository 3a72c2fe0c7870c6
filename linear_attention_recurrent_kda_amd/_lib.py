"""ctypes view of libkda.so (the C ABI in include/kda.h).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_F32 = 0
KDA_BF16 = 1
KDA_CONV_SILU = 1
KDA_STREAM_STATE = 2
KDA_STATE_RESIDENT = 4
KDA_STATIC_WORKSPACE_BYTES = 256 << 20

STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
          4: "KDA_ERR_ALIGN", 5: "KDA_ERR_UNSUPPORTED", 6: "KDA_ERR_WORKSPACE",
          7: "KDA_ERR_LAUNCH", 8: "KDA_ERR_ALIAS"}

# every function include/kda.h declares
EXPORTS = ("kda_decode", "kda_spec_verify", "kda_spec_commit", "kda_spec_delta_bytes",
           "kda_spec_verify_delta", "kda_spec_commit_delta", "kda_chunk_prefill", "kda_chunk_prefill_ckpt",
           "kda_chunk_prefill_static",
           "kda_chunk_prefill_workspace_bytes", "kda_build_metadata", "kda_copy_probe",
           "kda_status_string", "kda_abi_version")


class KdaLayer(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("conv_w", ctypes.c_int32), ("A", ctypes.c_void_p), ("conv_wt", ctypes.c_void_p),
                ("norm_w", ctypes.c_void_p), ("q_scale", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


class KdaCache(ctypes.Structure):
    _fields_ = [("state", ctypes.c_void_p), ("conv_state", ctypes.c_void_p),
                ("n_slots", ctypes.c_int32), ("err_flag", ctypes.c_void_p)]


class KdaInputs(ctypes.Structure):
    _fields_ = [("x_q", ctypes.c_void_p), ("x_k", ctypes.c_void_p), ("x_v", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("b", ctypes.c_void_p), ("z", ctypes.c_void_p),
                ("dtype", ctypes.c_int)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so once.  torch is imported first so that the library binds
    to the HIP runtime torch already uses (one runtime per process)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(there is no fallback implementation)")
    import torch  # noqa: F401  (binds the process to torch's HIP runtime first)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode.argtypes = [ctypes.POINTER(KdaLayer), ctypes.POINTER(KdaCache), P, i32,
                               ctypes.POINTER(KdaInputs), P, P]
    lib.kda_spec_verify.restype = ctypes.c_int
    lib.kda_spec_verify.argtypes = [ctypes.POINTER(KdaLayer), ctypes.POINTER(KdaCache), P, P,
                                    i32, i32, P, ctypes.POINTER(KdaInputs), P, P]
    lib.kda_spec_commit.restype = ctypes.c_int
    lib.kda_spec_commit.argtypes = [ctypes.POINTER(KdaLayer), ctypes.POINTER(KdaCache), P, P, P,
                                    i32, i32, ctypes.c_int, P]
    lib.kda_spec_delta_bytes.restype = ctypes.c_size_t
    lib.kda_spec_delta_bytes.argtypes = [ctypes.POINTER(KdaLayer), i32, i32, ctypes.c_int]
    lib.kda_spec_verify_delta.restype = ctypes.c_int
    lib.kda_spec_verify_delta.argtypes = [ctypes.POINTER(KdaLayer), ctypes.POINTER(KdaCache), P, i32, i32,
                                          P, ctypes.POINTER(KdaInputs), P, P, ctypes.c_size_t, P]
    lib.kda_spec_commit_delta.restype = ctypes.c_int
    lib.kda_spec_commit_delta.argtypes = [ctypes.POINTER(KdaLayer), ctypes.POINTER(KdaCache), P, P,
                                          ctypes.c_size_t, P, i32, i32, ctypes.c_int, P]
    lib.kda_chunk_prefill.restype = ctypes.c_int
    lib.kda_chunk_prefill.argtypes = [ctypes.POINTER(KdaLayer), ctypes.POINTER(KdaCache), P, P,
                                      i32, i32, i32, ctypes.POINTER(KdaInputs), P, P,
                                      ctypes.c_size_t, P]
    lib.kda_chunk_prefill_ckpt.restype = ctypes.c_int
    lib.kda_chunk_prefill_ckpt.argtypes = [ctypes.POINTER(KdaLayer), ctypes.POINTER(KdaCache), P, P,
                                           i32, i32, i32, ctypes.POINTER(KdaInputs), P, P, i32, i32, P,
                                           ctypes.c_size_t, P]
    lib.kda_chunk_prefill_static.restype = ctypes.c_int
    lib.kda_chunk_prefill_static.argtypes = [ctypes.POINTER(KdaLayer), ctypes.POINTER(KdaCache), P, P,
                                             i32, i32, i32, ctypes.POINTER(KdaInputs), P, P]
    lib.kda_chunk_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_prefill_workspace_bytes.argtypes = [ctypes.POINTER(KdaLayer), i32, i32, i32]
    lib.kda_build_metadata.restype = ctypes.c_int
    lib.kda_build_metadata.argtypes = [P, P, i32, i32, P, P, P, P, P, P]
    lib.kda_copy_probe.restype = ctypes.c_int
    lib.kda_copy_probe.argtypes = [P, P, ctypes.c_size_t, P]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_abi_version.restype = ctypes.c_int32
    lib.kda_abi_version.argtypes = []
    _lib = lib
    return lib
