"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/kda.h declares, and its host-side validation returns the
documented status codes before any HIP call (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

from linear_attention_recurrent_kda_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

FAKE = 0x10000   # a 16-byte aligned non-null address; never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libkda.so is not built (run __graft_entry__.build())")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 2
    for code in range(9):
        s = lib.kda_status_string(code)
        assert s and s != b"unknown status"
    assert lib.kda_status_string(99) == b"unknown status"


def good_layer(H=4, dk=128, dv=128):
    return _lib.KdaLayer(H, dk, dv, 4, FAKE, FAKE, FAKE, dk ** -0.5, 1e-6, 1e-6, _lib.KDA_CONV_SILU)


def good_cache():
    return _lib.KdaCache(FAKE, FAKE, 16, None)


def good_inputs(dtype=_lib.KDA_BF16):
    return _lib.KdaInputs(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dtype)


def decode(lib, layer=None, cache=None, inputs=None, slots=FAKE, B=2, y=FAKE):
    L = layer or good_layer()
    C = cache or good_cache()
    I = inputs or good_inputs()
    return lib.kda_decode(ctypes.byref(L), ctypes.byref(C), slots, B, ctypes.byref(I), y, None)


def test_decode_validation(lib):
    assert lib.kda_decode(None, ctypes.byref(good_cache()), FAKE, 1, ctypes.byref(good_inputs()), FAKE, None) == 1
    L = good_layer()
    L.A = None
    assert decode(lib, layer=L) == 1
    assert decode(lib, layer=good_layer(dk=32)) == 5
    assert decode(lib, layer=good_layer(dv=96)) == 5
    L = good_layer()
    L.conv_w = 3
    assert decode(lib, layer=L) == 5
    L = good_layer()
    L.flags = 8   # no such flag (1, 2 and 4 are defined)
    assert decode(lib, layer=L) == 5
    L = good_layer()
    L.H = 0
    assert decode(lib, layer=L) == 2
    L = good_layer()
    L.l2_eps = -1.0
    assert decode(lib, layer=L) == 2
    L = good_layer()
    L.q_scale = float("nan")
    assert decode(lib, layer=L) == 2
    L = good_layer()
    L.conv_wt = FAKE + 4
    assert decode(lib, layer=L) == 4
    C = good_cache()
    C.n_slots = 0
    assert decode(lib, cache=C) == 2
    C = good_cache()
    C.state = FAKE + 8
    assert decode(lib, cache=C) == 4
    assert decode(lib, inputs=good_inputs(dtype=7)) == 3
    I = good_inputs()
    I.z = None
    assert decode(lib, inputs=I) == 1
    I = good_inputs()
    I.x_v = FAKE + 2
    assert decode(lib, inputs=I) == 4
    I = good_inputs(_lib.KDA_F32)
    I.b = FAKE + 2
    assert decode(lib, inputs=I) == 4
    assert decode(lib, B=-1) == 2
    assert decode(lib, slots=None) == 1
    assert decode(lib, y=FAKE + 4) == 4
    # B = 0 is a no-op that needs no inputs at all
    assert lib.kda_decode(ctypes.byref(good_layer()), ctypes.byref(good_cache()), None, 0, None, None, None) == 0


def test_spec_validation(lib):
    L, C, I = good_layer(), good_cache(), good_inputs()
    v = lambda B, T, snaps=FAKE, dl=None: lib.kda_spec_verify(
        ctypes.byref(L), ctypes.byref(C), FAKE, snaps, B, T, dl, ctypes.byref(I), FAKE, None)
    assert v(2, 0) == 2
    assert v(2, 17) == 2
    assert v(2, 8, snaps=None) == 1
    assert v(2, 8, dl=FAKE + 2) == 4
    assert v(0, 8) == 0
    c = lambda B, T, wd=_lib.KDA_BF16, acc=FAKE: lib.kda_spec_commit(
        ctypes.byref(L), ctypes.byref(C), FAKE, FAKE, acc, B, T, wd, None)
    assert c(2, 8, wd=5) == 3
    assert c(2, 20) == 2
    assert c(2, 8, acc=None) == 1
    assert c(0, 8) == 0


def test_spec_delta_validation(lib):
    L, C, I = good_layer(), good_cache(), good_inputs()
    rec = (2 * L.d_k + L.d_v) * (4 + 2)      # bf16 inputs: fp32 alpha, k^, d + raw q|k|v
    assert lib.kda_spec_delta_bytes(ctypes.byref(L), 3, 8, _lib.KDA_BF16) == 3 * 8 * L.H * rec
    assert lib.kda_spec_delta_bytes(ctypes.byref(L), 3, 8, _lib.KDA_F32) == 3 * 8 * L.H * (2 * L.d_k + L.d_v) * 8
    assert lib.kda_spec_delta_bytes(ctypes.byref(L), 3, 17, _lib.KDA_BF16) == 0
    assert lib.kda_spec_delta_bytes(ctypes.byref(L), 3, 8, 9) == 0
    need = lib.kda_spec_delta_bytes(ctypes.byref(L), 2, 8, _lib.KDA_BF16)
    v = lambda B, T, d=FAKE, nb=need, dl=None: lib.kda_spec_verify_delta(
        ctypes.byref(L), ctypes.byref(C), FAKE, B, T, dl, ctypes.byref(I), FAKE, d, nb, None)
    assert v(2, 0) == 2
    assert v(2, 17) == 2
    assert v(2, 8, d=None) == 1
    assert v(2, 8, d=FAKE + 4) == 4
    assert v(2, 8, nb=need - 1) == 6
    assert v(2, 8, dl=FAKE + 2) == 4
    assert v(0, 8, d=None) == 0
    c = lambda B, T, d=FAKE, nb=need, acc=FAKE, wd=_lib.KDA_BF16: lib.kda_spec_commit_delta(
        ctypes.byref(L), ctypes.byref(C), FAKE, d, nb, acc, B, T, wd, None)
    assert c(2, 8, wd=5) == 3
    assert c(2, 20) == 2
    assert c(2, 8, acc=None) == 1
    assert c(2, 8, d=None) == 1
    assert c(2, 8, nb=need - 1) == 6
    assert c(2, 8, acc=FAKE + 2) == 4
    assert c(0, 8) == 0


def test_prefill_validation(lib):
    L, C, I = good_layer(), good_cache(), good_inputs()
    p = lambda chunk=64, n=1, T=128, ws=FAKE, wb=1 << 30, cu=FAKE: lib.kda_chunk_prefill(
        ctypes.byref(L), ctypes.byref(C), FAKE, cu, n, T, chunk, ctypes.byref(I), FAKE, ws, wb, None)
    assert p(chunk=32) == 5
    assert p(n=0) == 2
    assert p(T=-1) == 2
    assert p(cu=None) == 1
    need = lib.kda_chunk_prefill_workspace_bytes(ctypes.byref(L), 128, 1, 64)
    if need:
        assert p(wb=need - 1) == 6
        assert p(ws=None) == 1
    assert lib.kda_chunk_prefill_workspace_bytes(ctypes.byref(L), 128, 1, 32) == 0
    # tokens need their input pointers; with no tokens only the dtype is checked
    Inull = good_inputs()
    Inull.x_q = None
    assert lib.kda_chunk_prefill(ctypes.byref(L), ctypes.byref(C), FAKE, FAKE, 1, 128, 64,
                                 ctypes.byref(Inull), FAKE, FAKE, 1 << 30, None) == 1
    Ibad = good_inputs()
    Ibad.dtype = 7
    assert lib.kda_chunk_prefill(ctypes.byref(L), ctypes.byref(C), FAKE, FAKE, 1, 0, 64,
                                 ctypes.byref(Ibad), None, FAKE, 1 << 30, None) == 3


def test_prefill_ckpt_validation(lib):
    L, C, I = good_layer(), good_cache(), good_inputs()
    p = lambda ck=FAKE, iv=128, per=2, chunk=64, n=1, T=128: lib.kda_chunk_prefill_ckpt(
        ctypes.byref(L), ctypes.byref(C), FAKE, FAKE, n, T, chunk, ctypes.byref(I), FAKE, ck, iv, per,
        FAKE, 1 << 30, None)
    assert p(ck=None) == 1
    assert p(ck=FAKE + 2) == 4
    assert p(iv=0) == 2
    assert p(iv=32) == 2
    assert p(iv=96) == 2
    assert p(per=0) == 2
    assert p(chunk=32, iv=64) == 5
    assert p(n=0) == 2


def test_copy_probe_validation(lib):
    assert lib.kda_copy_probe(FAKE, FAKE, 0, None) == 0
    assert lib.kda_copy_probe(None, FAKE, 4, None) == 1
    assert lib.kda_copy_probe(FAKE + 4, FAKE, 4, None) == 4


def test_prepared_needs_exactly_one_launch():
    """api.prepared() records the C call of a launching entry point instead
    of issuing it; a function that issues none is refused, and it does not
    nest."""
    from linear_attention_recurrent_kda_amd import api
    with pytest.raises(ValueError):
        api.prepared(lambda: None)
    with pytest.raises(RuntimeError):
        api.prepared(lambda: api.prepared(lambda: None))
    assert getattr(api._tls, "recording", None) is None


def test_prepared_records_only_on_its_own_thread():
    """While one thread prepares a call, a call issued on another thread is
    not captured by it (the recording is per thread)."""
    import threading
    from linear_attention_recurrent_kda_amd import api
    seen = {}

    def other():
        seen["other"] = getattr(api._tls, "recording", None)

    def entry():
        t = threading.Thread(target=other)
        t.start()
        t.join()
        seen["own"] = list(getattr(api._tls, "recording", None))
        api._call("kda_abi_version")   # recorded, not issued

    call = api.prepared(entry)
    assert seen["other"] is None and seen["own"] == []
    assert callable(call)


def test_build_metadata_validation(lib):
    P = ctypes.c_void_p
    args = lambda n=4, ns=8, nt=FAKE, rs=FAKE, cu=FAKE, si=FAKE, cs=FAKE, ct=FAKE, ef=None: \
        (P(nt) if nt else None, P(rs) if rs else None, n, ns, P(cu) if cu else None, P(si) if si else None,
         P(cs) if cs else None, P(ct) if ct else None, P(ef) if ef else None, None)
    assert lib.kda_build_metadata(*args(n=-1)) == 2
    assert lib.kda_build_metadata(*args(ns=0)) == 2
    assert lib.kda_build_metadata(*args(cu=0)) == 1
    assert lib.kda_build_metadata(*args(ct=0)) == 1
    assert lib.kda_build_metadata(*args(nt=0)) == 1
    assert lib.kda_build_metadata(*args(si=0)) == 1
    assert lib.kda_build_metadata(*args(cs=FAKE + 2)) == 4
    assert lib.kda_build_metadata(*args(ef=FAKE + 1)) == 4


def test_prefill_static_validation(lib):
    """kda_chunk_prefill_static rejects a call whose workspace exceeds the
    static array before any HIP call, and checks its other arguments like
    kda_chunk_prefill."""
    L, C, I = good_layer(H=32), good_cache(), good_inputs()
    call = lambda total_T, N=1, slots=FAKE, cu=FAKE, y=FAKE: lib.kda_chunk_prefill_static(
        ctypes.byref(L), ctypes.byref(C), slots, cu, N, total_T, 64, ctypes.byref(I), y, None)
    assert lib.kda_chunk_prefill_workspace_bytes(ctypes.byref(L), 4096, 1, 64) > _lib.KDA_STATIC_WORKSPACE_BYTES
    assert call(4096) == 6
    assert call(100, slots=None) == 1
    assert call(100, y=FAKE + 4) == 4
    assert call(100, N=0) == 2
