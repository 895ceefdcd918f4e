"""CPU checks of the C ABI: the library loads, exports every symbol that
include/mqa.h declares, and rejects bad arguments on the host before any HIP
call (no kernel is launched here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mqa.h")

OK, ENULL, ESHAPE, EDHEAD, EALIGN, EWS, ELAUNCH, EDTYPE, ELENS = 0, -1, -2, -3, -4, -5, -6, -7, -8


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mqa_[a-z_]+)\s*\(", text)))


class Cache(ctypes.Structure):
    """mqa_cache as include/mqa.h lays it out (independent of the binding)."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("b", ctypes.c_int32),
                ("m_cap", ctypes.c_int32), ("G", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


@pytest.fixture(scope="module")
def lib(libmqa_path):
    """A ctypes handle of our own, typed from the header, not from the binding."""
    L = ctypes.CDLL(libmqa_path)
    P, I32, F, SZ, CP = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t,
                         ctypes.POINTER(Cache))
    L.mqa_kv_append.argtypes = [P, P, CP, P, P, P]
    L.mqa_decode_workspace_size.argtypes = [I32, CP]
    L.mqa_decode_workspace_size.restype = SZ
    L.mqa_decode.argtypes = [P, I32, CP, P, F, I32, P, P, SZ, P]
    L.mqa_append_decode.argtypes = [P, P, P, I32, CP, P, P, F, I32, P, P, SZ, P]
    L.mqa_decode_ex.argtypes = [P, P, P, I32, CP, P, P, F, I32, P, P, SZ, P, P, P]
    L.mqa_decode_noalloc.argtypes = [P, P, P, I32, CP, P, P, F, I32, P, P]
    L.mqa_prefill_causal.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, F, CP, P, P, P]
    L.mqa_check_lens.argtypes = [P, I32, I32, P]
    L.mqa_kv_reorder.argtypes = [CP, P, P, I32, P, P]
    L.mqa_kv_reorder_to.argtypes = [CP, P, P, P, I32, P, P]
    L.mqa_read_probe.argtypes = [P, SZ, P, P]
    L64 = ctypes.c_int64
    L.mqa_attend.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, I32, F, P, L64, L64, L64,
                             P, P]
    return L


FAKE = ctypes.c_void_p(0x7F0000001000)       # aligned, never dereferenced
FAKE_MIS = ctypes.c_void_p(0x7F0000001008)   # 8-byte aligned only


def cache(b=2, m_cap=64, G=1, dh=128, dtype=1, k=FAKE, v=FAKE):
    return Cache(k.value if k else None, v.value if v else None, b, m_cap, G, dh, dtype)


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted([
        "mqa_abi_version", "mqa_append_decode", "mqa_check_lens", "mqa_decode",
        "mqa_decode_ex", "mqa_decode_noalloc", "mqa_decode_workspace_size",
        "mqa_attend", "mqa_kv_append", "mqa_kv_reorder", "mqa_kv_reorder_to", "mqa_prefill_causal",
        "mqa_read_probe",
        "mqa_strerror"])


def test_library_exports_every_declared_symbol(lib, libmqa_path):
    out = subprocess.run(["nm", "-D", "--defined-only", libmqa_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mqa_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    import query_decode_attention_amd as q
    assert set(q.EXPORTED) == set(declared_functions())


def test_strerror_and_version(lib):
    import query_decode_attention_amd as q
    assert q.abi_version() == 205
    for code in (OK, ENULL, ESHAPE, EDHEAD, EALIGN, EWS, ELAUNCH, EDTYPE, ELENS):
        assert q.strerror(code) and q.strerror(code) != "unknown status"
    assert q.strerror(12345) == "unknown status"


def test_workspace_size_is_pure_host_arithmetic(lib):
    f = lib.mqa_decode_workspace_size
    c = cache(b=64, m_cap=8448, G=1, dh=128)
    n = f(32, ctypes.byref(c))
    # schedule header (b + 4 = 68 ints -> 512 B) + 2 * 2048 records of 32*130 floats
    assert n == 512 + 2 * 2048 * (32 * 130 * 4)
    small = cache(b=1, m_cap=128, G=1, dh=64)
    assert f(4, ctypes.byref(small)) == 256 + 2 * 4 * ((4 * 66 + 3) // 4 * 4 * 4)
    gqa = cache(b=32, m_cap=32768, G=8, dh=128)
    assert f(64, ctypes.byref(gqa)) == 256 + 2 * 2048 * (8 * 130 * 4)
    assert f(3, ctypes.byref(cache(G=2))) == 0          # G does not divide h
    assert f(64, ctypes.byref(cache(G=1))) == 0         # h/G > 32
    assert f(4, ctypes.byref(cache(dh=96))) == 0        # d_h
    assert f(4, None) == 0


def test_decode_rejects_bad_arguments_before_launching(lib):
    d = lib.mqa_decode
    ws = 1 << 30

    def call(h=4, c=None, q=FAKE, lens=FAKE, o=FAKE, w=FAKE, wsb=ws, window=0):
        c = c if c is not None else cache()
        return d(q, h, ctypes.byref(c), lens, 1.0, window, o, w, wsb, None)

    assert d(FAKE, 4, None, FAKE, 1.0, 0, FAKE, FAKE, ws, None) == ENULL
    assert call(q=None) == ENULL
    assert call(lens=None) == ENULL
    assert call(c=cache(k=None)) == ENULL
    assert call(h=3, c=cache(G=2)) == ESHAPE
    assert call(h=33) == ESHAPE
    assert call(window=-1) == ESHAPE
    assert call(c=cache(m_cap=0)) == ESHAPE
    assert call(c=cache(dh=96)) == EDHEAD
    assert call(c=cache(dtype=5)) == EDTYPE
    assert call(q=FAKE_MIS) == EALIGN
    assert call(c=cache(k=FAKE_MIS)) == EALIGN
    assert call(w=None) == EWS
    assert call(wsb=100) == EWS
    assert call(w=FAKE_MIS) == EWS
    assert call(c=cache(b=0)) == OK                     # nothing to do, nothing launched


def test_fused_append_decode_rejects_bad_arguments(lib):
    ad = lib.mqa_append_decode
    c = cache()
    ws = 1 << 30

    def call(kn=FAKE, vn=FAKE, q=FAKE, lens=FAKE, w=FAKE, wsb=ws, c=c):
        return ad(q, kn, vn, 4, ctypes.byref(c), lens, None, 1.0, 0, FAKE, w, wsb, None)

    assert call(kn=None) == ENULL
    assert call(vn=None) == ENULL
    assert call(lens=None) == ENULL
    assert call(kn=FAKE_MIS) == EALIGN
    assert call(wsb=64) == EWS
    assert call(c=cache(dh=48)) == EDHEAD
    ex = lib.mqa_decode_ex
    # exactly one of k_new / v_new given
    assert ex(FAKE, FAKE, None, 4, ctypes.byref(c), FAKE, None, 1.0, 0, FAKE, FAKE, ws, None,
              None, None) == ENULL


def test_noalloc_decode_rejects_bad_arguments_before_any_hip_call(lib):
    f = lib.mqa_decode_noalloc

    def call(h=4, c=None, q=FAKE, kn=None, vn=None, lens=FAKE, o=FAKE, window=0):
        c = c if c is not None else cache()
        return f(q, kn, vn, h, ctypes.byref(c), lens, None, 1.0, window, o, None)

    assert f(FAKE, None, None, 4, None, FAKE, None, 1.0, 0, FAKE, None) == ENULL
    assert call(q=None) == ENULL
    assert call(o=None) == ENULL
    assert call(lens=None) == ENULL
    assert call(kn=FAKE) == ENULL                       # k_new without v_new
    assert call(h=3, c=cache(G=2)) == ESHAPE
    assert call(h=33) == ESHAPE
    assert call(window=-1) == ESHAPE
    assert call(c=cache(dh=96)) == EDHEAD
    assert call(c=cache(dtype=5)) == EDTYPE
    assert call(o=FAKE_MIS) == EALIGN
    assert call(kn=FAKE, vn=FAKE_MIS) == EALIGN
    assert call(c=cache(b=0)) == OK                     # nothing to do, nothing launched


def test_append_and_prefill_reject_bad_arguments(lib):
    a = lib.mqa_kv_append
    c = cache()
    assert a(None, FAKE, ctypes.byref(c), FAKE, None, None) == ENULL
    assert a(FAKE, FAKE, ctypes.byref(c), None, None, None) == ENULL
    assert a(FAKE_MIS, FAKE, ctypes.byref(c), FAKE, None, None) == EALIGN
    assert a(FAKE, FAKE, ctypes.byref(cache(dh=32)), FAKE, None, None) == EDHEAD
    z = cache(b=0)
    assert a(None, None, ctypes.byref(z), None, None, None) == OK

    p = lib.mqa_prefill_causal

    def pf(b=2, n=16, h=4, G=1, dh=128, dt=1, c=None, Q=FAKE, O=FAKE):
        return p(Q, FAKE, FAKE, b, n, h, G, dh, dt, 1.0, ctypes.byref(c) if c else None, None,
                 O, None)

    assert pf(dt=3) == EDTYPE
    assert pf(dh=80) == EDHEAD
    assert pf(n=0) == ESHAPE
    assert pf(h=6, G=4) == ESHAPE
    assert pf(Q=None) == ENULL
    assert pf(O=FAKE_MIS) == EALIGN
    assert pf(c=cache(b=2, m_cap=8)) == ESHAPE          # n > m_cap
    assert pf(c=cache(b=3, m_cap=64)) == ESHAPE         # batch mismatch
    assert pf(b=0) == OK


def test_check_lens_argument_errors(lib):
    assert lib.mqa_check_lens(None, 3, 10, None) == ENULL
    assert lib.mqa_check_lens(FAKE, -1, 10, None) == ESHAPE
    assert lib.mqa_check_lens(None, 0, 10, None) == OK


def test_read_probe_rejects_bad_arguments_before_launching(lib):
    f = lib.mqa_read_probe
    assert f(None, 1024, FAKE, None) == ENULL
    assert f(FAKE, 1024, None, None) == ENULL
    assert f(FAKE_MIS, 1024, FAKE, None) == EALIGN
    assert f(FAKE, 1000, FAKE, None) == EALIGN              # not a multiple of 16 bytes
    assert f(FAKE, 0, FAKE, None) == OK                     # nothing to read: nothing launched


def test_reorder_to_rejects_bad_arguments_before_launching(lib):
    r = lib.mqa_kv_reorder_to
    OTHER = ctypes.c_void_p(0x7F0000002000)

    def call(c=None, lens=FAKE, out=OTHER, parent=FAKE, beam=4):
        c = c if c is not None else cache(b=8)
        return r(ctypes.byref(c), lens, out, parent, beam, None, None)

    assert r(None, FAKE, OTHER, FAKE, 4, None, None) == ENULL
    assert call(lens=None) == ENULL
    assert call(out=None) == ENULL
    assert call(parent=None) == ENULL
    assert call(out=FAKE) == ESHAPE                     # lens_out == lens_in
    assert call(beam=3) == ESHAPE
    assert call(c=cache(b=8, dh=96)) == EDHEAD
    assert call(c=cache(b=0)) == OK                     # nothing to reorder


def test_reorder_rejects_bad_arguments_before_launching(lib):
    r = lib.mqa_kv_reorder

    def call(c=None, lens=FAKE, parent=FAKE, beam=4):
        c = c if c is not None else cache(b=8)
        return r(ctypes.byref(c), lens, parent, beam, None, None)

    assert r(None, FAKE, FAKE, 4, None, None) == ENULL
    assert call(lens=None) == ENULL
    assert call(parent=None) == ENULL
    assert call(c=cache(b=8, k=None)) == ENULL
    assert call(beam=0) == ESHAPE
    assert call(beam=3) == ESHAPE                       # does not divide b = 8
    assert call(c=cache(b=32), beam=32) == ESHAPE       # beam > 16
    assert call(c=cache(b=8, dh=96)) == EDHEAD
    assert call(c=cache(b=8, k=FAKE_MIS)) == EALIGN
    assert call(c=cache(b=0)) == OK                     # nothing to do, nothing launched


def test_attend_rejects_bad_arguments_before_launching(lib):
    a = lib.mqa_attend

    def call(Q=FAKE, K=FAKE, V=FAKE, b=2, n=3, m=5, h=4, G=1, dh=128, dtype=1, mask=None,
             sb=0, sh=0, sn=0, O=FAKE):
        return a(Q, K, V, b, n, m, h, G, dh, dtype, 1.0, mask, sb, sh, sn, O, None)

    assert call(Q=None) == ENULL
    assert call(O=None) == ENULL
    assert call(n=0) == ESHAPE
    assert call(m=0) == ESHAPE
    assert call(h=3, G=2) == ESHAPE
    assert call(h=64) == ESHAPE                         # h/G > 32
    assert call(dh=96) == EDHEAD
    assert call(dtype=3) == EDTYPE
    assert call(mask=FAKE, sb=-1) == ESHAPE
    assert call(K=FAKE_MIS) == EALIGN
    assert call(mask=ctypes.c_void_p(0x7F0000001002)) == EALIGN
    assert call(b=0) == OK                              # nothing to do, nothing launched
