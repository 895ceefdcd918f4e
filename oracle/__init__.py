"""fp64 CPU oracle for MQA/GQA decoding -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``query_decode_attention_amd``) never imports, links or calls it, and the
two share no code: the arithmetic lives in ``mqa_oracle.c`` (plain C, fp64,
built with gcc); this file only builds it and marshals arrays.

What each function follows (all from the pages' statement of the method):
  * ``kv_append``  -- the incremental concat of one new K/V row onto the cache
                      (paper review, section 3 multi-query incremental code).
  * ``decode``     -- o_i = softmax(q_i K^T * scale) V with K/V shared by the
                      h/G heads of a group (study notes section 4 formula;
                      GQA essay section 3 grouping).
  * ``prefill``    -- softmax(Q K^T * scale + M) V with M = -inf above the
                      diagonal (study notes section 1 formula and section 1.1
                      causal rule; paper review section 2.3 additive mask).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mqa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (IEEE fp64, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.oracle_kv_append.argtypes = [I, I, I, I, I, P, P, P, P, P, P]
        lib.oracle_kv_reorder.argtypes = [I, I, I, I, I, I, P, P, P, P, P]
        lib.oracle_decode.argtypes = [I, I, I, I, I, I, P, P, P, P, D, I, P, I]
        lib.oracle_decode_weights.argtypes = [I, I, I, I, I, I, P, P, P, P, D, I, I, I, P]
        lib.oracle_prefill.argtypes = [I, I, I, I, I, I, P, P, P, D, P, ctypes.c_int64, P, I]
        L64 = ctypes.c_int64
        lib.oracle_attend.argtypes = [I, I, I, I, I, I, I, P, P, P, D, P, L64, L64, L64, P, L64,
                                      P, I]
        for f in (lib.oracle_kv_append, lib.oracle_decode, lib.oracle_decode_weights,
                  lib.oracle_prefill):
            f.restype = I
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _raw(x):
    """Return (contiguous numpy array of raw element storage, dtype code).

    Accepts numpy float32 / uint16 (bf16 bit patterns) arrays or torch CPU
    tensors of dtype float32 / bfloat16.
    """
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            raise TypeError("oracle takes float32 or bfloat16 tensors, got %s" % x.dtype)
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("oracle takes float32 or uint16(bf16 bits) arrays, got %s" % x.dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def kv_append(k_new, v_new, K, V, lens):
    """In-place append on numpy arrays (raw storage).  Returns overflow count.

    k_new, v_new: [b, G, dh]; K, V: [b, m_cap, G, dh]; lens: int32 [b].
    """
    kn, dt = _raw(k_new)
    vn, dt2 = _raw(v_new)
    assert dt == dt2
    assert isinstance(K, np.ndarray) and K.flags.c_contiguous and isinstance(V, np.ndarray)
    assert lens.dtype == np.int32 and lens.flags.c_contiguous
    b, m_cap, G, dh = K.shape
    assert kn.shape == (b, G, dh) and vn.shape == (b, G, dh) and V.shape == K.shape
    over = ctypes.c_int32(0)
    rc = _load().oracle_kv_append(dt, b, G, dh, m_cap, _ptr(kn), _ptr(vn), _ptr(K), _ptr(V),
                                  _ptr(lens), ctypes.byref(over))
    if rc != 0:
        raise ValueError("oracle_kv_append rejected its arguments")
    return over.value


def kv_reorder(K, V, lens, parent, beam):
    """In-place beam reorder on numpy arrays (raw storage).  Returns the number
    of invalid parents.

    K, V: [b, m_cap, G, dh] (float32 or uint16 bf16 bits); lens, parent:
    int32 [b]; hypothesis i takes the cache of (i // beam) * beam + parent[i].
    """
    assert isinstance(K, np.ndarray) and K.flags.c_contiguous and isinstance(V, np.ndarray)
    assert V.flags.c_contiguous and V.shape == K.shape and V.dtype == K.dtype
    dt = F32 if K.dtype == np.float32 else BF16
    assert K.dtype in (np.float32, np.uint16)
    assert lens.dtype == np.int32 and lens.flags.c_contiguous
    par = np.ascontiguousarray(parent, dtype=np.int32)
    b, m_cap, G, dh = K.shape
    assert lens.shape == (b,) and par.shape == (b,)
    bad = ctypes.c_int32(0)
    rc = _load().oracle_kv_reorder(dt, b, G, dh, m_cap, int(beam), _ptr(par), _ptr(K), _ptr(V),
                                   _ptr(lens), ctypes.byref(bad))
    if rc != 0:
        raise ValueError("oracle_kv_reorder rejected its arguments")
    return bad.value


def decode(q, K, V, lens, scale, window=0, nthreads=None) -> np.ndarray:
    """fp64 [b, h, dh] decode output.  q [b,h,dh]; K,V [b,m_cap,G,dh]; lens int32 [b]."""
    qa, dt = _raw(q)
    Ka, dk = _raw(K)
    Va, dv = _raw(V)
    assert dt == dk == dv, "q, K and V must share one dtype"
    ln = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    b, h, dh = qa.shape
    b2, m_cap, G, dh2 = Ka.shape
    assert b2 == b and dh2 == dh and Va.shape == Ka.shape and ln.shape == (b,)
    o = np.zeros((b, h, dh), dtype=np.float64)
    rc = _load().oracle_decode(dt, b, h, G, dh, m_cap, _ptr(qa), _ptr(Ka), _ptr(Va), _ptr(ln),
                               float(scale), int(window), _ptr(o),
                               int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return o


def decode_weights(q, K, V, lens, scale, bi, i, window=0) -> np.ndarray:
    """Softmax weights of decode row (bi, i) over its visible positions."""
    qa, dt = _raw(q)
    Ka, _ = _raw(K)
    Va, _ = _raw(V)
    ln = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    b, h, dh = qa.shape
    _, m_cap, G, _ = Ka.shape
    w = np.zeros(max(m_cap, 1), dtype=np.float64)
    n = _load().oracle_decode_weights(dt, b, h, G, dh, m_cap, _ptr(qa), _ptr(Ka), _ptr(Va),
                                      _ptr(ln), float(scale), int(window), int(bi), int(i),
                                      _ptr(w))
    if n < 0:
        raise ValueError("oracle_decode_weights rejected its arguments")
    return w[:n].copy()


def prefill(Q, K, V, scale, rows=None, nthreads=None) -> np.ndarray:
    """fp64 causal prefill.  Q [b,n,h,dh]; K,V [b,n,G,dh].

    rows: optional sequence of flattened (b, t) indices; returns [nrows, h, dh]
    (or [b, n, h, dh] when rows is None).
    """
    Qa, dt = _raw(Q)
    Ka, dk = _raw(K)
    Va, dv = _raw(V)
    assert dt == dk == dv
    b, n, h, dh = Qa.shape
    assert Ka.shape[:2] == (b, n) and Ka.shape[3] == dh and Va.shape == Ka.shape
    G = Ka.shape[2]
    if rows is None:
        out = np.zeros((b * n, h, dh), dtype=np.float64)
        rp, nr = None, b * n
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.zeros((r.size, h, dh), dtype=np.float64)
        rp, nr = _ptr(r), r.size
    rc = _load().oracle_prefill(dt, b, n, h, G, dh, _ptr(Qa), _ptr(Ka), _ptr(Va), float(scale),
                                rp, nr, _ptr(out), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return out.reshape(b, n, h, dh) if rows is None else out


def attend(Q, K, V, scale, mask=None, strides=None, rows=None, nthreads=None) -> np.ndarray:
    """fp64 attention over a fixed memory.  Q [b,n,h,dh]; K,V [b,m,G,dh].

    mask: optional float32 array (any shape) read at
    b*sb + i*sh + t*sn + j with strides=(sb, sh, sn) in elements; with
    strides None the mask must be a dense [b, h, n, m] array.
    rows: as in prefill; returns [nrows, h, dh] or [b, n, h, dh].
    """
    Qa, dt = _raw(Q)
    Ka, dk = _raw(K)
    Va, dv = _raw(V)
    assert dt == dk == dv
    b, n, h, dh = Qa.shape
    m, G = Ka.shape[1], Ka.shape[2]
    assert Ka.shape == (b, m, G, dh) and Va.shape == Ka.shape
    mp, sb, sh, sn = None, 0, 0, 0
    if mask is not None:
        mk = mask.numpy() if hasattr(mask, "numpy") else mask
        mk = np.ascontiguousarray(mk, dtype=np.float32)
        if strides is None:
            assert mk.shape == (b, h, n, m)
            strides = (h * n * m, n * m, m)
        sb, sh, sn = (int(x) for x in strides)
        mp = _ptr(mk)
    if rows is None:
        out = np.zeros((b * n, h, dh), dtype=np.float64)
        rp, nr = None, b * n
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.zeros((r.size, h, dh), dtype=np.float64)
        rp, nr = _ptr(r), r.size
    rc = _load().oracle_attend(dt, b, n, m, h, G, dh, _ptr(Qa), _ptr(Ka), _ptr(Va), float(scale),
                               mp, sb, sh, sn, rp, nr, _ptr(out),
                               int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_attend rejected its arguments")
    return out.reshape(b, n, h, dh) if rows is None else out
