"""query_decode_attention_amd -- MQA/GQA incremental decoding on MI355X (gfx950).

Thin ctypes binding over ``libmqa.so`` (C ABI in ``include/mqa.h``).  This
module only marshals arguments: it checks tensor placement, dtype, shape and
contiguity, then passes raw device pointers and the current HIP stream of
PyTorch.  Every step of the computation runs in the library's HIP kernels;
there is no fallback: the first call (or ``load()``) raises ImportError if
the library is missing.  PyTorch supplies device memory and streams only.

Entry points (same names as the C ABI, minus the ``mqa_`` prefix):
  kv_append(k_new, v_new, K, V, lens, err_flag=None)
  decode_workspace_size(h, K) / workspace_for(h, K)
  decode(q, K, V, lens, scale, window=0, out=None, workspace=None)
  append_decode(q, k_new, v_new, K, V, lens, scale, ...)   (append fused in)
  decode_noalloc(q, K, V, lens, scale, ..., k_new=None, v_new=None)
                                            (no workspace; library scratch)
  prefill_causal(Q, K, V, scale, cache_K=None, cache_V=None, lens=None, out=None)
  check_lens(lens, m_cap)
  strerror(status)
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import workloads  # noqa: F401  (seeded inputs; no arithmetic)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmqa.so")

MQA_F32, MQA_BF16 = 0, 1
_DTYPES = {torch.float32: MQA_F32, torch.bfloat16: MQA_BF16}

# Symbols include/mqa.h declares (tests check the library exports each one).
EXPORTED = ("mqa_kv_append", "mqa_kv_reorder", "mqa_kv_reorder_to", "mqa_decode_workspace_size",
            "mqa_decode", "mqa_append_decode", "mqa_decode_ex", "mqa_decode_noalloc",
            "mqa_prefill_causal", "mqa_attend",
            "mqa_check_lens", "mqa_read_probe", "mqa_strerror", "mqa_abi_version")


class MQAError(RuntimeError):
    """A libmqa call returned a non-zero mqa_status."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({strerror(status)})")


class _Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("b", ctypes.c_int32),
                ("m_cap", ctypes.c_int32), ("G", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m query_decode_attention_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    CP = ctypes.POINTER(_Cache)
    sig = {
        "mqa_kv_append": ([P, P, CP, P, P, P], ctypes.c_int),
        "mqa_kv_reorder": ([CP, P, P, I32, P, P], ctypes.c_int),
        "mqa_kv_reorder_to": ([CP, P, P, P, I32, P, P], ctypes.c_int),
        "mqa_decode_workspace_size": ([I32, CP], SZ),
        "mqa_decode": ([P, I32, CP, P, F, I32, P, P, SZ, P], ctypes.c_int),
        "mqa_append_decode": ([P, P, P, I32, CP, P, P, F, I32, P, P, SZ, P], ctypes.c_int),
        "mqa_decode_ex": ([P, P, P, I32, CP, P, P, F, I32, P, P, SZ, P, P, P], ctypes.c_int),
        "mqa_decode_noalloc": ([P, P, P, I32, CP, P, P, F, I32, P, P], ctypes.c_int),
        "mqa_prefill_causal": ([P, P, P, I32, I32, I32, I32, I32, I32, F, CP, P, P, P],
                               ctypes.c_int),
        "mqa_attend": ([P, P, P, I32, I32, I32, I32, I32, I32, I32, F, P, ctypes.c_int64,
                        ctypes.c_int64, ctypes.c_int64, P, P], ctypes.c_int),
        "mqa_check_lens": ([P, I32, I32, P], ctypes.c_int),
        "mqa_read_probe": ([P, SZ, P, P], ctypes.c_int),
        "mqa_strerror": ([ctypes.c_int], ctypes.c_char_p),
        "mqa_abi_version": ([], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


_lib_handle = None


def load():
    """Load libmqa.so (once); raises ImportError when it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        _lib_handle = _load()
    return _lib_handle


class _LazyLib:
    def __getattr__(self, name):
        return getattr(load(), name)


_lib = _LazyLib()


def lib():
    return load()


def strerror(status: int) -> str:
    return _lib.mqa_strerror(int(status)).decode()


def abi_version() -> int:
    return _lib.mqa_abi_version()


def _check(fn, status):
    if status != 0:
        raise MQAError(fn, status)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError("libmqa takes CUDA (HIP) tensors only")
        if not t.is_contiguous():
            raise ValueError("libmqa takes contiguous tensors only")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must live on one device")
    return dev


def _cache(K, V):
    if K.dim() != 4 or V.shape != K.shape or V.dtype != K.dtype:
        raise ValueError("K and V caches must both be [b, m_cap, G, d_h] of one dtype")
    if K.dtype not in _DTYPES:
        raise ValueError(f"unsupported cache dtype {K.dtype}")
    b, m_cap, G, dh = K.shape
    return _Cache(K.data_ptr(), V.data_ptr(), b, m_cap, G, dh, _DTYPES[K.dtype])


def _shape_only(K):
    b, m_cap, G, dh = K.shape
    return _Cache(None, None, b, m_cap, G, dh, _DTYPES.get(K.dtype, -1))


def _event_handle(e):
    """hipEvent_t of a torch.cuda.Event (already created) or a raw handle."""
    h = e.cuda_event if isinstance(e, torch.cuda.Event) else e
    h = h.value if isinstance(h, ctypes.c_void_p) else h
    if not h:
        raise ValueError("timing events must be created (recorded once) before use")
    return ctypes.c_void_p(h)


def _check_new_rows(k_new, v_new, K, lens):
    b, _, G, dh = K.shape
    if k_new.shape != (b, G, dh) or v_new.shape != (b, G, dh):
        raise ValueError("k_new / v_new must be [b, G, d_h]")
    if k_new.dtype != K.dtype or v_new.dtype != K.dtype:
        raise ValueError("k_new / v_new must have the cache dtype")
    if lens.dtype != torch.int32 or lens.shape != (b,):
        raise ValueError("lens must be int32 [b]")


def kv_append(k_new, v_new, K, V, lens, err_flag=None):
    """K[b, lens[b]] = k_new[b]; V likewise; lens[b] += 1 (in place, async)."""
    dev = _dev(k_new, v_new, K, V, lens, err_flag)
    _check_new_rows(k_new, v_new, K, lens)
    if err_flag is not None and (err_flag.dtype != torch.int32 or err_flag.numel() < 1):
        raise ValueError("err_flag must be an int32 tensor")
    c = _cache(K, V)
    _check("mqa_kv_append", _lib.mqa_kv_append(_ptr(k_new), _ptr(v_new), ctypes.byref(c),
                                                 _ptr(lens), _ptr(err_flag), _stream(dev)))


def kv_reorder(K, V, lens, parent, beam: int, err_flag=None, lens_out=None):
    """Beam reorder (async): hypothesis i takes the cached rows and the length
    of hypothesis (i // beam) * beam + parent[i].  K and V are reordered in
    place; the lengths too, or, with ``lens_out``, into that tensor (lens
    only read; one launch instead of two).

    K, V: [b, m_cap, G, d_h]; lens, parent, lens_out: int32 [b] on the same device."""
    dev = _dev(K, V, lens, parent, err_flag, lens_out)
    b = K.shape[0]
    named = [("lens", lens), ("parent", parent)] + ([("lens_out", lens_out)] if lens_out is not None
                                                     else [])
    for name, t in named:
        if t.dtype != torch.int32 or t.shape != (b,) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor of shape [{b}]")
    if err_flag is not None and (err_flag.dtype != torch.int32 or err_flag.numel() < 1):
        raise ValueError("err_flag must be an int32 tensor")
    c = _cache(K, V)
    if lens_out is None:
        _check("mqa_kv_reorder", _lib.mqa_kv_reorder(ctypes.byref(c), _ptr(lens), _ptr(parent),
                                                       int(beam), _ptr(err_flag), _stream(dev)))
    else:
        _check("mqa_kv_reorder_to", _lib.mqa_kv_reorder_to(
            ctypes.byref(c), _ptr(lens), _ptr(lens_out), _ptr(parent), int(beam), _ptr(err_flag),
            _stream(dev)))


def decode_workspace_size(h: int, K) -> int:
    n = _lib.mqa_decode_workspace_size(int(h), ctypes.byref(_shape_only(K)))
    if n == 0:
        raise ValueError("invalid decode shapes")
    return int(n)


def workspace_for(h: int, K):
    """Allocate a decode workspace (uint8 device tensor; needs no initialisation).

    Invalid shapes give a 1-byte tensor, so that the decode call itself
    reports the exact status."""
    n = _lib.mqa_decode_workspace_size(int(h), ctypes.byref(_shape_only(K)))
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=K.device)


def _decode_call(q, k_new, v_new, K, V, lens, scale, window, out, workspace, err_flag, events):
    if workspace is None:
        workspace = workspace_for(q.shape[1], K)
    if out is None:
        out = torch.empty_like(q)
    dev = _dev(q, k_new, v_new, K, V, lens, out, workspace, err_flag)
    b, m_cap, G, dh = K.shape
    if q.dim() != 3 or q.shape[0] != b or q.shape[2] != dh:
        raise ValueError("q must be [b, h, d_h] matching the cache")
    if q.dtype != K.dtype or out.dtype != K.dtype or out.shape != q.shape:
        raise ValueError("q / out must match the cache dtype and q's shape")
    if lens.dtype != torch.int32 or lens.shape != (b,):
        raise ValueError("lens must be int32 [b]")
    if k_new is not None:
        _check_new_rows(k_new, v_new, K, lens)
    c = _cache(K, V)
    ev0 = ev1 = None
    if events is not None:
        ev0, ev1 = (_event_handle(e) for e in events)
    _check("mqa_decode_ex", _lib.mqa_decode_ex(
        _ptr(q), _ptr(k_new), _ptr(v_new), q.shape[1], ctypes.byref(c), _ptr(lens),
        _ptr(err_flag), float(scale), int(window), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev), ev0, ev1))
    return out


def decode(q, K, V, lens, scale, window=0, out=None, workspace=None, events=None):
    """One decode step: o[b,i] = softmax(scale * q[b,i] . K[b,:L,g(i)]) V[b,:L,g(i)].

    events: optional (begin, end) torch.cuda.Event pair, already created on
    q's device, recorded around the decode kernel.
    """
    return _decode_call(q, None, None, K, V, lens, scale, window, out, workspace, None, events)


def append_decode(q, k_new, v_new, K, V, lens, scale, window=0, out=None, workspace=None,
                  err_flag=None, events=None):
    """kv_append followed by decode, with the append done by the decode kernels."""
    if k_new is None or v_new is None:
        raise ValueError("append_decode needs k_new and v_new")
    return _decode_call(q, k_new, v_new, K, V, lens, scale, window, out, workspace, err_flag,
                        events)


def decode_noalloc(q, K, V, lens, scale, window=0, out=None, k_new=None, v_new=None,
                   err_flag=None):
    """decode (k_new / v_new None) or append_decode through mqa_decode_noalloc:
    no workspace argument and no allocation by the library; the split-K
    records use the library's fixed per-device scratch array, so calls on one
    device must be ordered (one stream).  ``out`` is allocated here when None;
    pass it to allocate nothing at all."""
    if out is None:
        out = torch.empty_like(q)
    dev = _dev(q, k_new, v_new, K, V, lens, out, err_flag)
    b, m_cap, G, dh = K.shape
    if q.dim() != 3 or q.shape[0] != b or q.shape[2] != dh:
        raise ValueError("q must be [b, h, d_h] matching the cache")
    if q.dtype != K.dtype or out.dtype != K.dtype or out.shape != q.shape:
        raise ValueError("q / out must match the cache dtype and q's shape")
    if lens.dtype != torch.int32 or lens.shape != (b,):
        raise ValueError("lens must be int32 [b]")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _check_new_rows(k_new, v_new, K, lens)
    c = _cache(K, V)
    _check("mqa_decode_noalloc", _lib.mqa_decode_noalloc(
        _ptr(q), _ptr(k_new), _ptr(v_new), q.shape[1], ctypes.byref(c), _ptr(lens),
        _ptr(err_flag), float(scale), int(window), _ptr(out), _stream(dev)))
    return out


def prefill_causal(Q, K, V, scale, cache_K=None, cache_V=None, lens=None, out=None):
    """Causal attention over a prompt; optionally fills the cache and lens."""
    if out is None:
        out = torch.empty_like(Q)
    dev = _dev(Q, K, V, out, cache_K, cache_V, lens)
    b, n, h, dh = Q.shape
    if K.dim() != 4 or K.shape[:2] != (b, n) or K.shape[3] != dh or V.shape != K.shape:
        raise ValueError("K / V must be [b, n, G, d_h] matching Q")
    if K.dtype != Q.dtype or V.dtype != Q.dtype or out.dtype != Q.dtype or out.shape != Q.shape:
        raise ValueError("Q, K, V and out must share one dtype and Q's shape")
    if Q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {Q.dtype}")
    G = K.shape[2]
    cp = None
    if cache_K is not None:
        c = _cache(cache_K, cache_V)
        cp = ctypes.byref(c)
    if lens is not None and (lens.dtype != torch.int32 or lens.shape != (b,)):
        raise ValueError("lens must be int32 [b]")
    _check("mqa_prefill_causal", _lib.mqa_prefill_causal(
        _ptr(Q), _ptr(K), _ptr(V), b, n, h, G, dh, _DTYPES[Q.dtype], float(scale), cp,
        _ptr(lens), _ptr(out), _stream(dev)))
    return out


def attend(Q, K, V, scale, mask=None, out=None):
    """Attention of Q [b,n,h,d_h] over a fixed memory K, V [b,m,G,d_h] with no
    causal structure: O = softmax(scale * Q K^T + mask) V per head, head i
    reading K/V group i // (h/G).

    mask: optional float32 tensor on the same device, any shape that
    broadcasts to [b, h, n, m] with the key dimension contiguous (a [b,1,1,m]
    key-padding mask or a full [b,h,n,m] one); -inf hides a key, and a row
    whose every key is hidden gives zeros."""
    if out is None:
        out = torch.empty_like(Q)
    dev = _dev(Q, K, V, out, mask)
    b, n, h, dh = Q.shape
    if K.dim() != 4 or K.shape[0] != b or K.shape[3] != dh or V.shape != K.shape:
        raise ValueError("K / V must be [b, m, G, d_h] matching Q")
    if K.dtype != Q.dtype or V.dtype != Q.dtype or out.dtype != Q.dtype or out.shape != Q.shape:
        raise ValueError("Q, K, V and out must share one dtype and Q's shape")
    if Q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {Q.dtype}")
    m, G = K.shape[1], K.shape[2]
    sb = sh = sn = 0
    if mask is not None:
        if mask.dtype != torch.float32:
            raise ValueError("mask must be float32")
        mask = mask.expand(b, h, n, m)
        if mask.stride(3) != 1:
            raise ValueError("the mask's key dimension must be contiguous")
        sb, sh, sn = mask.stride(0), mask.stride(1), mask.stride(2)
    _check("mqa_attend", _lib.mqa_attend(
        _ptr(Q), _ptr(K), _ptr(V), b, n, m, h, G, dh, _DTYPES[Q.dtype], float(scale),
        _ptr(mask), sb, sh, sn, _ptr(out), _stream(dev)))
    return out


def check_lens(lens, m_cap):
    """Synchronising host check that every lens[b] lies in [0, m_cap]."""
    dev = _dev(lens)
    _check("mqa_check_lens", _lib.mqa_check_lens(_ptr(lens), lens.numel(), int(m_cap),
                                                 _stream(dev)))


def read_probe(buf, sink):
    """Stream-read the device tensor ``buf`` once (a measurement aid: the
    practical HBM read rate); ``sink`` is a 4-byte device tensor."""
    dev = _dev(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    _check("mqa_read_probe", _lib.mqa_read_probe(_ptr(buf), nbytes - nbytes % 16, _ptr(sink),
                                                 _stream(dev)))


class DecodeStep:
    """One serving step over fixed tensors: append + decode (append fused into
    the decode by default, or kv_append then decode with ``fused=False``), or
    a plain decode when k_new/v_new are None.

    Validates the arguments once and keeps the ctypes argument lists, so a
    call costs one or two C calls; used where per-step Python overhead would
    show (benchmarks, HIP-graph capture).  The stream is read at call time,
    so a step issued inside ``torch.cuda.graph`` is captured on the capture
    stream.
    """

    def __init__(self, q, K, V, lens, scale, out=None, workspace=None, k_new=None, v_new=None,
                 window=0, fused=True):
        if workspace is None:
            workspace = workspace_for(q.shape[1], K)
        if out is None:
            out = torch.empty_like(q)
        self._keep = (q, K, V, lens, out, workspace, k_new, v_new)
        if (k_new is None) != (v_new is None):
            raise ValueError("give both k_new and v_new, or neither")
        self.device = _dev(q, K, V, lens, out, workspace, k_new, v_new)
        b = K.shape[0]
        if k_new is not None:
            _check_new_rows(k_new, v_new, K, lens)
        if q.dim() != 3 or q.shape[0] != b or q.shape[2] != K.shape[3] or q.dtype != K.dtype:
            raise ValueError("q must be [b, h, d_h] in the cache dtype")
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q")
        if lens.dtype != torch.int32 or lens.shape != (b,):
            raise ValueError("lens must be int32 [b]")
        self.out = out
        self._c = _cache(K, V)
        cref = ctypes.byref(self._c)
        wsb = workspace.numel() * workspace.element_size()
        lib_ = load()
        self._fa, self._fx = lib_.mqa_kv_append, lib_.mqa_decode_ex
        self._append = None
        new = (_ptr(k_new), _ptr(v_new)) if (k_new is not None and fused) else (None, None)
        if k_new is not None and not fused:
            self._append = (_ptr(k_new), _ptr(v_new), cref, _ptr(lens), None)
        self._decode = (_ptr(q),) + new + (q.shape[1], cref, _ptr(lens), None, float(scale),
                                           int(window), _ptr(out), _ptr(workspace), wsb)

    def __call__(self, events=None):
        s = ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)
        if self._append is not None:
            rc = self._fa(*self._append, s)
            if rc:
                raise MQAError("mqa_kv_append", rc)
        if events is None:
            rc = self._fx(*self._decode, s, None, None)
        else:
            rc = self._fx(*self._decode, s, _event_handle(events[0]), _event_handle(events[1]))
        if rc:
            raise MQAError("mqa_decode_ex", rc)
        return self.out
