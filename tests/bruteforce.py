"""A second, independent high-precision implementation for tiny shapes.

Pure Python (``math.fsum`` for every sum, one query at a time), written
straight from the attention definition (study notes section 2:
S = Q K^T / sqrt(d_h), A = softmax(S), O = A V) so the C oracle can be
checked against something that is not itself.  Only for b, h, L, d_h of a
few units: it is quadratic Python.
"""
from __future__ import annotations

import math

import numpy as np


def attend(qvec, keys, values, scale):
    """softmax(scale * q.k_j) weighted sum of values; keys/values are lists."""
    if not keys:
        return [0.0] * len(qvec), []
    logits = [scale * math.fsum(a * b for a, b in zip(qvec, k)) for k in keys]
    top = max(logits)
    e = [math.exp(x - top) for x in logits]
    z = math.fsum(e)
    w = [x / z for x in e]
    out = [math.fsum(wj * v[d] for wj, v in zip(w, values)) for d in range(len(values[0]))]
    return out, w


def decode(q, K, V, lens, scale, window=0):
    """q [b,h,dh], K/V [b,m,G,dh] as float64 numpy; returns [b,h,dh]."""
    b, h, dh = q.shape
    m, G = K.shape[1], K.shape[2]
    hg = h // G
    out = np.zeros((b, h, dh))
    for bi in range(b):
        L = max(0, min(int(lens[bi]), m))
        j0 = max(0, L - window) if window > 0 else 0
        for i in range(h):
            g = i // hg
            keys = [list(K[bi, j, g]) for j in range(j0, L)]
            vals = [list(V[bi, j, g]) for j in range(j0, L)]
            if keys:
                out[bi, i] = attend(list(q[bi, i]), keys, vals, scale)[0]
    return out


def prefill(Q, K, V, scale):
    """Causal: row t sees keys 0..t.  Q [b,n,h,dh], K/V [b,n,G,dh]."""
    b, n, h, dh = Q.shape
    G = K.shape[2]
    hg = h // G
    out = np.zeros((b, n, h, dh))
    for bi in range(b):
        for t in range(n):
            for i in range(h):
                g = i // hg
                keys = [list(K[bi, j, g]) for j in range(t + 1)]
                vals = [list(V[bi, j, g]) for j in range(t + 1)]
                out[bi, t, i] = attend(list(Q[bi, t, i]), keys, vals, scale)[0]
    return out


def memory(Q, K, V, scale, mask=None):
    """Non-causal attention over a memory with an additive mask (paper review
    section 2.3: softmax(logits + mask)).  Q [b,n,h,dh], K/V [b,m,G,dh],
    mask [b,h,n,m] or None; a row whose logits are all -inf gives zeros."""
    b, n, h, dh = Q.shape
    m, G = K.shape[1], K.shape[2]
    hg = h // G
    out = np.zeros((b, n, h, dh))
    for bi in range(b):
        for t in range(n):
            for i in range(h):
                g = i // hg
                logits = [scale * math.fsum(x * y for x, y in zip(Q[bi, t, i], K[bi, j, g]))
                          + (0.0 if mask is None else float(mask[bi, i, t, j]))
                          for j in range(m)]
                top = max(logits)
                if top == -math.inf:
                    continue
                e = [math.exp(x - top) for x in logits]
                z = math.fsum(e)
                for d in range(dh):
                    out[bi, t, i, d] = math.fsum(ej / z * V[bi, j, g, d] for j, ej in enumerate(e))
    return out
