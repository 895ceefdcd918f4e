"""Seeded random sweep of the decode path against the fp64 oracle.

Each case draws its shape (batch, heads, groups, head size, dtype, cache
capacity), a length mix (uniform, mostly-short with a few long, with empty
rows, constant, a single long row among empty ones, all full), a local
window, a scale and the append mode from one fixed seed, so the cases are
the same on every run.  The mixes stress the work split: segments of very
different tile counts in one workgroup range, many segments per range, and
ranges that start or end inside a segment."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import announce, assert_parity
from query_decode_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import query_decode_attention_amd as mqa

MIXES = ("uniform", "short_long", "with_empty", "constant", "one_long", "full")


CAPS = (1, 31, 32, 33, 96, 257, 600, 1500, 4000)
# around the capacity up to which a decode keeps every sequence whole in one
# workgroup (8 tiles of 32 positions) and runs no merge
CAPS_WHOLE_EDGE = (200, 224, 255, 256, 257, 288)


def _draw_cases(n, seed, caps=CAPS, first=0):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        dh = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 1, 2, 4, 8]))
        hg = int(rng.choice([1, 2, 3, 5, 8, 16, 24, 32]))
        b = int(rng.choice([1, 2, 7, 33, 64, 65, 130, 300, 700, 2100]))
        m_cap = int(rng.choice(caps))
        mix = str(rng.choice(MIXES))
        append = bool(rng.random() < 0.5)
        if append and mix == "full":
            continue  # full caches under append are covered by their own test
        fused = bool(rng.random() < 0.6)
        window = 0 if rng.random() < 0.75 else int(rng.integers(1, m_cap + 2))
        scale_mult = float(rng.uniform(0.5, 2.0))
        # keep the oracle to seconds and the caches to a few hundred MB
        while b > 1 and (b * m_cap * G * dh > 40_000_000 or b * hg * G * m_cap * dh > 300_000_000):
            b = max(1, b // 3)
        cases.append((first + len(cases), dtype, b, hg * G, G, dh, m_cap, mix, append, fused, window,
                      scale_mult, int(rng.integers(1, 1 << 30))))
    return cases


CASES = _draw_cases(64, 20261203) + _draw_cases(24, 20261207, CAPS_WHOLE_EDGE, first=64)


def _lens(mix, b, m_cap, append, gen):
    top = m_cap - 1 if append else m_cap       # room for the appended row
    r = lambda lo, hi, n: torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int64)
    if mix == "uniform":
        lens = r(0, top, b)
    elif mix == "short_long":
        lens = r(0, min(top, 40), b)
        long_ = torch.rand(b, generator=gen) < 0.1
        lens[long_] = r(max(0, (7 * top) // 10), top, b)[long_]
    elif mix == "with_empty":
        lens = r(1 if top >= 1 else 0, top, b)
        lens[torch.rand(b, generator=gen) < 0.3] = 0
    elif mix == "constant":
        lens = torch.full((b,), int(r(0, top, 1)[0]), dtype=torch.int64)
    elif mix == "one_long":
        lens = torch.zeros(b, dtype=torch.int64)
        lens[int(r(0, b - 1, 1)[0])] = top
    else:  # full
        lens = torch.full((b,), m_cap, dtype=torch.int64)
    return lens.to(torch.int32)


def _id(c):
    i, dt, b, h, G, dh, m, mix, app, fused, win, _, _ = c
    a = ("fused" if fused else "2call") if app else "noapp"
    return f"{i:02d}-{dt}-b{b}h{h}G{G}d{dh}m{m}-{mix}-{a}-w{win}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_decode_random_sweep(case):
    i, dt, b, h, G, dh, m_cap, mix, append, fused, window, scale_mult, seed = case
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    announce(f"sweep {_id(case)} seed={seed}")
    cfg = W.DecodeConfig("sweep", dtype, b, h, G, dh, m_cap, 0, 0, append, seed)
    inp = W.decode_inputs(cfg)
    gen = torch.Generator("cpu").manual_seed(seed + 1)
    inp["lens"] = _lens(mix, b, m_cap, append, gen)
    scale = cfg.scale * scale_mult

    # oracle first, on the CPU copies (the GPU call updates its own copies)
    q, K, V, lens = inp["q"], inp["K"], inp["V"], inp["lens"].numpy().copy()
    if append:
        Kr, _ = oracle._raw(K)
        Vr, _ = oracle._raw(V)
        Kr, Vr = Kr.copy(), Vr.copy()
        oracle.kv_append(inp["k_new"], inp["v_new"], Kr, Vr, lens)
        K, V = Kr, Vr
    ref = oracle.decode(q, K, V, lens, scale, window=window)

    d = {k: v.cuda() for k, v in inp.items()}
    if append and fused:
        o = mqa.append_decode(d["q"], d["k_new"], d["v_new"], d["K"], d["V"], d["lens"], scale,
                              window=window)
    else:
        if append:
            mqa.kv_append(d["k_new"], d["v_new"], d["K"], d["V"], d["lens"])
        o = mqa.decode(d["q"], d["K"], d["V"], d["lens"], scale, window=window)
    torch.cuda.synchronize()
    assert_parity(o, ref, dtype, _id(case))
    assert np.array_equal(d["lens"].cpu().numpy(), lens), "lens after the step"
