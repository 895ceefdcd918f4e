"""Seeded random sweep of the causal prefill and of attention over a memory
against the fp64 oracle.

Each case draws its shape (batch, prompt or query length, memory length,
heads, groups, head size, dtype), a scale (usually 1/sqrt(d_h) times a
factor, sometimes zero or negative), a mask kind for attention (none, key
padding, a general additive mask, a general mask with hidden keys and fully
hidden rows) and, for the prefill, whether the cache is filled too, all from
one fixed seed, so the cases are the same on every run.  The lengths land on
and around the 32-key tiles and the row blocks of the workgroups; the head
counts per group cover the padded column layouts (1, 3, 5, 12, ...)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import announce, assert_parity
from query_decode_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import query_decode_attention_amd as mqa

LENGTHS = (1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 129, 200, 257, 320, 400)
HEADS_PER_GROUP = (1, 2, 3, 5, 8, 12, 16, 24, 32)
MASKS = ("none", "none", "pad", "full", "full_inf")


def _scale(rng, dh):
    u = rng.random()
    if u < 0.08:
        return 0.0
    if u < 0.16:
        return -float(rng.uniform(0.05, 0.3))
    return float(rng.uniform(0.5, 2.0)) / dh ** 0.5


def _shrink(b, work):
    # keep every oracle call to about a second
    while b > 1 and work(b) > 1.2e9:
        b -= 1
    return b


def _prefill_cases(n_cases, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        dh = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 1, 2, 4, 8]))
        hg = int(rng.choice(HEADS_PER_GROUP))
        n = int(rng.choice(LENGTHS))
        b = int(rng.integers(1, 4))
        b = _shrink(b, lambda bb: bb * n * n * hg * G * dh)
        fill = bool(rng.random() < 0.3)
        cases.append((i, dtype, b, n, hg * G, G, dh, _scale(rng, dh), fill,
                      int(rng.integers(1, 1 << 30))))
    return cases


def _attend_cases(n_cases, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        dh = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 1, 2, 4, 8]))
        hg = int(rng.choice(HEADS_PER_GROUP))
        n = int(rng.choice(LENGTHS))
        m = int(rng.choice(LENGTHS + (600,)))
        b = int(rng.integers(1, 4))
        kind = str(rng.choice(MASKS))
        # a general mask is b*h*n*m floats on the host and the device
        if kind.startswith("full"):
            while n * m * hg * G > 2_000_000 and n > 1:
                n = max(1, n // 2)
        b = _shrink(b, lambda bb: bb * n * m * hg * G * dh)
        cases.append((i, dtype, b, n, m, hg * G, G, dh, kind, _scale(rng, dh),
                      int(rng.integers(1, 1 << 30))))
    return cases


PREFILL_CASES = _prefill_cases(40, 20261204)
ATTEND_CASES = _attend_cases(40, 20261205)
DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def _pid(c):
    i, dt, b, n, h, G, dh, scale, fill, _ = c
    return f"{i:02d}-{dt}-b{b}n{n}h{h}G{G}d{dh}-s{scale:+.3f}" + ("-cache" if fill else "")


def _aid(c):
    i, dt, b, n, m, h, G, dh, kind, scale, _ = c
    return f"{i:02d}-{dt}-b{b}n{n}m{m}h{h}G{G}d{dh}-{kind}-s{scale:+.3f}"


@pytest.mark.parametrize("case", PREFILL_CASES, ids=_pid)
def test_prefill_sweep(case):
    i, dt, b, n, h, G, dh, scale, fill, seed = case
    dtype = DTYPES[dt]
    what = f"prefill sweep {_pid(case)}"
    announce(what)
    cfg = W.PrefillConfig("sweep", dtype, b, n, h, G, dh, seed)
    inp = W.prefill_inputs(cfg)
    Q, K, V = inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda()
    if fill:
        m_cap = n + 7
        cK = torch.full((b, m_cap, G, dh), float("nan"), dtype=dtype, device="cuda")
        cV = torch.full((b, m_cap, G, dh), float("nan"), dtype=dtype, device="cuda")
        lens = torch.full((b,), -5, dtype=torch.int32, device="cuda")
        O = mqa.prefill_causal(Q, K, V, scale, cache_K=cK, cache_V=cV, lens=lens)
    else:
        O = mqa.prefill_causal(Q, K, V, scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], scale)
    assert_parity(O, ref, dtype, what)
    if fill:
        # positions [0, n) hold the prompt's K / V bit for bit; the rest is
        # untouched; every lens entry is n
        bits = lambda t: t.contiguous().cpu().view(torch.uint8)
        assert torch.equal(bits(cK[:, :n]), bits(inp["K"])), what + ": cache K"
        assert torch.equal(bits(cV[:, :n]), bits(inp["V"])), what + ": cache V"
        assert bool(torch.isnan(cK[:, n:].float()).all()) and bool(torch.isnan(cV[:, n:].float()).all())
        assert torch.equal(lens.cpu(), torch.full((b,), n, dtype=torch.int32)), what + ": lens"


def _mask(kind, b, h, n, m, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    if kind == "none":
        return None
    if kind == "pad":
        # visible prefix lengths in [0, m]: 0 (every key hidden) included
        vis = torch.randint(0, m + 1, (b,), generator=g)
        mask = torch.zeros(b, 1, 1, m)
        for bi in range(b):
            mask[bi, 0, 0, int(vis[bi]):] = float("-inf")
        return mask
    mask = torch.randn(b, h, n, m, generator=g) * 1.5
    if kind == "full_inf":
        mask[torch.rand(b, h, n, m, generator=g) < 0.4] = float("-inf")
        mask[b - 1, 0, n - 1, :] = float("-inf")   # a row with every key hidden
    return mask


@pytest.mark.parametrize("case", ATTEND_CASES, ids=_aid)
def test_attend_sweep(case):
    i, dt, b, n, m, h, G, dh, kind, scale, seed = case
    dtype = DTYPES[dt]
    what = f"attend sweep {_aid(case)}"
    announce(what)
    cfg = W.MemoryConfig("sweep", dtype, b, n, m, h, G, dh, m, m, seed)
    inp = W.memory_inputs(cfg)
    mask = _mask(kind, b, h, n, m, seed + 1)
    out = mqa.attend(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), scale,
                     mask=None if mask is None else mask.cuda())
    torch.cuda.synchronize()
    if mask is None:
        ref = oracle.attend(inp["Q"], inp["K"], inp["V"], scale)
    else:
        full = mask.expand(b, h, n, m).contiguous()
        ref = oracle.attend(inp["Q"], inp["K"], inp["V"], scale, full.numpy())
    assert_parity(out, ref, dtype, what)
