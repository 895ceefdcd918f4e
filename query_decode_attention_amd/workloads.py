"""Seeded synthetic workloads for MQA/GQA decoding and causal prefill.

This module only draws random inputs and names shapes.  It holds none of the
method's arithmetic, so both the HIP path and the CPU oracle can be fed from
it without sharing any computation.

Recipe (identical for every consumer):
  * generator: ``torch.Generator('cpu').manual_seed(seed)``; one call per
    tensor in the fixed draw order q, K, V, k_new, v_new, lens (prefill: Q, K, V);
  * values: fp32 N(0, 1), rounded to bfloat16 by round-to-nearest-even
    (``Tensor.to(torch.bfloat16)``) for bf16 workloads;
  * lens: uniform integers in the configured range, or a constant.

The shapes stand in for the paper's workload (a WMT14 encoder-decoder on
TPUv2, batch 1024, length 128: study notes section 6.2), which needs data and
trained weights that are not used here; only the attention core's shapes and
value distributions matter to it.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    dtype: torch.dtype
    b: int
    h: int
    G: int
    dh: int
    m_cap: int
    lens_lo: int          # pre-append lens drawn uniformly from [lens_lo, lens_hi]
    lens_hi: int
    append: bool          # one kv_append per sequence before the decode
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dh)


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    dtype: torch.dtype
    b: int
    n: int
    h: int
    G: int
    dh: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dh)


# The five workloads (shapes of the pages' problem statement, enlarged to
# serving sizes).  Seeds are 1000 + workload number.
C1 = DecodeConfig("c1_tiny_fp32", torch.float32, b=1, h=4, G=1, dh=64, m_cap=128,
                  lens_lo=128, lens_hi=128, append=False, seed=1001)
C2 = DecodeConfig("c2_mqa_b8_m2048", torch.bfloat16, b=8, h=32, G=1, dh=128, m_cap=2048,
                  lens_lo=2048, lens_hi=2048, append=False, seed=1002)
C2_MHA = DecodeConfig("c2_mha_b8_m2048", torch.bfloat16, b=8, h=32, G=32, dh=128,
                      m_cap=2048, lens_lo=2048, lens_hi=2048, append=False, seed=1012)
C3 = DecodeConfig("c3_serving_b64_ragged8k", torch.bfloat16, b=64, h=32, G=1, dh=128,
                  m_cap=8192 + 256, lens_lo=1, lens_hi=8192, append=True, seed=1003)
C4 = DecodeConfig("c4_gqa_b32_h64_g8_m32k", torch.bfloat16, b=32, h=64, G=8, dh=128,
                  m_cap=32768, lens_lo=32768, lens_hi=32768, append=False, seed=1004)
C5 = PrefillConfig("c5_prefill_b4_n4096", torch.bfloat16, b=4, n=4096, h=32, G=1, dh=128,
                   seed=1005)

# The pages' own incremental-decoding speed setting (study notes, section
# 6.2, which reports the paper's section 4.3 and Table 2): batch 1024, h = 8
# heads of d_h = 128, length 128, with the decoder self-attention K/V padded
# to the full length of 128 so that every step costs the same.  One step here
# is the attention over all 128 positions (decode only, no append).  MQA, and
# the MHA comparison point (one K/V head per query head).
PAPER_MQA = DecodeConfig("paper_mqa_b1024_h8_m128", torch.bfloat16, b=1024, h=8, G=1, dh=128,
                         m_cap=128, lens_lo=128, lens_hi=128, append=False, seed=1021)
PAPER_MHA = DecodeConfig("paper_mha_b1024_h8_m128", torch.bfloat16, b=1024, h=8, G=8, dh=128,
                         m_cap=128, lens_lo=128, lens_hi=128, append=False, seed=1022)


@dataclasses.dataclass(frozen=True)
class SerialConfig:
    """Serial incremental decoding of ``tokens`` output tokens for ``b``
    sequences through ``layers`` decoder self-attention layers: every token
    appends one K/V row per sequence and layer and attends over the cache
    grown so far (1, 2, ..., tokens positions), so the whole loop re-reads
    sum_{t<=n} t = n(n+1)/2 cached positions (study notes, section 1.2).
    ``window`` > 0 is local attention over the last ``window`` positions."""
    name: str
    dtype: torch.dtype
    b: int
    h: int
    G: int
    dh: int
    tokens: int
    layers: int
    window: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dh)


# The pages' decoder at its speed setting (study notes, sections 6.1 and 6.2:
# 6 decoder layers, batch 1024, h = 8, d_k = d_v = 128, target length 128;
# the local variant attends over the current position and the 31 before it).
SERIAL_MQA = SerialConfig("serial_mqa_b1024_h8_n128_l6", torch.bfloat16, b=1024, h=8, G=1,
                          dh=128, tokens=128, layers=6, window=0, seed=1031)
SERIAL_MHA = SerialConfig("serial_mha_b1024_h8_n128_l6", torch.bfloat16, b=1024, h=8, G=8,
                          dh=128, tokens=128, layers=6, window=0, seed=1032)
SERIAL_LOCAL_MQA = SerialConfig("serial_local_mqa_b1024_h8_n128_l6_w32", torch.bfloat16, b=1024,
                                h=8, G=1, dh=128, tokens=128, layers=6, window=32, seed=1033)
SERIAL_LOCAL_MHA = SerialConfig("serial_local_mha_b1024_h8_n128_l6_w32", torch.bfloat16, b=1024,
                                h=8, G=8, dh=128, tokens=128, layers=6, window=32, seed=1034)

@dataclasses.dataclass(frozen=True)
class BeamConfig:
    """Beam decoding: ``sources`` source sequences x ``beam`` hypotheses, each
    hypothesis one cache row; the hypotheses of a source share its length."""
    name: str
    dtype: torch.dtype
    sources: int
    beam: int
    h: int
    G: int
    dh: int
    m_cap: int
    lens_lo: int          # per-source pre-step lens, uniform in [lens_lo, lens_hi]
    lens_hi: int
    seed: int

    @property
    def b(self) -> int:
        return self.sources * self.beam

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dh)


# Beam-4 serving step (the study notes' section 6.2 beam-4 rows) at the c3
# serving shapes: 16 sources x 4 beams = 64 cache rows.
BEAM4 = BeamConfig("beam4_b16x4_ragged8k", torch.bfloat16, sources=16, beam=4, h=32, G=1,
                   dh=128, m_cap=8192 + 256, lens_lo=1, lens_hi=8192, seed=1006)

@dataclasses.dataclass(frozen=True)
class MemoryConfig:
    """Attention of n queries over a fixed memory of m positions (encoder-
    decoder attention); each sequence's memory holds mem_len valid positions,
    the rest hidden by a key-padding mask."""
    name: str
    dtype: torch.dtype
    b: int
    n: int
    m: int
    h: int
    G: int
    dh: int
    mem_lo: int           # valid memory positions, uniform in [mem_lo, mem_hi]
    mem_hi: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dh)


# Encoder-decoder attention at the prefill's sizes (the study notes' section
# 6.1: multi-query layers also serve encoder-decoder attention).
ENCDEC = MemoryConfig("encdec_b4_n4096_m4096", torch.bfloat16, b=4, n=4096, m=4096, h=32, G=1,
                      dh=128, mem_lo=2048, mem_hi=4096, seed=1007)

DECODE_CONFIGS = {c.name: c for c in (C1, C2, C2_MHA, C3, C4)}
PREFILL_CONFIGS = {C5.name: C5}


def _normal(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    return x.to(dtype) if dtype != torch.float32 else x


def _normal_chunked(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    """Same draw as ``_normal`` (one contiguous stream of N(0,1)), produced in
    slices along dim 0 to bound host memory for multi-GB caches."""
    if dtype == torch.float32 or shape[0] <= 1:
        return _normal(g, shape, dtype)
    out = torch.empty(*shape, dtype=dtype)
    for i in range(shape[0]):
        out[i] = torch.randn(*shape[1:], generator=g, dtype=torch.float32).to(dtype)
    return out


def decode_inputs(cfg: DecodeConfig, seed: Optional[int] = None, b: Optional[int] = None,
                  m_cap: Optional[int] = None, lens_lo: Optional[int] = None,
                  lens_hi: Optional[int] = None):
    """CPU tensors for one decode step of ``cfg`` (optionally resized).

    Returns a dict with q [b,h,dh], K,V [b,m_cap,G,dh], k_new,v_new [b,G,dh]
    and lens int32 [b] (pre-append when cfg.append).
    """
    b = cfg.b if b is None else b
    m_cap = cfg.m_cap if m_cap is None else m_cap
    lo = cfg.lens_lo if lens_lo is None else lens_lo
    hi = cfg.lens_hi if lens_hi is None else lens_hi
    g = torch.Generator("cpu").manual_seed(cfg.seed if seed is None else seed)
    q = _normal(g, (b, cfg.h, cfg.dh), cfg.dtype)
    K = _normal_chunked(g, (b, m_cap, cfg.G, cfg.dh), cfg.dtype)
    V = _normal_chunked(g, (b, m_cap, cfg.G, cfg.dh), cfg.dtype)
    k_new = _normal(g, (b, cfg.G, cfg.dh), cfg.dtype)
    v_new = _normal(g, (b, cfg.G, cfg.dh), cfg.dtype)
    lens = torch.randint(lo, hi + 1, (b,), generator=g, dtype=torch.int64).to(torch.int32)
    return dict(q=q, K=K, V=V, k_new=k_new, v_new=v_new, lens=lens)


def beam_inputs(cfg: BeamConfig, steps: int = 1, seed: Optional[int] = None,
                sources: Optional[int] = None, m_cap: Optional[int] = None,
                lens_lo: Optional[int] = None, lens_hi: Optional[int] = None):
    """CPU tensors for ``steps`` beam steps of ``cfg`` (optionally resized).

    Draw order: K, V [b,m_cap,G,dh]; per-source lens (repeated over the
    source's beams); then per step: parent int32 [b] uniform in [0, beam),
    q [b,h,dh], k_new, v_new [b,G,dh].  Stacked per step along dim 0.
    """
    src_n = cfg.sources if sources is None else sources
    b = src_n * cfg.beam
    m_cap = cfg.m_cap if m_cap is None else m_cap
    lo = cfg.lens_lo if lens_lo is None else lens_lo
    hi = cfg.lens_hi if lens_hi is None else lens_hi
    g = torch.Generator("cpu").manual_seed(cfg.seed if seed is None else seed)
    K = _normal_chunked(g, (b, m_cap, cfg.G, cfg.dh), cfg.dtype)
    V = _normal_chunked(g, (b, m_cap, cfg.G, cfg.dh), cfg.dtype)
    per_src = torch.randint(lo, hi + 1, (src_n,), generator=g, dtype=torch.int64)
    lens = per_src.repeat_interleave(cfg.beam).to(torch.int32)
    parent, q, k_new, v_new = [], [], [], []
    for _ in range(steps):
        parent.append(torch.randint(0, cfg.beam, (b,), generator=g, dtype=torch.int64)
                      .to(torch.int32))
        q.append(_normal(g, (b, cfg.h, cfg.dh), cfg.dtype))
        k_new.append(_normal(g, (b, cfg.G, cfg.dh), cfg.dtype))
        v_new.append(_normal(g, (b, cfg.G, cfg.dh), cfg.dtype))
    return dict(K=K, V=V, lens=lens, parent=torch.stack(parent), q=torch.stack(q),
                k_new=torch.stack(k_new), v_new=torch.stack(v_new))


def memory_inputs(cfg: MemoryConfig, seed: Optional[int] = None, b: Optional[int] = None,
                  n: Optional[int] = None, m: Optional[int] = None):
    """CPU tensors Q [b,n,h,dh], K, V [b,m,G,dh], mem_len int32 [b] and the
    key-padding mask float32 [b,1,1,m] (0 on valid positions, -inf past
    mem_len).  Draw order Q, K, V, mem_len."""
    b = cfg.b if b is None else b
    n = cfg.n if n is None else n
    m = cfg.m if m is None else m
    g = torch.Generator("cpu").manual_seed(cfg.seed if seed is None else seed)
    Q = _normal_chunked(g, (b, n, cfg.h, cfg.dh), cfg.dtype)
    K = _normal_chunked(g, (b, m, cfg.G, cfg.dh), cfg.dtype)
    V = _normal_chunked(g, (b, m, cfg.G, cfg.dh), cfg.dtype)
    lo, hi = min(cfg.mem_lo, m), min(cfg.mem_hi, m)
    mem_len = torch.randint(lo, hi + 1, (b,), generator=g, dtype=torch.int64).to(torch.int32)
    mask = torch.zeros(b, 1, 1, m, dtype=torch.float32)
    for bi in range(b):
        mask[bi, 0, 0, int(mem_len[bi]):] = float("-inf")
    return dict(Q=Q, K=K, V=V, mem_len=mem_len, mask=mask)


def prefill_inputs(cfg: PrefillConfig, seed: Optional[int] = None, b: Optional[int] = None,
                   n: Optional[int] = None):
    """CPU tensors Q [b,n,h,dh], K,V [b,n,G,dh] for a causal prefill."""
    b = cfg.b if b is None else b
    n = cfg.n if n is None else n
    g = torch.Generator("cpu").manual_seed(cfg.seed if seed is None else seed)
    Q = _normal_chunked(g, (b, n, cfg.h, cfg.dh), cfg.dtype)
    K = _normal_chunked(g, (b, n, cfg.G, cfg.dh), cfg.dtype)
    V = _normal_chunked(g, (b, n, cfg.G, cfg.dh), cfg.dtype)
    return dict(Q=Q, K=K, V=V)


def poison_beyond(cache: torch.Tensor, lens: torch.Tensor, values=(float("nan"),
                  float("inf"), float("-inf"))) -> torch.Tensor:
    """Copy of ``cache`` [b,m_cap,G,dh] with every position >= lens[b] set to a
    cycling pattern of non-finite values (used to show they are never read)."""
    out = cache.clone()
    b, m_cap = cache.shape[:2]
    pat = torch.tensor(values, dtype=torch.float32).to(cache.dtype)
    for bi in range(b):
        L = int(lens[bi])
        if L < m_cap:
            tail = out[bi, L:]
            idx = torch.arange(tail.numel()) % pat.numel()
            out[bi, L:] = pat[idx].reshape(tail.shape)
    return out
