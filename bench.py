#!/usr/bin/env python3
"""MQA incremental decode on one MI355X: steps/s and effective KV GB/s.

Headline workload: batched serving decode, b=64 sequences, h=32 query heads
sharing G=1 K/V head, d_h=128, bf16 cache, pre-append lengths uniform in
[1, 8192], one kv_append per sequence, then the decode (split-K attention +
combine).  One step = append + decode for the whole batch.

Timing discipline:
  * R independently drawn caches are rotated step by step so every pass
    touches >= 1 GiB (several times the 256 MB Infinity Cache) and the K/V
    stream really comes from HBM; each copy has its own lens and workspace;
  * W untimed warm-up steps; then exactly K steps (step i on copy i % R) are
    captured in one HIP graph and replayed in T trials (default 7), each
    bracketed by a pair of events on the launch stream, with every copy's
    lens restored (outside the events) before each trial; the median is the
    reported figure, min and max are given beside it;
  * bytes per step are counted from the actual lens of each timed step.

The JSON line adds
  * roofline: the split-K attention kernel (the dominant kernel), timed with
    HIP events recorded on its own stream around each launch;
  * cpu_baseline: the fp64 oracle on the host cores, on a bounded sample;
  * extra: the other workloads (MQA/MHA comparison point, the pages' speed
    setting, the serial decoding loop with full and local attention, GQA
    long context, causal prefill, encoder-decoder attention, beam-4), each
    with its own rotation and the same trial discipline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_c3_hbm_traffic.md")
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, vendor figure
METRIC = "MQA decode steps/s + effective KV GB/s (%HBM peak), b=64 h=32 d=128 m=8K"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """Raw HIP events for kernel timing, created without the system-scope
    fence that a default event record adds, so that an event pair around one
    kernel measures that kernel (as the profiler's dispatch timestamps do)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            e0, e1 = ctypes.c_void_p(), ctypes.c_void_p()
            for e in (e0, e1):
                if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE):
                    raise RuntimeError("hipEventCreateWithFlags failed")
            self.pairs.append((e0.value, e1.value))

    def elapsed_s(self, i):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.pairs[i][0], self.pairs[i][1]):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e-3

    def close(self):
        for e0, e1 in self.pairs:
            self.hip.hipEventDestroy(e0)
            self.hip.hipEventDestroy(e1)


def measured_traffic():
    """HBM bytes per decode-kernel launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's readings),
    or None when the kernel sources changed since those counters were taken."""
    import hashlib
    try:
        line = next(l for l in open(TRAFFIC_PROFILE) if l.strip().startswith("traffic-json:"))
    except (OSError, StopIteration):
        return None
    info = json.loads(line.split("traffic-json:", 1)[1])
    h = hashlib.sha256()
    for f in info["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return info["traffic_bytes_per_launch"] if h.hexdigest() == info["sources_sha256"] else None


# --------------------------------------------------------------------------- timing


def event_trials(torch, run, trials):
    """Seconds of `run()` (work it enqueues on the current stream), timed by a
    pair of events on that stream, over `trials` trials; `run` may take a
    `prepare` step outside the events (see timed_trials)."""
    out = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(trials):
        e0.record()
        run()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1) * 1e-3)
    return out


def timed_trials(torch, prepare, run, trials):
    """As event_trials, with `prepare()` (e.g. restoring lens) issued and
    completed before each trial's first event."""
    out = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(trials):
        prepare()
        torch.cuda.synchronize()
        e0.record()
        run()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1) * 1e-3)
    return out


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def capture(torch, body):
    """A HIP graph of everything `body()` enqueues (captured on a side
    stream, so nothing runs while it is recorded)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


# --------------------------------------------------------------------------- decode


class DecodeBench:
    """R rotated copies of one decode workload living in HBM, each with its
    own lens and workspace.  Step i of a timed run uses copy i % R; before
    every trial the lens of every copy are restored, so every trial appends
    (and reads) exactly the same bytes."""

    def __init__(self, cfg, R, torch, mqa, seed_base=0, fused=True, window=0):
        self.cfg, self.R, self.torch = cfg, R, torch
        dev = torch.device("cuda")
        b, h, G, dh, m_cap = cfg.b, cfg.h, cfg.G, cfg.dh, cfg.m_cap
        self.copies = []
        self.lens_host = []
        for r in range(R):
            gg = torch.Generator(device=dev).manual_seed(cfg.seed * 1000 + seed_base + r)
            gc = torch.Generator().manual_seed(cfg.seed * 1000 + seed_base + r)
            K = torch.randn(b, m_cap, G, dh, generator=gg, device=dev).to(cfg.dtype)
            V = torch.randn(b, m_cap, G, dh, generator=gg, device=dev).to(cfg.dtype)
            q = torch.randn(b, h, dh, generator=gg, device=dev).to(cfg.dtype)
            kn = torch.randn(b, G, dh, generator=gg, device=dev).to(cfg.dtype)
            vn = torch.randn(b, G, dh, generator=gg, device=dev).to(cfg.dtype)
            lens_cpu = torch.randint(cfg.lens_lo, cfg.lens_hi + 1, (b,), generator=gc,
                                     dtype=torch.int64).to(torch.int32)
            lens = lens_cpu.to(dev)
            self.copies.append(dict(K=K, V=V, q=q, kn=kn, vn=vn, lens=lens, lens0=lens.clone(),
                                    ws=mqa.workspace_for(h, K)))
            self.lens_host.append(lens_cpu.tolist())
        self.out = torch.empty(b, h, dh, dtype=cfg.dtype, device=dev)
        self.steps = []
        for c in self.copies:
            kw = dict(k_new=c["kn"], v_new=c["vn"]) if cfg.append else {}
            self.steps.append(mqa.DecodeStep(c["q"], c["K"], c["V"], c["lens"], cfg.scale,
                                             out=self.out, workspace=c["ws"], fused=fused,
                                             window=window, **kw))
        self.window = window
        self.elem = 2 if cfg.dtype == torch.bfloat16 else 4

    def restore(self):
        for c in self.copies:
            c["lens"].copy_(c["lens0"])

    def kv_bytes(self, r, n_app):
        """Algorithmic K/V bytes of a step of copy r that is its n_app-th
        append since the lens were restored (n_app counts this step)."""
        cfg = self.cfg
        tot = 0
        for L0 in self.lens_host[r]:
            L = min(L0 + (n_app if cfg.append else 0), cfg.m_cap)
            tot += min(L, self.window) if self.window > 0 else L
        return tot * cfg.G * cfg.dh * 2 * self.elem

    def other_bytes(self):
        """q in, o out, lens; plus for an appending step the new rows read and
        written and lens written."""
        cfg = self.cfg
        b = 2 * cfg.b * cfg.h * cfg.dh * self.elem + 4 * cfg.b
        if cfg.append:
            b += 2 * 2 * cfg.b * cfg.G * cfg.dh * self.elem + 4 * cfg.b
        return b

    def flops(self, kv):
        cfg = self.cfg
        return 4 * cfg.h * cfg.dh * (kv // (cfg.G * cfg.dh * 2 * self.elem))

    def eager(self, n):
        for i in range(n):
            self.steps[i % self.R]()

    def run(self, steps, warmup, trials, use_graph=True):
        """Median (and spread) over `trials` of exactly `steps` steps."""
        torch = self.torch
        self.restore()
        self.eager(warmup)
        torch.cuda.synchronize()
        if use_graph:
            g = capture(torch, lambda: self.eager(steps))
            body = g.replay
        else:
            body = lambda: self.eager(steps)
        kv = sum(self.kv_bytes(i % self.R, i // self.R + 1) for i in range(steps))
        secs = timed_trials(torch, self.restore, body, trials)
        dt = median(secs)
        tot = kv + steps * self.other_bytes()
        return dict(steps=steps, trials=trials, seconds_median=dt, seconds_min=min(secs),
                    seconds_max=max(secs), steps_per_s=steps / dt, ms_per_step=1e3 * dt / steps,
                    ms_per_step_min=1e3 * min(secs) / steps,
                    ms_per_step_max=1e3 * max(secs) / steps,
                    kv_gbps=kv / dt / 1e9, total_gbps=tot / dt / 1e9,
                    kv_frac_of_peak=kv / dt / 1e9 / HBM_PEAK_GBPS, tflops=self.flops(kv) / dt / 1e12,
                    kv_bytes_per_step=kv / steps)

    def kernel_timing(self, n):
        """Average duration of the decode kernel (HIP events recorded on its
        launch stream right around it) and its algorithmic bytes per launch,
        over n eager steps queued behind a GPU sleep so that launches never
        wait for the host."""
        torch = self.torch
        self.restore()
        ev = HipEvents(n)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.02))      # ~20 ms of GPU spin: launches queue up
        kv = 0
        for i in range(n):
            r = i % self.R
            kv += self.kv_bytes(r, i // self.R + 1)
            self.steps[r](ev.pairs[i])
        torch.cuda.synchronize()
        dur = [ev.elapsed_s(i) for i in range(n)]
        ev.close()
        return sum(dur) / n, (kv + n * self.other_bytes()) / n, kv / n


def rounded(d):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}


# --------------------------------------------------------------------------- serial loop


class SerialBench:
    """Serial incremental decoding: `tokens` steps through `layers`
    self-attention layers, each step a fused append + decode per layer on a
    cache that grows from 0 to `tokens` positions.  The lens of all layers
    are reset (one fill kernel) at the start of the loop, inside the timed
    graph."""

    def __init__(self, cfg, torch, mqa):
        self.cfg, self.torch = cfg, torch
        dev = torch.device("cuda")
        b, h, G, dh, n = cfg.b, cfg.h, cfg.G, cfg.dh, cfg.tokens
        self.lens = torch.zeros(cfg.layers, b, dtype=torch.int32, device=dev)
        self.out = torch.empty(b, h, dh, dtype=cfg.dtype, device=dev)
        self.layers = []
        self.steps = []
        for l in range(cfg.layers):
            gg = torch.Generator(device=dev).manual_seed(cfg.seed * 1000 + l)
            K = torch.randn(b, n, G, dh, generator=gg, device=dev).to(cfg.dtype)
            V = torch.randn(b, n, G, dh, generator=gg, device=dev).to(cfg.dtype)
            q = torch.randn(b, h, dh, generator=gg, device=dev).to(cfg.dtype)
            kn = torch.randn(b, G, dh, generator=gg, device=dev).to(cfg.dtype)
            vn = torch.randn(b, G, dh, generator=gg, device=dev).to(cfg.dtype)
            ws = mqa.workspace_for(h, K)
            self.layers.append((K, V, q, kn, vn, ws))
            self.steps.append(mqa.DecodeStep(q, K, V, self.lens[l], cfg.scale, out=self.out,
                                             workspace=ws, k_new=kn, v_new=vn,
                                             window=cfg.window))
        self.elem = 2 if cfg.dtype == torch.bfloat16 else 4

    def loop(self):
        self.lens.zero_()
        for _ in range(self.cfg.tokens):
            for st in self.steps:
                st()

    def kv_bytes(self):
        cfg = self.cfg
        vis = sum(min(t, cfg.window) if cfg.window > 0 else t for t in range(1, cfg.tokens + 1))
        return cfg.layers * cfg.b * vis * cfg.G * cfg.dh * 2 * self.elem

    def run(self, trials):
        torch, cfg = self.torch, self.cfg
        self.loop()                                    # warm-up, eager
        torch.cuda.synchronize()
        g = capture(torch, self.loop)
        secs = event_trials(torch, g.replay, trials)
        dt = median(secs)
        kv = self.kv_bytes()
        per_token = dt / cfg.tokens
        return dict(trials=trials, loop_ms_median=1e3 * dt, loop_ms_min=1e3 * min(secs),
                    loop_ms_max=1e3 * max(secs), us_per_token_step=1e6 * per_token,
                    us_per_output_token=1e6 * per_token / cfg.b,
                    us_per_layer_step=1e6 * per_token / cfg.layers,
                    kv_bytes_per_loop=kv, kv_gbps=kv / dt / 1e9,
                    kv_frac_of_peak=kv / dt / 1e9 / HBM_PEAK_GBPS)


# --------------------------------------------------------------------------- prefill


def prefill_result(cfg, trials, torch, mqa, R=2, calls=4):
    """Causal prefill (with the cache write and lens); R input copies
    alternate; median over trials of `calls` calls."""
    dev = torch.device("cuda")
    copies = []
    for r in range(R):
        g = torch.Generator(device=dev).manual_seed(cfg.seed * 1000 + r)
        Q = torch.randn(cfg.b, cfg.n, cfg.h, cfg.dh, generator=g, device=dev).to(cfg.dtype)
        K = torch.randn(cfg.b, cfg.n, cfg.G, cfg.dh, generator=g, device=dev).to(cfg.dtype)
        V = torch.randn(cfg.b, cfg.n, cfg.G, cfg.dh, generator=g, device=dev).to(cfg.dtype)
        copies.append((Q, K, V))
    O = torch.empty_like(copies[0][0])
    cK = torch.empty(cfg.b, cfg.n, cfg.G, cfg.dh, dtype=cfg.dtype, device=dev)
    cV = torch.empty_like(cK)
    lens = torch.zeros(cfg.b, dtype=torch.int32, device=dev)

    def body():
        for i in range(calls):
            Q, K, V = copies[i % R]
            mqa.prefill_causal(Q, K, V, cfg.scale, cache_K=cK, cache_V=cV, lens=lens, out=O)

    body()
    torch.cuda.synchronize()
    secs = event_trials(torch, body, trials)
    dt = median(secs) / calls
    pairs = cfg.n * (cfg.n + 1) // 2
    flops = 4 * cfg.b * cfg.h * cfg.dh * pairs
    return dict(trials=trials, ms_per_call=dt * 1e3, ms_per_call_min=1e3 * min(secs) / calls,
                ms_per_call_max=1e3 * max(secs) / calls, tflops=flops / dt / 1e12,
                mfma_frac_of_peak=flops / dt / 1e12 / BF16_PEAK_TFLOPS, causal_flops=flops)


def attend_result(cfg, trials, torch, mqa, R=2, calls=4):
    """Attention over a fixed memory with a key-padding mask (encoder-decoder
    attention).  The kernel stops each sequence after its last 32-key tile
    with a visible key, so `flops` counts the (query, key) pairs of the tiles
    it runs (visible keys rounded up to 32); `useful_tflops` counts only the
    pairs the mask leaves visible, `all_pairs_tflops` every pair of the m
    positions."""
    dev = torch.device("cuda")
    copies = []
    visible = []
    for r in range(R):
        g = torch.Generator(device=dev).manual_seed(cfg.seed * 1000 + r)
        gc = torch.Generator().manual_seed(cfg.seed * 1000 + r)
        Q = torch.randn(cfg.b, cfg.n, cfg.h, cfg.dh, generator=g, device=dev).to(cfg.dtype)
        K = torch.randn(cfg.b, cfg.m, cfg.G, cfg.dh, generator=g, device=dev).to(cfg.dtype)
        V = torch.randn(cfg.b, cfg.m, cfg.G, cfg.dh, generator=g, device=dev).to(cfg.dtype)
        mem = torch.randint(cfg.mem_lo, cfg.mem_hi + 1, (cfg.b,), generator=gc)
        mask = torch.where(torch.arange(cfg.m)[None, :] < mem[:, None], 0.0, float("-inf"))
        copies.append((Q, K, V, mask.view(cfg.b, 1, 1, cfg.m).to(dev)))
        visible.append((int(mem.sum()),
                        int(sum(min(cfg.m, -(-int(v) // 32) * 32) for v in mem))))
    O = torch.empty_like(copies[0][0])

    def body():
        for i in range(calls):
            Q, K, V, mk = copies[i % R]
            mqa.attend(Q, K, V, cfg.scale, mask=mk, out=O)

    body()
    torch.cuda.synchronize()
    secs = event_trials(torch, body, trials)
    dt = median(secs) / calls
    all_pairs = 4 * cfg.b * cfg.h * cfg.dh * cfg.n * cfg.m
    useful = sum(4 * cfg.h * cfg.dh * cfg.n * visible[i % R][0] for i in range(calls)) / calls
    flops = sum(4 * cfg.h * cfg.dh * cfg.n * visible[i % R][1] for i in range(calls)) / calls
    return dict(trials=trials, ms_per_call=dt * 1e3, ms_per_call_min=1e3 * min(secs) / calls,
                ms_per_call_max=1e3 * max(secs) / calls, tflops=flops / dt / 1e12,
                mfma_frac_of_peak=flops / dt / 1e12 / BF16_PEAK_TFLOPS, flops=flops,
                useful_tflops=useful / dt / 1e12,
                useful_frac_of_peak=useful / dt / 1e12 / BF16_PEAK_TFLOPS,
                all_pairs_tflops=all_pairs / dt / 1e12)


# --------------------------------------------------------------------------- beam


def beam_result(cfg, steps, trials, torch, mqa, R=4, warmup=8):
    """Beam step = mqa_kv_reorder_to (random parents, ~3/4 of the rows move;
    the lengths alternate between two arrays per cache) followed by the fused
    append + decode on the new lengths.  Step k uses cache k % R, which takes
    its (k // R)-th step; the lens of every cache are restored before each
    trial.  Bytes: the decode's K/V of every hypothesis plus the reorder's
    moved rows, read and written."""
    dev = torch.device("cuda")
    b, h, G, dh, m_cap, beam = cfg.b, cfg.h, cfg.G, cfg.dh, cfg.m_cap, cfg.beam
    elem = 2 if cfg.dtype == torch.bfloat16 else 4
    row = G * dh * elem
    copies, per_src, moved = [], [], []
    for r in range(R):
        gg = torch.Generator(device=dev).manual_seed(cfg.seed * 1000 + r)
        gc = torch.Generator().manual_seed(cfg.seed * 1000 + r)
        K = torch.randn(b, m_cap, G, dh, generator=gg, device=dev).to(cfg.dtype)
        V = torch.randn(b, m_cap, G, dh, generator=gg, device=dev).to(cfg.dtype)
        src_lens = torch.randint(cfg.lens_lo, cfg.lens_hi + 1, (cfg.sources,), generator=gc,
                                 dtype=torch.int64)
        parent = torch.randint(0, beam, (b,), generator=gc, dtype=torch.int64).to(torch.int32)
        lens0 = src_lens.repeat_interleave(beam).to(torch.int32).to(dev)
        c = dict(K=K, V=V, lens=[lens0.clone(), torch.empty_like(lens0)], lens0=lens0,
                 parent=parent.to(dev), ws=mqa.workspace_for(h, K),
                 q=torch.randn(b, h, dh, generator=gg, device=dev).to(cfg.dtype),
                 kn=torch.randn(b, G, dh, generator=gg, device=dev).to(cfg.dtype),
                 vn=torch.randn(b, G, dh, generator=gg, device=dev).to(cfg.dtype))
        copies.append(c)
        per_src.append(src_lens.tolist())
        # moved rows per source (a moved row copies its source's length)
        moved.append([sum(1 for i in range(s_i * beam, (s_i + 1) * beam)
                          if int(parent[i]) != i % beam) for s_i in range(cfg.sources)])
    out = torch.empty(b, h, dh, dtype=cfg.dtype, device=dev)
    dsteps = [[mqa.DecodeStep(c["q"], c["K"], c["V"], c["lens"][ph], cfg.scale, out=out,
                              workspace=c["ws"], k_new=c["kn"], v_new=c["vn"]) for ph in range(2)]
              for c in copies]

    def run(n):
        for k in range(n):
            r, ph = k % R, (k // R) % 2
            c = copies[r]
            mqa.kv_reorder(c["K"], c["V"], c["lens"][ph], c["parent"], beam,
                           lens_out=c["lens"][1 - ph])
            dsteps[r][1 - ph]()

    def restore():
        for c in copies:
            c["lens"][0].copy_(c["lens0"])

    def step_bytes(r, j):
        # hypotheses of a source share its length before and after every step
        rd = mv = 0
        for s_i, L0 in enumerate(per_src[r]):
            L_pre = min(L0 + j, m_cap)            # length entering this step
            L = min(L_pre + 1, m_cap)             # after the append
            rd += beam * L * row * 2              # decode reads K and V
            mv += moved[r][s_i] * L_pre
        return rd, 2 * 2 * mv * row               # moved rows: read + write, K and V

    restore()
    run(max(2 * R, warmup))
    torch.cuda.synchronize()
    g = capture(torch, lambda: run(steps))
    kv = mvb = 0
    for k in range(steps):
        a, m = step_bytes(k % R, k // R)
        kv += a
        mvb += m
    secs = timed_trials(torch, restore, g.replay, trials)
    dt = median(secs)
    return dict(steps=steps, trials=trials, ms_per_step=1e3 * dt / steps,
                ms_per_step_min=1e3 * min(secs) / steps, ms_per_step_max=1e3 * max(secs) / steps,
                steps_per_s=steps / dt, us_per_output_token=1e6 * dt / steps / cfg.sources,
                kv_gbps=kv / dt / 1e9, reorder_gbps=mvb / dt / 1e9,
                total_gbps=(kv + mvb) / dt / 1e9,
                total_frac_of_peak=(kv + mvb) / dt / 1e9 / HBM_PEAK_GBPS,
                moved_rows_per_step=sum(sum(m) for m in moved) / R, hypotheses=b)


# --------------------------------------------------------------------------- cpu baseline


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s=12.0):
    """The oracle (fp64 C, threads over (sequence, head) rows) on the host:
    full serving steps (append + decode, all 64 sequences) repeated until
    ~budget_s; the value is the median step rate.  Threads: the CPUs this
    process may run on, at most 16 (the CPU share of one GPU on a shared
    8-GPU node)."""
    import numpy as np
    import oracle
    from query_decode_attention_amd import workloads as W
    cfg = W.C3
    inp = W.decode_inputs(cfg)
    Kr, _ = oracle._raw(inp["K"])
    Vr, _ = oracle._raw(inp["V"])
    Kr, Vr = Kr.copy(), Vr.copy()
    lens = inp["lens"].numpy().copy()
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(16, avail))
    times, kvs = [], []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.kv_append(inp["k_new"], inp["v_new"], Kr, Vr, lens)
        oracle.decode(inp["q"], Kr, Vr, lens, cfg.scale, nthreads=threads)
        times.append(time.perf_counter() - t0)
        kvs.append(int(np.minimum(lens, cfg.m_cap).sum()) * cfg.G * cfg.dh * 2 * 2)
        if time.perf_counter() - t_all >= budget_s:
            break
    dt = median(times)
    n = len(times)
    return dict(value=1.0 / dt, unit="steps/s", cores=threads, kind="oracle",
                sample=f"{n} full serving steps (append + decode, b=64, h=32, d_h=128, "
                       f"ragged lens 1..8192) in {sum(times):.1f} s, median step "
                       f"{1e3 * dt:.1f} ms; fp64 C oracle with {threads} threads over "
                       f"(sequence, head) rows",
                threads=threads, nproc=os.cpu_count(), cpus_available=avail,
                cpu_model=cpu_model(), kv_gbps=median(kvs) / dt / 1e9, seconds=sum(times))


# ------------------------------------------------------------------- ceilings


def measured_ceilings(torch, mqa):
    """Practical ceilings measured on this GPU, next to the vendor peaks: the
    HBM read rate of a plain streaming kernel over 1 GiB (mqa_read_probe), and
    the bf16 rate of a large torch.matmul (8192^3)."""
    dev = torch.device("cuda")
    out = {}
    buf = torch.zeros(1 << 28, dtype=torch.float32, device=dev)          # 1 GiB
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        mqa.read_probe(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        mqa.read_probe(buf, sink)
    e1.record()
    e1.synchronize()
    out["read_probe_gbps"] = round(buf.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del buf
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(3):
        c = torch.matmul(a, b)
    reps = 10
    e0.record()
    for _ in range(reps):
        c = torch.matmul(a, b)
    e1.record()
    e1.synchronize()
    out["torch_bf16_matmul_tflops"] = round(2 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12,
                                            1)
    del a, b, c
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- main


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400, help="timed steps per trial (exactly)")
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--trials", type=int, default=7, help="trials; the median is reported")
    ap.add_argument("--rotate", type=int, default=8, help="cache copies for the headline")
    ap.add_argument("--eager", action="store_true", help="launch steps eagerly (no HIP graph)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--kernel-steps", type=int, default=64)
    ap.add_argument("--two-call", action="store_true",
                    help="append with mqa_kv_append, then mqa_decode (two launches per step)")
    ap.add_argument("--probe-copy", type=int, default=0, metavar="MB",
                    help="also run 3 plain device copies of MB MiB (calibrates profiler byte counters)")
    ap.add_argument("--only", choices=["c2", "c4", "c5", "encdec", "beam4", "paper", "serial",
                                       "headline"],
                    help="run just this workload and print its numbers (for profiling one "
                         "workload alone); no headline line")
    args = ap.parse_args()
    trials = max(5, args.trials)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: the decode path is built and measured on a "
                  "single MI355X (multi-GPU sharding is a design note, not a run). "
                  f"Refusing --gpus {args.gpus}.", file=sys.stderr)
        sys.exit(2)

    import torch
    import query_decode_attention_amd as mqa
    from query_decode_attention_amd import workloads as W
    mqa.load()
    torch.cuda.set_device(0)
    use_graph = not args.eager

    if args.probe_copy:
        n = args.probe_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"probe copy: 3 x {args.probe_copy} MiB read + written")
        del src, dst

    def dec(cfg, R, steps, warmup, window=0):
        r = DecodeBench(cfg, R, torch, mqa, window=window).run(steps, warmup, trials, use_graph)
        torch.cuda.empty_cache()
        return rounded(r)

    def serial(cfg):
        r = SerialBench(cfg, torch, mqa).run(trials)
        torch.cuda.empty_cache()
        return rounded(r)

    if args.only:
        steps = args.steps if args.steps != ap.get_default("steps") else None
        run = {
            "headline": lambda: dec(W.C3, args.rotate, steps or 400, args.warmup),
            "c2": lambda: dec(W.C2, 64, steps or 640, 64),
            "c4": lambda: dec(W.C4, 1, steps or 30, 3),
            "c5": lambda: rounded(prefill_result(W.C5, trials, torch, mqa)),
            "encdec": lambda: rounded(attend_result(W.ENCDEC, trials, torch, mqa)),
            "beam4": lambda: rounded(beam_result(W.BEAM4, steps or 96, trials, torch, mqa)),
            "paper": lambda: dec(W.PAPER_MQA, 8, steps or 320, 32),
            "serial": lambda: serial(W.SERIAL_MQA),
        }[args.only]
        r = run()
        print(json.dumps({"only": args.only, **r}), flush=True)
        return

    log("headline: serving decode c3 (b=64, h=32, G=1, d_h=128, lens U[1,8192] + append)")
    head = DecodeBench(W.C3, args.rotate, torch, mqa, fused=not args.two_call)
    res = head.run(args.steps, args.warmup, trials, use_graph)
    log(f"headline {res['steps_per_s']:.1f} steps/s (median of {trials} trials of "
        f"{args.steps} steps; {res['ms_per_step_min'] * 1e3:.2f}..{res['ms_per_step_max'] * 1e3:.2f}"
        f" us/step), {res['kv_gbps']:.1f} GB/s KV ({100 * res['kv_frac_of_peak']:.1f}% of 8 TB/s)")
    kdur, kbytes, kkv = head.kernel_timing(args.kernel_steps)
    achieved = kbytes / kdur / 1e9
    log(f"decode kernel avg {kdur * 1e6:.2f} us, {achieved:.1f} GB/s")
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=measured_traffic(),
                    kernel="decode_kernel<bf16,128,8,false>",
                    avg_launch_us=round(kdur * 1e6, 3),
                    algorithmic_bytes_per_launch=int(kbytes))
    del head
    torch.cuda.empty_cache()

    log("measured ceilings: streaming read of 1 GiB, bf16 torch.matmul 8192^3")
    ceil = measured_ceilings(torch, mqa)
    ceil["kv_frac_of_read_probe"] = round(res["kv_gbps"] / ceil["read_probe_gbps"], 4)
    ceil["decode_kernel_frac_of_read_probe"] = round(achieved / ceil["read_probe_gbps"], 4)
    log(f"read probe {ceil['read_probe_gbps']} GB/s, bf16 matmul {ceil['torch_bf16_matmul_tflops']} "
        f"TFLOP/s")

    extra = {}
    if not args.no_extra:
        log("c2 MQA vs MHA comparison point")
        c2 = dec(W.C2, 64, 640, 64)
        c2m = dec(W.C2_MHA, 4, 200, 8)
        extra["c2_mqa_b8_m2048"] = c2
        extra["c2_mha_b8_m2048"] = c2m
        extra["mha_over_mqa_time_ratio"] = round(c2m["ms_per_step"] / c2["ms_per_step"], 2)
        log(f"MHA/MQA time ratio {extra['mha_over_mqa_time_ratio']}")
        log("the pages' speed setting: b=1024, h=8, d_h=128, 128 positions (decode only)")
        pq = dec(W.PAPER_MQA, 8, 320, 32)
        ph = dec(W.PAPER_MHA, 4, 160, 8)
        extra["paper_mqa_b1024_h8_m128_decode_only"] = pq
        extra["paper_mha_b1024_h8_m128_decode_only"] = ph
        extra["paper_mha_over_mqa_time_ratio"] = round(ph["ms_per_step"] / pq["ms_per_step"], 2)
        log(f"paper setting MHA/MQA time ratio {extra['paper_mha_over_mqa_time_ratio']}")
        log("serial decoding loop: 128 tokens x 6 layers, caches growing 1..128, b=1024, h=8")
        for key, cfg in (("serial_mqa", W.SERIAL_MQA), ("serial_mha", W.SERIAL_MHA),
                         ("serial_local_mqa_w32", W.SERIAL_LOCAL_MQA),
                         ("serial_local_mha_w32", W.SERIAL_LOCAL_MHA)):
            extra[key] = serial(cfg)
            log(f"{key}: {extra[key]['us_per_output_token']:.4f} us per output token "
                f"({extra[key]['loop_ms_median']:.3f} ms per loop)")
        extra["serial_mha_over_mqa_time_ratio"] = round(
            extra["serial_mha"]["loop_ms_median"] / extra["serial_mqa"]["loop_ms_median"], 2)
        extra["serial_local_mha_over_local_mqa_time_ratio"] = round(
            extra["serial_local_mha_w32"]["loop_ms_median"] /
            extra["serial_local_mqa_w32"]["loop_ms_median"], 2)
        log("c4 GQA long context")
        extra["c4_gqa_b32_h64_g8_m32k"] = dec(W.C4, 1, 30, 3)
        log("c5 causal prefill")
        extra["c5_prefill_b4_n4096"] = rounded(prefill_result(W.C5, trials, torch, mqa))
        extra["c5_prefill_b4_n4096"]["frac_of_torch_bf16_matmul"] = round(
            extra["c5_prefill_b4_n4096"]["tflops"] / ceil["torch_bf16_matmul_tflops"], 4)
        torch.cuda.empty_cache()
        log("encoder-decoder attention: non-causal over a fixed memory, key-padding mask")
        extra["encdec_b4_n4096_m4096"] = rounded(attend_result(W.ENCDEC, trials, torch, mqa))
        extra["encdec_b4_n4096_m4096"]["frac_of_torch_bf16_matmul"] = round(
            extra["encdec_b4_n4096_m4096"]["tflops"] / ceil["torch_bf16_matmul_tflops"], 4)
        torch.cuda.empty_cache()
        log("beam-4 step: reorder + fused append + decode, 16 sources x 4 beams")
        extra["beam4_b16x4_ragged8k"] = rounded(beam_result(W.BEAM4, 96, trials, torch, mqa))
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host cores)")
        cpu = rounded(cpu_baseline())

    line = {
        "metric": METRIC,
        "value": round(res["steps_per_s"], 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "serving MQA decode: kv append + split-K decode + combine",
                   "b": 64, "h": 32, "G": 1, "d_h": 128, "lens": "uniform [1,8192] + 1 append",
                   "m_cap": W.C3.m_cap, "rotated_caches": args.rotate,
                   "launch": ("eager" if args.eager else "hip-graph") +
                             (", kv_append + decode + combine kernels" if args.two_call
                              else ", decode (append fused) + combine kernels")},
        "trials": {"n": trials, "statistic": "median", "timer": "events on the launch stream",
                   "ms_per_step_min": round(res["ms_per_step_min"], 5),
                   "ms_per_step_max": round(res["ms_per_step_max"], 5)},
        "kv_gbps": round(res["kv_gbps"], 1),
        "kv_frac_of_hbm_peak": round(res["kv_frac_of_peak"], 4),
        "roofline": roofline,
        "ceilings": ceil,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
