#!/usr/bin/env python3
"""MQA incremental decode on one MI355X: steps/s and effective KV GB/s.

Headline workload: batched serving decode, b=64 sequences, h=32 query heads
sharing G=1 K/V head, d_h=128, bf16 cache, pre-append lengths uniform in
[1, 8192], one kv_append per sequence, then the decode (split-K attention +
combine).  One step = append + decode for the whole batch.

Timing discipline:
  * R independently drawn caches are rotated step by step so every pass
    touches >= 1 GiB (several times the 256 MB Infinity Cache) and the K/V
    stream really comes from HBM;
  * W untimed warm-up steps; then K timed steps between two
    torch.cuda.synchronize() calls; steps are replayed from a HIP graph of R
    steps so host launch overhead stays out of the GPU timeline;
  * bytes per step are counted from the actual lens of each timed step.

The JSON line adds
  * roofline: the split-K attention kernel (the dominant kernel), timed with
    HIP events recorded on its own stream around each launch;
  * cpu_baseline: the fp64 oracle on the host cores, on a bounded sample;
  * extra: the other workloads (MQA/MHA comparison point, GQA long context,
    causal prefill), each with its own rotation.
"""
from __future__ import annotations

import argparse
import json
import math
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


# --------------------------------------------------------------------------- decode


class DecodeBench:
    """R rotated copies of one decode workload living in HBM."""

    def __init__(self, cfg, R, torch, mqa, seed_base=0, fused=True):
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
            self.copies.append(dict(K=K, V=V, q=q, kn=kn, vn=vn, lens=lens))
            self.lens_host.append(lens_cpu.tolist())
        self.out = torch.empty(b, h, dh, dtype=cfg.dtype, device=dev)
        self.ws = mqa.workspace_for(h, self.copies[0]["K"])
        self.steps = []
        for c in self.copies:
            kw = dict(k_new=c["kn"], v_new=c["vn"]) if cfg.append else {}
            self.steps.append(mqa.DecodeStep(c["q"], c["K"], c["V"], c["lens"], cfg.scale,
                                             out=self.out, workspace=self.ws, fused=fused, **kw))
        self.appends = [0] * R   # appends issued per copy so far
        self.elem = 2 if cfg.dtype == torch.bfloat16 else 4

    # effective (algorithmic) bytes of one step of copy r given its current appends
    def kv_bytes(self, r, extra_appends=0):
        cfg = self.cfg
        n_app = self.appends[r] + extra_appends
        tot = 0
        for L0 in self.lens_host[r]:
            L = min(L0 + (n_app if cfg.append else 0), cfg.m_cap)
            tot += L
        return tot * cfg.G * cfg.dh * 2 * self.elem

    def other_bytes(self):
        """q in, o out, lens; plus for an appending step the new rows read and written."""
        cfg = self.cfg
        b = 2 * cfg.b * cfg.h * cfg.dh * self.elem + 4 * cfg.b
        if cfg.append:
            b += 2 * 2 * cfg.b * cfg.G * cfg.dh * self.elem + 4 * cfg.b
        return b

    def flops(self, r, extra_appends=0):
        cfg = self.cfg
        return 4 * cfg.h * cfg.dh * self.kv_bytes(r, extra_appends) // (cfg.G * cfg.dh * 2 * self.elem)

    def eager(self, n, events=None):
        for i in range(n):
            r = i % self.R
            self.appends[r] += 1 if self.cfg.append else 0
            self.steps[r](None if events is None else events[i])

    def capture(self):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for r in range(self.R):
                    self.steps[r]()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        return g

    def timed(self, steps, use_graph):
        """Returns (seconds, total effective KV bytes, total bytes, flops, steps run)."""
        torch = self.torch
        R = self.R
        graph = self.capture() if use_graph else None
        n_rep = max(1, math.ceil(steps / R)) if use_graph else None
        n_steps = n_rep * R if use_graph else steps
        kv = tot = fl = 0
        for i in range(n_steps):
            r = i % R
            kv += self.kv_bytes(r, 1 + i // R)
            fl += self.flops(r, 1 + i // R)
        tot = kv + n_steps * self.other_bytes()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if use_graph:
            for _ in range(n_rep):
                graph.replay()
        else:
            self.eager(n_steps)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if use_graph:
            for r in range(R):
                self.appends[r] += n_rep if self.cfg.append else 0
        return dt, kv, tot, fl, n_steps

    def kernel_timing(self, n):
        """Average duration of the decode kernel (HIP events recorded on its launch
        stream right around it) and its algorithmic bytes per launch, over n eager
        steps queued behind a GPU sleep so that launches never wait for the host."""
        torch = self.torch
        ev = HipEvents(n)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.02))      # ~20 ms of GPU spin: launches queue up
        kv = 0
        other = self.other_bytes()
        for i in range(n):
            r = i % self.R
            self.appends[r] += 1 if self.cfg.append else 0
            kv += self.kv_bytes(r)
            self.steps[r](ev.pairs[i])
        torch.cuda.synchronize()
        dur = [ev.elapsed_s(i) for i in range(n)]
        ev.close()
        return sum(dur) / n, (kv + n * other) / n, kv / n


def decode_result(bench, steps, warmup, use_graph):
    bench.eager(warmup)
    bench.torch.cuda.synchronize()
    dt, kv, tot, fl, n = bench.timed(steps, use_graph)
    return dict(seconds=dt, steps=n, steps_per_s=n / dt, ms_per_step=1e3 * dt / n,
                kv_gbps=kv / dt / 1e9, total_gbps=tot / dt / 1e9,
                kv_frac_of_peak=kv / dt / 1e9 / HBM_PEAK_GBPS, tflops=fl / dt / 1e12,
                kv_bytes_per_step=kv / n)


# --------------------------------------------------------------------------- prefill


def prefill_result(cfg, steps, torch, mqa, R=2):
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
    for i in range(3):
        Q, K, V = copies[i % R]
        mqa.prefill_causal(Q, K, V, cfg.scale, cache_K=cK, cache_V=cV, lens=lens, out=O)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        Q, K, V = copies[i % R]
        mqa.prefill_causal(Q, K, V, cfg.scale, cache_K=cK, cache_V=cV, lens=lens, out=O)
    e1.record()
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) * 1e-3 / steps
    pairs = cfg.n * (cfg.n + 1) // 2
    flops = 4 * cfg.b * cfg.h * cfg.dh * pairs
    return dict(ms_per_call=dt * 1e3, tflops=flops / dt / 1e12,
                mfma_frac_of_peak=flops / dt / 1e12 / BF16_PEAK_TFLOPS,
                causal_flops=flops)


def attend_result(cfg, steps, torch, mqa, R=2):
    """Attention over a fixed memory with a key-padding mask (encoder-decoder
    attention).  Flops count every (query, memory position) pair: masked
    logits are computed too."""
    dev = torch.device("cuda")
    copies = []
    for r in range(R):
        g = torch.Generator(device=dev).manual_seed(cfg.seed * 1000 + r)
        gc = torch.Generator().manual_seed(cfg.seed * 1000 + r)
        Q = torch.randn(cfg.b, cfg.n, cfg.h, cfg.dh, generator=g, device=dev).to(cfg.dtype)
        K = torch.randn(cfg.b, cfg.m, cfg.G, cfg.dh, generator=g, device=dev).to(cfg.dtype)
        V = torch.randn(cfg.b, cfg.m, cfg.G, cfg.dh, generator=g, device=dev).to(cfg.dtype)
        mem = torch.randint(cfg.mem_lo, cfg.mem_hi + 1, (cfg.b,), generator=gc)
        mask = torch.where(torch.arange(cfg.m)[None, :] < mem[:, None], 0.0, float("-inf"))
        copies.append((Q, K, V, mask.view(cfg.b, 1, 1, cfg.m).to(dev)))
    O = torch.empty_like(copies[0][0])
    for i in range(3):
        Q, K, V, mk = copies[i % R]
        mqa.attend(Q, K, V, cfg.scale, mask=mk, out=O)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        Q, K, V, mk = copies[i % R]
        mqa.attend(Q, K, V, cfg.scale, mask=mk, out=O)
    e1.record()
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) * 1e-3 / steps
    flops = 4 * cfg.b * cfg.h * cfg.dh * cfg.n * cfg.m
    return dict(ms_per_call=dt * 1e3, tflops=flops / dt / 1e12,
                mfma_frac_of_peak=flops / dt / 1e12 / BF16_PEAK_TFLOPS, flops=flops)


# --------------------------------------------------------------------------- beam


def beam_result(cfg, steps, torch, mqa, R=4):
    """Beam step = mqa_kv_reorder_to (random parents, ~3/4 of the rows move;
    the lengths alternate between two arrays per cache) followed by the fused
    append + decode on the new lengths, over R rotated caches, replayed from
    a HIP graph of 2R steps (each cache once in each direction).  Bytes: the
    decode's K/V of every hypothesis plus the reorder's moved rows, read and
    written."""
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
        c = dict(K=K, V=V, lens=[lens0, torch.empty_like(lens0)],
                 parent=parent.to(dev),
                 q=torch.randn(b, h, dh, generator=gg, device=dev).to(cfg.dtype),
                 kn=torch.randn(b, G, dh, generator=gg, device=dev).to(cfg.dtype),
                 vn=torch.randn(b, G, dh, generator=gg, device=dev).to(cfg.dtype))
        copies.append(c)
        per_src.append(src_lens.tolist())
        # moved rows per source (a moved row copies its source's length)
        moved.append([sum(1 for i in range(s_i * beam, (s_i + 1) * beam)
                          if int(parent[i]) != i % beam) for s_i in range(cfg.sources)])
    out = torch.empty(b, h, dh, dtype=cfg.dtype, device=dev)
    ws = mqa.workspace_for(h, copies[0]["K"])
    dsteps = [[mqa.DecodeStep(c["q"], c["K"], c["V"], c["lens"][ph], cfg.scale, out=out,
                              workspace=ws, k_new=c["kn"], v_new=c["vn"]) for ph in range(2)]
              for c in copies]

    def step(r, ph):
        """Reorder lens[ph] -> lens[1 - ph], then append + decode on lens[1 - ph]."""
        c = copies[r]
        mqa.kv_reorder(c["K"], c["V"], c["lens"][ph], c["parent"], beam, lens_out=c["lens"][1 - ph])
        dsteps[r][1 - ph]()

    appends = [0] * R

    def step_bytes(r, n_app):
        # hypotheses of a source share its length before and after every step
        rd = mv = 0
        for s_i, L0 in enumerate(per_src[r]):
            L_pre = min(L0 + n_app, m_cap)        # length entering this step
            L = min(L_pre + 1, m_cap)             # after the append
            rd += beam * L * row * 2              # decode reads K and V
            mv += moved[r][s_i] * L_pre
        return rd, 2 * 2 * mv * row               # moved rows: read + write, K and V

    for ph in range(2):                            # warm-up: two steps per cache
        for r in range(R):
            step(r, ph)
            appends[r] += 1
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for ph in range(2):
                for r in range(R):
                    step(r, ph)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    n_rep = max(1, math.ceil(steps / (2 * R)))
    # (capturing records the steps without running them: appends unchanged)
    kv = mvb = 0
    for k in range(n_rep):
        for j in range(2):
            for r in range(R):
                a, m = step_bytes(r, appends[r] + 2 * k + j)
                kv += a
                mvb += m
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_rep):
        g.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    n = n_rep * 2 * R
    return dict(ms_per_step=1e3 * dt / n, steps_per_s=n / dt,
                us_per_output_token=1e6 * dt / n / cfg.sources,
                kv_gbps=kv / dt / 1e9, reorder_gbps=mvb / dt / 1e9,
                total_gbps=(kv + mvb) / dt / 1e9,
                total_frac_of_peak=(kv + mvb) / dt / 1e9 / HBM_PEAK_GBPS,
                moved_rows_per_step=sum(sum(m) for m in moved) / R, hypotheses=b)


# --------------------------------------------------------------------------- cpu baseline


def cpu_baseline(budget_s=12.0):
    """The oracle (fp64 C, threads over rows) on the host: full serving steps
    (append + decode, all 64 sequences) repeated until ~budget_s."""
    import numpy as np
    import oracle
    from query_decode_attention_amd import workloads as W
    cfg = W.C3
    inp = W.decode_inputs(cfg)
    Kr, _ = oracle._raw(inp["K"])
    Vr, _ = oracle._raw(inp["V"])
    Kr, Vr = Kr.copy(), Vr.copy()
    lens = inp["lens"].numpy().copy()
    threads = oracle.default_threads()
    n = 0
    kv = 0
    t0 = time.perf_counter()
    while True:
        oracle.kv_append(inp["k_new"], inp["v_new"], Kr, Vr, lens)
        oracle.decode(inp["q"], Kr, Vr, lens, cfg.scale, nthreads=threads)
        n += 1
        kv += int(np.minimum(lens, cfg.m_cap).sum()) * cfg.G * cfg.dh * 2 * 2
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="steps/s", cores=threads, kind="oracle",
                sample=f"{n} full serving steps (append + decode, b=64, h=32, d_h=128, "
                       f"ragged lens 1..8192) in {dt:.1f} s; fp64 C oracle with {threads} "
                       f"threads over (sequence, head) rows",
                kv_gbps=kv / dt / 1e9, seconds=dt)


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
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--rotate", type=int, default=8, help="cache copies for the headline")
    ap.add_argument("--eager", action="store_true", help="launch steps eagerly (no HIP graph)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--kernel-steps", type=int, default=64)
    ap.add_argument("--two-call", action="store_true",
                    help="append with mqa_kv_append, then mqa_decode (two launches per step)")
    ap.add_argument("--probe-copy", type=int, default=0, metavar="MB",
                    help="also run 3 plain device copies of MB MiB (calibrates profiler byte counters)")
    ap.add_argument("--only", choices=["c2", "c4", "c5", "encdec", "beam4", "paper"],
                    help="run just this secondary workload and print its numbers (for profiling "
                         "one workload alone); no headline line")
    args = ap.parse_args()

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

    if args.only:
        steps = args.steps if args.steps != ap.get_default("steps") else None
        run = {
            "c2": lambda: decode_result(DecodeBench(W.C2, 64, torch, mqa), steps or 640, 64,
                                        use_graph),
            "c4": lambda: decode_result(DecodeBench(W.C4, 1, torch, mqa), steps or 30, 3,
                                        use_graph),
            "c5": lambda: prefill_result(W.C5, steps or 10, torch, mqa),
            "encdec": lambda: attend_result(W.ENCDEC, steps or 10, torch, mqa),
            "beam4": lambda: beam_result(W.BEAM4, steps or 96, torch, mqa),
            "paper": lambda: decode_result(DecodeBench(W.PAPER_MQA, 8, torch, mqa), steps or 320,
                                           32, use_graph),
        }[args.only]
        r = run()
        print(json.dumps({"only": args.only, **{k: (round(v, 4) if isinstance(v, float) else v)
                                               for k, v in r.items()}}), flush=True)
        return

    log("headline: serving decode c3 (b=64, h=32, G=1, d_h=128, lens U[1,8192] + append)")
    head = DecodeBench(W.C3, args.rotate, torch, mqa, fused=not args.two_call)
    res = decode_result(head, args.steps, args.warmup, use_graph)
    log(f"headline {res['steps_per_s']:.1f} steps/s, {res['kv_gbps']:.1f} GB/s KV "
        f"({100 * res['kv_frac_of_peak']:.1f}% of 8 TB/s)")
    kdur, kbytes, kkv = head.kernel_timing(args.kernel_steps)
    achieved = kbytes / kdur / 1e9
    log(f"decode kernel avg {kdur * 1e6:.2f} us, {achieved:.1f} GB/s")
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=measured_traffic(),
                    kernel="decode_kernel<bf16,128,8>",
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
        c2 = decode_result(DecodeBench(W.C2, 64, torch, mqa), 640, 64, use_graph)
        torch.cuda.empty_cache()
        c2m = decode_result(DecodeBench(W.C2_MHA, 4, torch, mqa), 200, 8, use_graph)
        torch.cuda.empty_cache()
        extra["c2_mqa_b8_m2048"] = {k: round(v, 4) for k, v in c2.items()}
        extra["c2_mha_b8_m2048"] = {k: round(v, 4) for k, v in c2m.items()}
        extra["mha_over_mqa_time_ratio"] = round(c2m["ms_per_step"] / c2["ms_per_step"], 2)
        log(f"MHA/MQA time ratio {extra['mha_over_mqa_time_ratio']}")
        log("the pages' speed setting: b=1024, h=8, d_h=128, 128 positions, MQA vs MHA")
        pq = decode_result(DecodeBench(W.PAPER_MQA, 8, torch, mqa), 320, 32, use_graph)
        torch.cuda.empty_cache()
        ph = decode_result(DecodeBench(W.PAPER_MHA, 4, torch, mqa), 160, 8, use_graph)
        torch.cuda.empty_cache()
        extra["paper_mqa_b1024_h8_m128"] = {k: round(v, 4) for k, v in pq.items()}
        extra["paper_mha_b1024_h8_m128"] = {k: round(v, 4) for k, v in ph.items()}
        extra["paper_mha_over_mqa_time_ratio"] = round(ph["ms_per_step"] / pq["ms_per_step"], 2)
        log(f"paper setting MHA/MQA time ratio {extra['paper_mha_over_mqa_time_ratio']}")
        log("c4 GQA long context")
        c4 = decode_result(DecodeBench(W.C4, 1, torch, mqa), 30, 3, use_graph)
        torch.cuda.empty_cache()
        extra["c4_gqa_b32_h64_g8_m32k"] = {k: round(v, 4) for k, v in c4.items()}
        log("c5 causal prefill")
        extra["c5_prefill_b4_n4096"] = {k: round(v, 4) if isinstance(v, float) else v
                                        for k, v in prefill_result(W.C5, 10, torch, mqa).items()}
        extra["c5_prefill_b4_n4096"]["frac_of_torch_bf16_matmul"] = round(
            extra["c5_prefill_b4_n4096"]["tflops"] / ceil["torch_bf16_matmul_tflops"], 4)
        torch.cuda.empty_cache()
        log("encoder-decoder attention: non-causal over a fixed memory, key-padding mask")
        extra["encdec_b4_n4096_m4096"] = {k: round(v, 4) if isinstance(v, float) else v
                                          for k, v in attend_result(W.ENCDEC, 10, torch,
                                                                    mqa).items()}
        extra["encdec_b4_n4096_m4096"]["frac_of_torch_bf16_matmul"] = round(
            extra["encdec_b4_n4096_m4096"]["tflops"] / ceil["torch_bf16_matmul_tflops"], 4)
        torch.cuda.empty_cache()
        log("beam-4 step: reorder + fused append + decode, 16 sources x 4 beams")
        extra["beam4_b16x4_ragged8k"] = {k: round(v, 4) if isinstance(v, float) else v
                                         for k, v in beam_result(W.BEAM4, 96, torch, mqa).items()}
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host cores)")
        cpu = cpu_baseline()
        cpu = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in cpu.items()}

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
