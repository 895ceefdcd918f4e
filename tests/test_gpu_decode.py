"""GPU parity of the decode path (append + split-K decode + combine) against
the fp64 oracle, on the same seeded inputs, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import announce, assert_parity
from query_decode_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import query_decode_attention_amd as mqa


def to_dev(d):
    return {k: v.cuda() for k, v in d.items()}


def run_decode(inp, scale, window=0, append=False, fused=True):
    """Runs (optional append +) decode on the GPU; returns (o, device tensors).

    fused=True appends inside the decode kernel (mqa_append_decode);
    fused=False issues mqa_kv_append then mqa_decode."""
    d = to_dev(inp)
    if append and fused:
        o = mqa.append_decode(d["q"], d["k_new"], d["v_new"], d["K"], d["V"], d["lens"], scale,
                              window=window)
    else:
        if append:
            mqa.kv_append(d["k_new"], d["v_new"], d["K"], d["V"], d["lens"])
        o = mqa.decode(d["q"], d["K"], d["V"], d["lens"], scale, window=window)
    torch.cuda.synchronize()
    return o, d


def oracle_step(inp, scale, window=0, append=False):
    q, K, V, lens = inp["q"], inp["K"], inp["V"], inp["lens"].numpy().copy()
    if append:
        Kr, _ = oracle._raw(K)
        Vr, _ = oracle._raw(V)
        Kr, Vr = Kr.copy(), Vr.copy()
        oracle.kv_append(inp["k_new"], inp["v_new"], Kr, Vr, lens)
        K, V = Kr, Vr
    return oracle.decode(q, K, V, lens, scale, window=window), lens


def make(dtype, b, h, G, dh, m_cap, lo, hi, seed, append=False):
    cfg = W.DecodeConfig("t", dtype, b, h, G, dh, m_cap, lo, hi, append, seed)
    return cfg, W.decode_inputs(cfg)


# ------------------------------------------------------------------ small grids


CASES = [
    # dtype, b, h, G, dh, m_cap, lens range
    (torch.bfloat16, 3, 32, 1, 128, 300, 1, 300),       # MQA, ragged, tail tiles
    (torch.bfloat16, 2, 32, 32, 128, 97, 60, 97),      # MHA (h/G = 1), m_cap not /32
    (torch.bfloat16, 4, 16, 2, 128, 256, 1, 256),      # GQA h/G = 8
    (torch.bfloat16, 2, 8, 1, 64, 160, 33, 160),       # d_h = 64
    (torch.bfloat16, 5, 24, 1, 64, 64, 1, 64),         # h/G = 24 (not a power of two)
    (torch.float32, 1, 4, 1, 64, 128, 128, 128),       # the tiny fp32 workload
    (torch.float32, 3, 8, 2, 128, 200, 1, 200),        # fp32, d_h 128, GQA
    (torch.float32, 2, 32, 1, 64, 130, 100, 130),      # fp32, full head block
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{str(c[0])[6:]}-b{c[1]}h{c[2]}G{c[3]}d{c[4]}m{c[5]}")
def test_decode_parity_grid(case):
    dtype, b, h, G, dh, m_cap, lo, hi = case
    announce(f"decode grid {case}")
    cfg, inp = make(dtype, b, h, G, dh, m_cap, lo, hi, seed=7000 + b * 31 + h + G + dh)
    o, _ = run_decode(inp, cfg.scale)
    ref, _ = oracle_step(inp, cfg.scale)
    assert_parity(o, ref, dtype, f"grid {case}")


# Caches of at most 8 tiles: every workgroup takes whole sequences, so the
# library writes no partial records (and does not launch the combine; after an
# append the decode kernel bumps lens itself).  The workspace is filled with a
# sentinel first; past its schedule header ((b + 4) int32, padded to 256
# bytes) it must still hold it afterwards.
WHOLE_CASES = [
    # dtype, b, h, G, dh, m_cap, lens range
    (torch.bfloat16, 300, 32, 1, 128, 256, 0, 256),     # MQA, ragged, empty sequences
    (torch.bfloat16, 1024, 8, 1, 128, 128, 128, 128),   # the pages' setting (uniform lengths)
    (torch.bfloat16, 77, 16, 4, 64, 200, 1, 200),       # GQA, d_h 64
    (torch.bfloat16, 2, 32, 32, 128, 64, 1, 64),        # MHA, fewer sequences than workgroups
    (torch.float32, 50, 8, 2, 128, 96, 0, 96),
]


@pytest.mark.parametrize("append", [False, True])
@pytest.mark.parametrize("case", WHOLE_CASES, ids=lambda c: f"{str(c[0])[6:]}-b{c[1]}h{c[2]}G{c[3]}d{c[4]}m{c[5]}")
def test_decode_short_caches_whole_segments(case, append):
    dtype, b, h, G, dh, m_cap, lo, hi = case
    announce(f"decode whole sequences {case} append={append}")
    cfg, inp = make(dtype, b, h, G, dh, m_cap, lo, hi, seed=7400 + b + h + G + dh + append)
    if append:
        lens = inp["lens"].clone()
        lens[::5] = m_cap  # full caches: no new row, lens kept, the flag set
        lens[1::11] = -3   # a negative length: no row either, nothing visible (zeros)
        inp["lens"] = lens
    d = to_dev(inp)
    ws = mqa.workspace_for(h, d["K"])
    ws.fill_(0xAB)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if append:
        o = mqa.append_decode(d["q"], d["k_new"], d["v_new"], d["K"], d["V"], d["lens"], cfg.scale,
                              workspace=ws, err_flag=err)
    else:
        o = mqa.decode(d["q"], d["K"], d["V"], d["lens"], cfg.scale, workspace=ws)
    torch.cuda.synchronize()
    ref, lens_ref = oracle_step(inp, cfg.scale, append=append)
    assert_parity(o, ref, dtype, f"whole {case}")
    assert d["lens"].cpu().tolist() == lens_ref.tolist()
    header = ((b + 4) * 4 + 255) // 256 * 256
    assert bool((ws[header:] == 0xAB).all()), "a partial record was written"
    if append:
        assert err.item() == 1
        Kr, _ = oracle._raw(inp["K"])
        Vr, _ = oracle._raw(inp["V"])
        Kr, Vr = Kr.copy(), Vr.copy()
        oracle.kv_append(inp["k_new"], inp["v_new"], Kr, Vr, inp["lens"].numpy().copy())
        Kg, _ = oracle._raw(d["K"].cpu())
        Vg, _ = oracle._raw(d["V"].cpu())
        assert np.array_equal(Kg, Kr) and np.array_equal(Vg, Vr), "cache rows differ"
    else:
        # a window over the same caches
        o = mqa.decode(d["q"], d["K"], d["V"], d["lens"], cfg.scale, window=17, workspace=ws)
        torch.cuda.synchronize()
        ref, _ = oracle_step(inp, cfg.scale, window=17)
        assert_parity(o, ref, dtype, f"whole window {case}")


# Caches of at most 8 tiles take whole sequences per workgroup; the schedule
# tests below also run with m_cap just above that (the same lengths), so that
# the split-K schedule's lens layouts stay covered.
SPLIT_M = 300


@pytest.mark.parametrize("m_cap", [96, SPLIT_M])
@pytest.mark.parametrize("append,fused", [(False, True), (True, True), (True, False)])
def test_decode_many_sequences_multi_chunk_scan(append, fused, m_cap):
    """b > 64 exercises the multi-chunk wave scan of the schedule."""
    announce(f"decode b=600 m_cap={m_cap} append={append} fused={fused}")
    cfg, inp = make(torch.bfloat16, 600, 8, 1, 64, m_cap, 0, 95, seed=7100 + append)
    o, _ = run_decode(inp, cfg.scale, append=append, fused=fused)
    ref, _ = oracle_step(inp, cfg.scale, append=append)
    assert_parity(o, ref, torch.bfloat16, "b=600")


@pytest.mark.parametrize("append", [False, True])
def test_decode_many_long_sequences_lead_in_schedule(append):
    """b > 64 with more tiles than one per wave of the grid: the schedule
    with lead-in units across several 64-lane chunks (the step above has
    fewer tiles, so it runs without lead-in)."""
    announce(f"decode b=150 long append={append}")
    cfg, inp = make(torch.bfloat16, 150, 16, 2, 64, 1000, 100, 900, seed=7110 + append)
    assert int(((inp["lens"] + 31) // 32).sum()) * cfg.G > 8 * 256
    o, _ = run_decode(inp, cfg.scale, append=append)
    ref, _ = oracle_step(inp, cfg.scale, append=append)
    assert_parity(o, ref, torch.bfloat16, "b=150 long")


@pytest.mark.parametrize("m_cap", [64, SPLIT_M])
@pytest.mark.parametrize("append,fused", [(False, True), (True, True), (True, False)])
def test_decode_short_sequences_several_rounds(append, fused, m_cap):
    """More segments than 8 per workgroup of the largest grid (256): some
    workgroup ranges cross more than NW = 8 segments, so they are streamed
    and folded in several rounds of at most 8 pieces."""
    announce(f"decode b=4096 short m_cap={m_cap} append={append} fused={fused}")
    cfg, inp = make(torch.bfloat16, 4096, 8, 1, 64, m_cap, 1, 40, seed=7300 + append)
    assert cfg.b * cfg.G > 8 * 256
    o, _ = run_decode(inp, cfg.scale, append=append, fused=fused)
    ref, _ = oracle_step(inp, cfg.scale, append=append)
    assert_parity(o, ref, torch.bfloat16, "b=4096 short")


def test_decode_short_sequences_several_rounds_gqa_d128():
    """The same with G = 2 groups of 8 heads, d_h = 128 and fp32 inputs."""
    announce("decode b=1500 G=2 fp32 short")
    cfg, inp = make(torch.float32, 1500, 16, 2, 128, 48, 0, 47, seed=7310)
    assert cfg.b * cfg.G > 8 * 256
    o, _ = run_decode(inp, cfg.scale, append=True)
    ref, _ = oracle_step(inp, cfg.scale, append=True)
    assert_parity(o, ref, torch.float32, "b=1500 G=2 fp32 short")


@pytest.mark.parametrize("m_cap", [48, SPLIT_M])
@pytest.mark.parametrize("append,fused", [(False, True), (True, True), (True, False)])
def test_decode_more_than_64_lens_chunks(append, fused, m_cap):
    """b = 5000 (79 chunks of 64 sequences): the schedule's general chunk walk,
    which refills the lens lane cache chunk by chunk; short ragged lengths
    with empty sequences."""
    announce(f"decode b=5000 m_cap={m_cap} append={append} fused={fused}")
    cfg, inp = make(torch.bfloat16, 5000, 8, 1, 64, m_cap, 0, 40, seed=7320 + 2 * append + fused)
    assert (cfg.b + 63) // 64 > 64 and int((inp["lens"] == 0).sum()) > 0
    o, d = run_decode(inp, cfg.scale, append=append, fused=fused)
    ref, lens_ref = oracle_step(inp, cfg.scale, append=append)
    assert_parity(o, ref, torch.bfloat16, "b=5000")
    assert d["lens"].cpu().numpy().tolist() == lens_ref.tolist()


@pytest.mark.parametrize("m_cap", [100, SPLIT_M])
@pytest.mark.parametrize("b", [65, 1024, 1025])
@pytest.mark.parametrize("append", [False, True])
def test_decode_lens_layout_boundaries(b, append, m_cap):
    """Batch sizes at the edges of the schedule's lens layouts (one entry per
    lane up to 64, lane blocks of 16 up to 1024, chunks of 64 beyond), with
    empty rows mixed in and two groups."""
    announce(f"decode layout boundary b={b} m_cap={m_cap} append={append}")
    cfg, inp = make(torch.bfloat16, b, 8, 2, 64, m_cap, 0, 99, seed=7400 + b + append)
    lens = inp["lens"].clone()
    lens[::7] = 0  # rows with nothing visible (one visible row after an append)
    inp["lens"] = lens
    o, _ = run_decode(inp, cfg.scale, append=append)
    ref, _ = oracle_step(inp, cfg.scale, append=append)
    assert_parity(o, ref, torch.bfloat16, f"layout boundary b={b}")


@pytest.mark.parametrize("window", [1, 7, 32, 33, 5000])
def test_decode_local_window(window):
    """Local attention over the last `window` positions (current + 31 previous is 32)."""
    announce(f"decode window={window}")
    cfg, inp = make(torch.bfloat16, 6, 32, 1, 128, 700, 1, 700, seed=7200 + window)
    o, _ = run_decode(inp, cfg.scale, window=window, append=True)
    ref, _ = oracle_step(inp, cfg.scale, window=window, append=True)
    assert_parity(o, ref, torch.bfloat16, f"window {window}")


# ------------------------------------------------------------------ workloads


def test_c1_tiny_fp32():
    announce("c1 full size")
    inp = W.decode_inputs(W.C1)
    o, _ = run_decode(inp, W.C1.scale)
    ref, _ = oracle_step(inp, W.C1.scale)
    assert_parity(o, ref, torch.float32, "c1")


@pytest.mark.parametrize("cfg", [W.C2, W.C2_MHA], ids=lambda c: c.name)
def test_c2_full(cfg):
    announce(f"{cfg.name} full size")
    inp = W.decode_inputs(cfg)
    o, _ = run_decode(inp, cfg.scale)
    ref, _ = oracle_step(inp, cfg.scale)
    assert_parity(o, ref, torch.bfloat16, cfg.name)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "two-call"])
def test_c3_serving_full_with_append(fused):
    """b=64, h=32, ragged lens U{1..8192} + one append, exactly as timed."""
    announce(f"c3 full size (append + decode), fused={fused}")
    inp = W.decode_inputs(W.C3)
    o, d = run_decode(inp, W.C3.scale, append=True, fused=fused)
    ref, lens_ref = oracle_step(inp, W.C3.scale, append=True)
    assert np.array_equal(d["lens"].cpu().numpy(), lens_ref)
    assert_parity(o, ref, torch.bfloat16, "c3")
    Kr, _ = oracle._raw(inp["K"])
    Kr = Kr.copy()
    Vr, _ = oracle._raw(inp["V"])
    Vr = Vr.copy()
    oracle.kv_append(inp["k_new"], inp["v_new"], Kr, Vr, inp["lens"].numpy().copy())
    assert d["K"].cpu().view(torch.int16).numpy().view(np.uint16).tobytes() == Kr.tobytes()
    assert d["V"].cpu().view(torch.int16).numpy().view(np.uint16).tobytes() == Vr.tobytes()


def test_c4_gqa_full():
    """b=32, h=64, G=8, m=32768: the GPU runs the full step and the threaded
    fp64 oracle checks every sequence and head."""
    announce("c4 full size, all sequences")
    cfg = W.C4
    inp = W.decode_inputs(cfg)
    o, _ = run_decode(inp, cfg.scale)
    o = o.cpu()
    ref = oracle.decode(inp["q"], inp["K"], inp["V"], inp["lens"].numpy(), cfg.scale)
    assert_parity(o, ref, torch.bfloat16, "c4 all 32 sequences")


# ------------------------------------------------------------------ exact cases


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_single_position_returns_value_exactly(dtype):
    announce(f"L=1 exact {dtype}")
    cfg, inp = make(dtype, 4, 32, 4, 128, 50, 1, 1, seed=7300)
    inp["q"] = (inp["q"].float() * 30).to(dtype)
    o, _ = run_decode(inp, cfg.scale)
    V = inp["V"]
    exp = torch.stack([V[b, 0, torch.arange(32) // 8] for b in range(4)])
    assert torch.equal(o.cpu(), exp)


def test_append_then_decode_sees_only_the_new_token_when_empty():
    announce("empty cache + append")
    cfg, inp = make(torch.bfloat16, 3, 32, 1, 128, 40, 0, 0, seed=7310)
    o, d = run_decode(inp, cfg.scale, append=True)
    exp = inp["v_new"][:, 0:1, :].expand(3, 32, 128)
    assert torch.equal(o.cpu(), exp)
    assert d["lens"].cpu().tolist() == [1, 1, 1]


def test_empty_rows_are_zero_and_lens_clamped():
    announce("L=0 rows and lens > m_cap")
    cfg, inp = make(torch.bfloat16, 4, 32, 1, 128, 70, 0, 0, seed=7320)
    inp["lens"] = torch.tensor([0, 70, -3, 500], dtype=torch.int32)
    o, _ = run_decode(inp, cfg.scale)
    ref, _ = oracle_step(inp, cfg.scale)
    assert torch.equal(o[0].cpu(), torch.zeros(32, 128, dtype=torch.bfloat16))
    assert torch.equal(o[2].cpu(), torch.zeros(32, 128, dtype=torch.bfloat16))
    assert_parity(o, ref, torch.bfloat16, "clamp")


def test_zero_scale_gives_mean_and_constant_v():
    announce("scale=0 mean; constant V")
    cfg, inp = make(torch.bfloat16, 3, 32, 1, 128, 500, 100, 500, seed=7330)
    o, _ = run_decode(inp, 0.0)
    ref, _ = oracle_step(inp, 0.0)
    assert_parity(o, ref, torch.bfloat16, "scale 0")
    inp["V"] = torch.full_like(inp["V"], 0.375)
    o, _ = run_decode(inp, cfg.scale)
    assert (o.float().cpu() - 0.375).abs().max().item() <= 2e-3


def test_large_logits_stay_finite():
    """q x 20: logits with std ~ 20 overflow fp32 exp without the running max."""
    announce("q x 20 stress")
    cfg, inp = make(torch.bfloat16, 4, 32, 1, 128, 2000, 1000, 2000, seed=7340)
    inp["q"] = (inp["q"].float() * 20).to(torch.bfloat16)
    o, _ = run_decode(inp, cfg.scale)
    ref, _ = oracle_step(inp, cfg.scale)
    assert_parity(o, ref, torch.bfloat16, "q x 20")


def test_negative_scale():
    announce("negative scale")
    cfg, inp = make(torch.bfloat16, 2, 32, 2, 64, 300, 200, 300, seed=7350)
    o, _ = run_decode(inp, -0.3)
    ref, _ = oracle_step(inp, -0.3)
    assert_parity(o, ref, torch.bfloat16, "scale -0.3")


# ------------------------------------------------------------------ invariants


def test_poison_beyond_lens_and_determinism():
    announce("poison + determinism")
    cfg, inp = make(torch.bfloat16, 8, 32, 1, 128, 1000, 1, 999, seed=7400)
    o1, _ = run_decode(inp, cfg.scale)
    o2, _ = run_decode(inp, cfg.scale)
    assert torch.equal(o1, o2)
    poisoned = dict(inp)
    poisoned["K"] = W.poison_beyond(inp["K"], inp["lens"])
    poisoned["V"] = W.poison_beyond(inp["V"], inp["lens"])
    o3, _ = run_decode(poisoned, cfg.scale)
    assert torch.isfinite(o3.float()).all()
    assert torch.equal(o1, o3)


def test_mqa_equals_tied_mha_on_gpu():
    announce("MQA == tied MHA")
    cfg, inp = make(torch.bfloat16, 3, 8, 1, 128, 400, 100, 400, seed=7410)
    o1, _ = run_decode(inp, cfg.scale)
    tied = dict(inp)
    tied["K"] = inp["K"].expand(3, 400, 8, 128).contiguous()
    tied["V"] = inp["V"].expand(3, 400, 8, 128).contiguous()
    o2, _ = run_decode(tied, cfg.scale)
    ref, _ = oracle_step(inp, cfg.scale)
    assert_parity(o1, ref, torch.bfloat16, "mqa")
    assert_parity(o2, ref, torch.bfloat16, "tied mha")


def test_permuted_cache_positions_give_the_same_output():
    """P10 on the GPU: the core has no positional term, so permuting the
    visible positions of every sequence (K and V together) changes only the
    summation order."""
    announce("position permutation invariance")
    cfg, inp = make(torch.bfloat16, 4, 32, 1, 128, 600, 40, 600, seed=7415)
    o1, _ = run_decode(inp, cfg.scale)
    g = torch.Generator().manual_seed(7416)
    perm = dict(inp)
    perm["K"], perm["V"] = inp["K"].clone(), inp["V"].clone()
    for bi, L in enumerate(inp["lens"].tolist()):
        p = torch.randperm(L, generator=g)
        perm["K"][bi, :L] = inp["K"][bi, p]
        perm["V"][bi, :L] = inp["V"][bi, p]
    o2, _ = run_decode(perm, cfg.scale)
    ref, _ = oracle_step(inp, cfg.scale)
    assert_parity(o1, ref, torch.bfloat16, "original order")
    assert_parity(o2, ref, torch.bfloat16, "permuted positions")


def test_gqa_endpoints_equal_per_head_mqa():
    """P7 on the GPU: with G = h every head has its own K/V head (the MHA
    route); it must equal h single-head MQA decodes over that head's K/V."""
    announce("G = h vs per-head G = 1")
    cfg, inp = make(torch.bfloat16, 3, 8, 8, 64, 300, 50, 300, seed=7417)
    o_all, _ = run_decode(inp, cfg.scale)
    for i in range(cfg.h):
        one = {"q": inp["q"][:, i:i + 1].contiguous(),
               "K": inp["K"][:, :, i:i + 1].contiguous(),
               "V": inp["V"][:, :, i:i + 1].contiguous(),
               "lens": inp["lens"]}
        o_i, _ = run_decode(one, cfg.scale)
        ref, _ = oracle_step(one, cfg.scale)
        assert_parity(o_i, ref, torch.bfloat16, f"head {i} as MQA")
        assert_parity(o_all[:, i:i + 1], ref, torch.bfloat16, f"head {i} within G = h")


def test_append_is_bit_exact_and_flags_full_caches():
    announce("append bit-exact")
    cfg, inp = make(torch.bfloat16, 5, 32, 2, 128, 64, 0, 64, seed=7420)
    inp["lens"] = torch.tensor([0, 63, 64, 10, 70], dtype=torch.int32)
    d = to_dev(inp)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    mqa.kv_append(d["k_new"], d["v_new"], d["K"], d["V"], d["lens"], err_flag=err)
    torch.cuda.synchronize()
    Kr, _ = oracle._raw(inp["K"])
    Vr, _ = oracle._raw(inp["V"])
    Kr, Vr = Kr.copy(), Vr.copy()
    lens = inp["lens"].numpy().copy()
    over = oracle.kv_append(inp["k_new"], inp["v_new"], Kr, Vr, lens)
    assert over == 2 and err.item() == 1
    assert np.array_equal(d["lens"].cpu().numpy(), lens)
    gk = d["K"].cpu().view(torch.int16).numpy().view(np.uint16)
    gv = d["V"].cpu().view(torch.int16).numpy().view(np.uint16)
    assert gk.tobytes() == Kr.tobytes() and gv.tobytes() == Vr.tobytes()
    with pytest.raises(mqa.MQAError) as e:
        mqa.check_lens(d["lens"], 64)                # lens[4] = 70 stays beyond m_cap
    assert e.value.status == -8
    mqa.check_lens(d["lens"][:4].contiguous(), 64)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "two-call"])
def test_serial_decode_loop_matches_oracle(fused):
    """Ten append+decode steps with a growing cache (the serial token loop),
    one workspace reused by every step."""
    announce(f"10-step loop fused={fused}")
    cfg, inp = make(torch.bfloat16, 4, 32, 1, 128, 300, 20, 250, seed=7430)
    d = to_dev(inp)
    Kr, _ = oracle._raw(inp["K"])
    Vr, _ = oracle._raw(inp["V"])
    Kr, Vr = Kr.copy(), Vr.copy()
    lens = inp["lens"].numpy().copy()
    g = torch.Generator().manual_seed(99)
    ws = mqa.workspace_for(32, d["K"])
    for step in range(10):
        kn = torch.randn(4, 1, 128, generator=g).to(torch.bfloat16)
        vn = torch.randn(4, 1, 128, generator=g).to(torch.bfloat16)
        q = torch.randn(4, 32, 128, generator=g).to(torch.bfloat16)
        if fused:
            o = mqa.append_decode(q.cuda(), kn.cuda(), vn.cuda(), d["K"], d["V"], d["lens"],
                                  cfg.scale, workspace=ws)
        else:
            mqa.kv_append(kn.cuda(), vn.cuda(), d["K"], d["V"], d["lens"])
            o = mqa.decode(q.cuda(), d["K"], d["V"], d["lens"], cfg.scale, workspace=ws)
        oracle.kv_append(kn, vn, Kr, Vr, lens)
        ref = oracle.decode(q, Kr, Vr, lens, cfg.scale)
        assert_parity(o, ref, torch.bfloat16, f"loop step {step}")


def test_fused_append_full_caches_flag_and_keep_lens():
    """Full caches get no new row in the fused path either: lens stays, the
    flag is set, the sequence attends over its m_cap rows."""
    announce("fused append with full caches")
    cfg, inp = make(torch.bfloat16, 5, 32, 2, 128, 64, 0, 64, seed=7440)
    inp["lens"] = torch.tensor([0, 63, 64, 10, 70], dtype=torch.int32)
    d = to_dev(inp)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = mqa.append_decode(d["q"], d["k_new"], d["v_new"], d["K"], d["V"], d["lens"], cfg.scale,
                          err_flag=err)
    torch.cuda.synchronize()
    ref, lens_ref = oracle_step(inp, cfg.scale, append=True)
    assert err.item() == 1
    assert d["lens"].cpu().tolist() == lens_ref.tolist() == [1, 64, 64, 11, 70]
    assert_parity(o, ref, torch.bfloat16, "fused full caches")


def test_decode_workspace_reused_across_shapes_of_lens():
    """One workspace across calls whose lens mixes alternate between split
    and unsplit segments: nothing stale leaks from one call to the next."""
    announce("workspace reuse")
    cfg, inp = make(torch.bfloat16, 4, 32, 1, 128, 3000, 1, 3000, seed=7450)
    d = to_dev(inp)
    ws = mqa.workspace_for(32, d["K"])
    g = torch.Generator().manual_seed(3)
    for it in range(6):
        lens = torch.randint(0, 3001 if it % 2 else 40, (4,), generator=g).to(torch.int32)
        o = mqa.decode(d["q"], d["K"], d["V"], lens.cuda(), cfg.scale, workspace=ws)
        ref = oracle.decode(inp["q"], inp["K"], inp["V"], lens.numpy(), cfg.scale)
        assert_parity(o, ref, torch.bfloat16, f"reuse {it}")


# ------------------------------------------------------------------ errors


def test_argument_errors_raise():
    announce("argument errors")
    K = torch.zeros(2, 64, 2, 128, dtype=torch.bfloat16, device="cuda")
    lens = torch.ones(2, dtype=torch.int32, device="cuda")
    q = torch.zeros(2, 6, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mqa.MQAError) as e:
        mqa.decode(torch.zeros(2, 5, 128, dtype=torch.bfloat16, device="cuda"), K, K, lens, 1.0)
    assert e.value.status == -2                      # G does not divide h
    with pytest.raises(mqa.MQAError) as e:
        mqa.decode(q, K, K, lens, 1.0, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == -5                      # workspace too small
    Kb = torch.zeros(2, 64, 1, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mqa.MQAError) as e:
        mqa.decode(torch.zeros(2, 64, 128, dtype=torch.bfloat16, device="cuda"), Kb, Kb, lens, 1.0)
    assert e.value.status == -2                      # h/G = 64 > 32
    K96 = torch.zeros(2, 64, 1, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mqa.MQAError) as e:
        mqa.decode(torch.zeros(2, 4, 96, dtype=torch.bfloat16, device="cuda"), K96, K96, lens, 1.0)
    assert e.value.status == -3                      # d_h = 96
