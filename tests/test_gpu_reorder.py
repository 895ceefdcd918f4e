"""GPU parity of the beam reorder (bit-exact against the oracle, whole cache
and lens) and of beam steps (reorder, then fused append + decode) against the
fp64 oracle, on the same seeded inputs, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import announce, assert_parity
from query_decode_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import query_decode_attention_amd as mqa


def raw(t):
    a, _ = oracle._raw(t)
    return a.copy()


def check_reorder(K, V, lens, parent, beam, what):
    """Reorder on the GPU and in the oracle; the whole cache must agree
    byte for byte (moved rows and untouched ones), lens exactly."""
    announce(what)
    dK, dV, dl, dp = K.cuda(), V.cuda(), lens.cuda(), parent.cuda()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    mqa.kv_reorder(dK, dV, dl, dp, beam, err_flag=flag)
    torch.cuda.synchronize()
    Kr, Vr, lr = raw(K), raw(V), lens.numpy().copy()
    bad = oracle.kv_reorder(Kr, Vr, lr, parent.numpy(), beam)
    assert np.array_equal(dl.cpu().numpy(), lr), what
    gK, gV = raw(dK.cpu()), raw(dV.cpu())
    rows_k = [i for i in range(K.shape[0]) if gK[i].tobytes() != Kr[i].tobytes()]
    rows_v = [i for i in range(K.shape[0]) if gV[i].tobytes() != Vr[i].tobytes()]
    assert not rows_k and not rows_v, f"{what}: rows differ K {rows_k} V {rows_v}"
    assert int(flag.item()) == (1 if bad else 0), what


def cache(dtype, b, m_cap, G, dh, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    K = torch.randn(b, m_cap, G, dh, generator=g).to(dtype)
    V = torch.randn(b, m_cap, G, dh, generator=g).to(dtype)
    return K, V, g


GRID = [
    # dtype, b, beam, G, dh, m_cap
    (torch.bfloat16, 8, 4, 1, 128, 70),
    (torch.bfloat16, 12, 3, 2, 64, 129),
    (torch.float32, 8, 4, 1, 64, 33),
    (torch.float32, 16, 8, 2, 128, 65),
    (torch.bfloat16, 32, 16, 1, 128, 40),
    (torch.bfloat16, 6, 1, 1, 64, 17),
    (torch.bfloat16, 10, 2, 8, 128, 9),
]


@pytest.mark.parametrize("dtype,b,beam,G,dh,m_cap", GRID)
def test_reorder_grid_bit_exact(dtype, b, beam, G, dh, m_cap):
    K, V, g = cache(dtype, b, m_cap, G, dh, 300 + b + m_cap)
    lens = torch.randint(0, m_cap + 1, (b,), generator=g, dtype=torch.int32)
    lens[0] = m_cap
    parent = torch.randint(0, beam, (b,), generator=g, dtype=torch.int32)
    check_reorder(K, V, lens, parent, beam, f"reorder {dtype} b={b} beam={beam} G={G} "
                                            f"dh={dh} m_cap={m_cap}")


@pytest.mark.parametrize("pattern", ["identity", "all_first", "swap", "rotate", "reverse"])
def test_reorder_in_place_patterns(pattern):
    """Permutations whose sources are themselves overwritten in the same call."""
    b, beam, m_cap = 16, 4, 100
    K, V, g = cache(torch.bfloat16, b, m_cap, 1, 128, 320)
    lens = torch.randint(1, m_cap + 1, (b,), generator=g, dtype=torch.int32)
    i = torch.arange(b) % beam
    parent = {"identity": i, "all_first": torch.zeros(b, dtype=torch.int64),
              "swap": i ^ 1, "rotate": (i + 1) % beam, "reverse": beam - 1 - i}[pattern]
    check_reorder(K, V, lens, parent.to(torch.int32), beam, f"reorder pattern {pattern}")


def test_reorder_out_of_range_lens_and_bad_parents():
    b, beam, m_cap = 8, 4, 50
    K, V, g = cache(torch.bfloat16, b, m_cap, 2, 64, 330)
    lens = torch.tensor([-3, 60, 0, 50, 7, 13, 50, 1], dtype=torch.int32)
    parent = torch.tensor([1, 0, 3, 2, 2, 9, -1, 0], dtype=torch.int32)   # rows 5, 6 bad
    check_reorder(K, V, lens, parent, beam, "reorder lens clamp + bad parents")


def test_reorder_full_beam4_shape():
    cfg = W.BEAM4
    inp = W.beam_inputs(cfg, steps=1)
    check_reorder(inp["K"], inp["V"], inp["lens"], inp["parent"][0], cfg.beam,
                  f"reorder {cfg.name}")


def run_beam_steps(cfg, inp, steps):
    """GPU: per step reorder, then fused append + decode.  Oracle: reorder,
    append, decode.  Returns after comparing every step's output and the
    final cache and lens."""
    d = {k: v.cuda() for k, v in inp.items()}
    Kr, Vr, lr = raw(inp["K"]), raw(inp["V"]), inp["lens"].numpy().copy()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for s in range(steps):
        announce(f"beam step {s} of {cfg.name}")
        mqa.kv_reorder(d["K"], d["V"], d["lens"], d["parent"][s].contiguous(), cfg.beam,
                       err_flag=flag)
        o = mqa.append_decode(d["q"][s].contiguous(), d["k_new"][s].contiguous(),
                              d["v_new"][s].contiguous(), d["K"], d["V"], d["lens"], cfg.scale,
                              err_flag=flag)
        torch.cuda.synchronize()
        oracle.kv_reorder(Kr, Vr, lr, inp["parent"][s].numpy(), cfg.beam)
        oracle.kv_append(inp["k_new"][s], inp["v_new"][s], Kr, Vr, lr)
        ref = oracle.decode(inp["q"][s], Kr, Vr, lr, cfg.scale)
        assert_parity(o, ref, cfg.dtype, f"{cfg.name} step {s}")
    assert int(flag.item()) == 0
    assert np.array_equal(d["lens"].cpu().numpy(), lr)
    assert raw(d["K"].cpu()).tobytes() == Kr.tobytes()
    assert raw(d["V"].cpu()).tobytes() == Vr.tobytes()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_beam_steps_small(dtype):
    cfg = W.BeamConfig("beam_small", dtype, sources=3, beam=4, h=8, G=2, dh=64, m_cap=200,
                       lens_lo=1, lens_hi=150, seed=340)
    run_beam_steps(cfg, W.beam_inputs(cfg, steps=4), 4)


def test_beam_steps_full_beam4():
    cfg = W.BEAM4
    run_beam_steps(cfg, W.beam_inputs(cfg, steps=2), 2)


@pytest.mark.parametrize("dtype,b,beam,G,dh,m_cap", GRID[:5])
def test_reorder_to_equals_in_place(dtype, b, beam, G, dh, m_cap):
    """Out-of-place lengths: the same cache bytes as the in-place reorder,
    lens_out equal to the in-place lens, lens_in untouched, the same flag."""
    what = f"reorder_to {dtype} b={b} beam={beam} G={G} dh={dh} m_cap={m_cap}"
    announce(what)
    K, V, g = cache(dtype, b, m_cap, G, dh, 350 + b + m_cap)
    lens = torch.randint(0, m_cap + 1, (b,), generator=g, dtype=torch.int32)
    parent = torch.randint(0, beam, (b,), generator=g, dtype=torch.int32)
    parent[b - 1] = beam + 2                                   # one bad parent
    runs = []
    for out_of_place in (False, True):
        dK, dV, dl, dp = K.cuda(), V.cuda(), lens.cuda(), parent.cuda()
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        lo = torch.full((b,), -7, dtype=torch.int32, device="cuda") if out_of_place else None
        mqa.kv_reorder(dK, dV, dl, dp, beam, err_flag=flag, lens_out=lo)
        torch.cuda.synchronize()
        runs.append((raw(dK.cpu()), raw(dV.cpu()), dl.cpu(), None if lo is None else lo.cpu(),
                     int(flag.item())))
    (k0, v0, l0, _, f0), (k1, v1, lin, lout, f1) = runs
    assert k0.tobytes() == k1.tobytes() and v0.tobytes() == v1.tobytes(), what
    assert torch.equal(lout, l0), what
    assert torch.equal(lin, lens), what
    assert f0 == f1 == 1, what


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_beam_steps_ping_pong_lens(dtype):
    """Beam steps with the lengths alternating between two arrays
    (reorder_to, then fused append + decode on the new one) against the
    oracle's reorder, append and decode."""
    cfg = W.BeamConfig("beam_pp", dtype, sources=3, beam=4, h=8, G=2, dh=64, m_cap=200,
                       lens_lo=1, lens_hi=150, seed=360)
    steps = 4
    inp = W.beam_inputs(cfg, steps=steps)
    d = {k: v.cuda() for k, v in inp.items()}
    lens = [d["lens"], torch.empty_like(d["lens"])]
    Kr, Vr, lr = raw(inp["K"]), raw(inp["V"]), inp["lens"].numpy().copy()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for s in range(steps):
        announce(f"ping-pong beam step {s}")
        src, dst = lens[s % 2], lens[1 - s % 2]
        mqa.kv_reorder(d["K"], d["V"], src, d["parent"][s].contiguous(), cfg.beam, err_flag=flag,
                       lens_out=dst)
        o = mqa.append_decode(d["q"][s].contiguous(), d["k_new"][s].contiguous(),
                              d["v_new"][s].contiguous(), d["K"], d["V"], dst, cfg.scale,
                              err_flag=flag)
        torch.cuda.synchronize()
        oracle.kv_reorder(Kr, Vr, lr, inp["parent"][s].numpy(), cfg.beam)
        oracle.kv_append(inp["k_new"][s], inp["v_new"][s], Kr, Vr, lr)
        ref = oracle.decode(inp["q"][s], Kr, Vr, lr, cfg.scale)
        assert_parity(o, ref, cfg.dtype, f"{cfg.name} step {s}")
        assert np.array_equal(dst.cpu().numpy(), lr)
    assert int(flag.item()) == 0
    assert raw(d["K"].cpu()).tobytes() == Kr.tobytes()
    assert raw(d["V"].cpu()).tobytes() == Vr.tobytes()


def _reorder_sweep_cases(n_cases, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        beam = int(rng.choice([1, 2, 3, 4, 4, 5, 8, 12, 16]))
        groups = int(rng.integers(1, 9))
        G = int(rng.choice([1, 1, 2, 4, 8]))
        dh = int(rng.choice([64, 128]))
        m_cap = int(rng.choice([1, 5, 31, 32, 33, 100, 257]))
        out_of_place = bool(rng.random() < 0.5)
        cases.append((i, dtype, groups * beam, beam, G, dh, m_cap, out_of_place,
                      int(rng.integers(1, 1 << 30))))
    return cases


REORDER_SWEEP = _reorder_sweep_cases(32, 20261206)


@pytest.mark.parametrize("case", REORDER_SWEEP,
                         ids=lambda c: f"{c[0]:02d}-{c[1]}-b{c[2]}beam{c[3]}G{c[4]}d{c[5]}m{c[6]}"
                                       + ("-to" if c[7] else ""))
def test_reorder_sweep_bit_exact(case):
    """Seeded random reorders: beam widths 1..16, groups, head sizes and
    capacities, lengths drawn past both ends of [0, m_cap], a few bad
    parents; in place or with the lengths written to a second array.  The
    whole cache must equal the oracle's byte for byte, the lengths exactly."""
    i, dt, b, beam, G, dh, m_cap, out_of_place, seed = case
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    what = f"reorder sweep {case}"
    announce(what)
    K, V, g = cache(dtype, b, m_cap, G, dh, seed)
    lens = torch.randint(-2, m_cap + 4, (b,), generator=g, dtype=torch.int32)
    parent = torch.randint(0, beam, (b,), generator=g, dtype=torch.int32)
    bad = torch.rand(b, generator=g) < 0.05
    parent[bad] = beam + 1
    dK, dV, dl, dp = K.cuda(), V.cuda(), lens.cuda(), parent.cuda()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    lo = torch.full((b,), -7, dtype=torch.int32, device="cuda") if out_of_place else None
    mqa.kv_reorder(dK, dV, dl, dp, beam, err_flag=flag, lens_out=lo)
    torch.cuda.synchronize()
    Kr, Vr, lr = raw(K), raw(V), lens.numpy().copy()
    oracle_bad = oracle.kv_reorder(Kr, Vr, lr, parent.numpy(), beam)
    got_lens = (lo if out_of_place else dl).cpu().numpy()
    assert np.array_equal(got_lens, lr), what
    if out_of_place:
        assert torch.equal(dl.cpu(), lens), what + ": lens_in changed"
    assert raw(dK.cpu()).tobytes() == Kr.tobytes(), what + ": K"
    assert raw(dV.cpu()).tobytes() == Vr.tobytes(), what + ": V"
    assert int(flag.item()) == (1 if oracle_bad else 0), what + ": flag"
