"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

None of these compare the oracle with a retyping of itself: each check uses a
closed form, an exact special case, an identity between two different routes,
or the independent pure-Python implementation in ``bruteforce.py``.  Chosen so
that a dropped scale, a wrong head->group index, a transposed operand, a
missing max-shift, an off-by-one in lens or a reversed causal mask fails one.
"""
import math

import numpy as np
import pytest
import torch

import bruteforce
import oracle
from query_decode_attention_amd import workloads


def f64(t):
    return t.double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def rand(shape, seed, dtype=torch.float32, mul=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(*shape, generator=g) * mul).to(dtype)


# ---------------------------------------------------------------- P1, P2


@pytest.mark.parametrize("pad", [0, 62])
def test_worked_example_closed_form(golden, pad):
    """Study notes section 4: two heads, one shared K, opposite preferences."""
    ex = golden("worked_example_shared_k.txt")
    dh = ex["d_h"] + pad
    K = np.zeros((1, 2, 1, dh), np.float32)
    K[0, 0, 0, :2] = ex["k1"]
    K[0, 1, 0, :2] = ex["k2"]
    V = np.zeros_like(K)          # V = identity rows, so o_i equals the weights
    V[0, 0, 0, 0] = 1.0
    V[0, 1, 0, 1] = 1.0
    q = np.zeros((1, 2, dh), np.float32)
    q[0, 0, :2] = ex["q1"]
    q[0, 1, :2] = ex["q2"]
    lens = np.array([2], np.int32)
    for scale in ex["scales"]:
        o = oracle.decode(q, K, V, lens, scale)
        fav = 1.0 / (1.0 + math.exp(-3.0 * scale))
        assert o[0, 0, ex["favoured_head1"]] == pytest.approx(fav, abs=1e-15)
        assert o[0, 0, 1 - ex["favoured_head1"]] == pytest.approx(1 - fav, abs=1e-15)
        assert o[0, 1, ex["favoured_head2"]] == pytest.approx(fav, abs=1e-15)
        assert o[0, 1, 1 - ex["favoured_head2"]] == pytest.approx(1 - fav, abs=1e-15)
        w = oracle.decode_weights(q, K, V, lens, scale, 0, 0)
        assert w[0] == pytest.approx(fav, abs=1e-15)
    # the two readings of the scale give different numbers (0.8930 vs 0.9526)
    assert abs(1 / (1 + math.exp(-3 / math.sqrt(2))) - 1 / (1 + math.exp(-3))) > 0.05


def test_shape_example(golden):
    """Study notes section 2: L_q=4, L_k=6, d_h=128 -> scores [4,6], output [4,128]."""
    ex = golden("shape_example.txt")
    Lq, Lk, dh = ex["L_q"], ex["L_k"], ex["d_h"]
    q = rand((1, Lq, dh), 1)                         # 4 queries sharing one K/V
    K = rand((1, Lk + 3, 1, dh), 2)                  # capacity > L_k
    V = rand((1, Lk + 3, 1, dh), 3)
    lens = np.array([Lk], np.int32)
    o = oracle.decode(q, K, V, lens, 1 / math.sqrt(dh))
    assert list(o.shape[1:]) == ex["output_shape"]
    scores = [oracle.decode_weights(q, K, V, lens, 1 / math.sqrt(dh), 0, i) for i in range(Lq)]
    assert [len(scores), len(scores[0])] == ex["scores_shape"]


# ---------------------------------------------------------------- P3 .. P5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_single_key_returns_value_exactly(dtype):
    q = rand((2, 8, 64), 10, dtype, mul=50.0)
    K = rand((2, 5, 2, 64), 11, dtype)
    V = rand((2, 5, 2, 64), 12, dtype)
    lens = np.array([1, 1], np.int32)
    o = oracle.decode(q, K, V, lens, 0.125)
    for b in range(2):
        for i in range(8):
            assert np.array_equal(o[b, i], f64(V[b, 0, i // 4]))


def test_constant_value_and_unit_weight_sum():
    q = rand((3, 4, 64), 20, mul=5.0)
    K = rand((3, 40, 1, 64), 21)
    V = torch.full((3, 40, 1, 64), 0.75)
    lens = np.array([40, 17, 3], np.int32)
    o = oracle.decode(q, K, V, lens, 0.125)
    assert np.allclose(o, 0.75, rtol=0, atol=1e-14)
    for b in range(3):
        for i in range(4):
            w = oracle.decode_weights(q, K, V, lens, 0.125, b, i)
            assert len(w) == lens[b]
            assert math.fsum(w) == pytest.approx(1.0, abs=1e-14)
            assert (w > 0).all()


def test_zero_scale_is_mean_of_values():
    q = rand((2, 4, 64), 30, mul=10.0)
    K = rand((2, 33, 1, 64), 31)
    V = rand((2, 33, 1, 64), 32)
    lens = np.array([33, 9], np.int32)
    o = oracle.decode(q, K, V, lens, 0.0)
    Vd = f64(V)
    for b in range(2):
        mean = np.array([math.fsum(Vd[b, :lens[b], 0, d]) / lens[b] for d in range(64)])
        for i in range(4):
            assert np.allclose(o[b, i], mean, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P6, P7


def test_mqa_equals_mha_with_tied_kv():
    """MQA is MHA whose h K/V heads are all the same (study notes section 4 table)."""
    h = 8
    q = rand((2, h, 64), 40)
    K1 = rand((2, 20, 1, 64), 41)
    V1 = rand((2, 20, 1, 64), 42)
    lens = np.array([20, 13], np.int32)
    o_mqa = oracle.decode(q, K1, V1, lens, 0.125)
    o_mha = oracle.decode(q, K1.expand(2, 20, h, 64).contiguous(),
                          V1.expand(2, 20, h, 64).contiguous(), lens, 0.125)
    assert np.allclose(o_mqa, o_mha, rtol=0, atol=1e-15)


@pytest.mark.parametrize("G", [1, 2, 4])
def test_gqa_grouping_against_bruteforce(G):
    """GQA essay section 3: G=1 is MQA, G=h is MHA; head i reads group i // (h/G)."""
    h = 4
    q = rand((2, h, 8), 50 + G)
    K = rand((2, 7, G, 8), 60 + G)
    V = rand((2, 7, G, 8), 70 + G)
    lens = np.array([7, 4], np.int32)
    o = oracle.decode(q, K, V, lens, 0.35)
    ref = bruteforce.decode(f64(q), f64(K), f64(V), lens, 0.35)
    assert np.allclose(o, ref, rtol=0, atol=1e-13)
    if G == h:   # MHA route: head i with its own K_i, V_i
        for i in range(h):
            per_head = bruteforce.decode(f64(q)[:, i:i + 1], f64(K)[:, :, i:i + 1],
                                         f64(V)[:, :, i:i + 1], lens, 0.35)
            assert np.allclose(o[:, i:i + 1], per_head, rtol=0, atol=1e-13)
    if G == 2:   # contiguous grouping, not interleaved: heads 0,1 -> group 0
        Ksw = K.flip(2).contiguous()
        Vsw = V.flip(2).contiguous()
        o_sw = oracle.decode(q, Ksw, Vsw, lens, 0.35)
        assert not np.allclose(o_sw, o)


# ---------------------------------------------------------------- P8


@pytest.mark.parametrize("G", [1, 2])
def test_prefill_row_equals_decode_with_prefix_cache(G):
    """One formula for prefill and decode (study notes section 1): prefill row t
    over the full masked row equals a decode step whose cache holds t+1 rows."""
    b, n, h, dh = 2, 23, 4, 64
    Q = rand((b, n, h, dh), 80, torch.bfloat16)
    K = rand((b, n, G, dh), 81, torch.bfloat16)
    V = rand((b, n, G, dh), 82, torch.bfloat16)
    O = oracle.prefill(Q, K, V, 0.125)
    for t in range(n):
        lens = np.full(b, t + 1, np.int32)
        o = oracle.decode(Q[:, t].contiguous(), K, V, lens, 0.125)
        assert np.allclose(O[:, t], o, rtol=0, atol=1e-14)


def test_prefill_first_row_and_causality():
    b, n, h, dh = 1, 9, 2, 64
    Q = rand((b, n, h, dh), 90)
    K = rand((b, n, 1, dh), 91)
    V = rand((b, n, 1, dh), 92)
    O = oracle.prefill(Q, K, V, 0.3)
    for i in range(h):
        assert np.array_equal(O[0, 0, i], f64(V[0, 0, 0]))      # row 0 sees only key 0
    K2, V2 = K.clone(), V.clone()
    K2[0, 5:] = 7.0
    V2[0, 5:] = -3.0
    O2 = oracle.prefill(Q, K2, V2, 0.3)
    assert np.array_equal(O[0, :5], O2[0, :5])                   # future keys are invisible
    assert not np.allclose(O[0, 5:], O2[0, 5:])
    ref = bruteforce.prefill(f64(Q), f64(K), f64(V), 0.3)
    assert np.allclose(O, ref, rtol=0, atol=1e-13)


def test_prefill_row_sample_matches_full():
    b, n, h, dh = 2, 12, 4, 64
    Q = rand((b, n, h, dh), 95, torch.bfloat16)
    K = rand((b, n, 2, dh), 96, torch.bfloat16)
    V = rand((b, n, 2, dh), 97, torch.bfloat16)
    full = oracle.prefill(Q, K, V, 0.125)
    rows = [0, 5, 11, 12, 23]
    part = oracle.prefill(Q, K, V, 0.125, rows=rows)
    for k, r in enumerate(rows):
        assert np.array_equal(part[k], full[r // n, r % n])


# ---------------------------------------------------------------- P9


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bruteforce_tiny(seed, dtype):
    g = torch.Generator("cpu").manual_seed(500 + seed)
    b = 1 + seed % 2
    G = [1, 2][seed % 2]
    h = G * (1 + seed % 3)
    dh = [4, 8, 6][seed % 3]
    m = 16
    q = torch.randn(b, h, dh, generator=g).to(dtype)
    K = torch.randn(b, m, G, dh, generator=g).to(dtype)
    V = torch.randn(b, m, G, dh, generator=g).to(dtype)
    lens = torch.randint(1, m + 1, (b,), generator=g).to(torch.int32).numpy()
    scale = 1 / math.sqrt(dh)
    o = oracle.decode(q, K, V, lens, scale)
    ref = bruteforce.decode(f64(q), f64(K), f64(V), lens, scale)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P10


def test_permutation_invariance_over_positions():
    q = rand((1, 4, 64), 100)
    K = rand((1, 30, 1, 64), 101)
    V = rand((1, 30, 1, 64), 102)
    lens = np.array([30], np.int32)
    perm = torch.randperm(30, generator=torch.Generator().manual_seed(3))
    o = oracle.decode(q, K, V, lens, 0.125)
    op = oracle.decode(q, K[:, perm].contiguous(), V[:, perm].contiguous(), lens, 0.125)
    assert np.allclose(o, op, rtol=0, atol=1e-14)


def test_linearity_in_values():
    g = torch.Generator().manual_seed(7)
    q = rand((2, 4, 64), 110)
    K = rand((2, 25, 1, 64), 111)
    V1 = torch.randint(-8, 9, (2, 25, 1, 64), generator=g).float()
    V2 = torch.randint(-8, 9, (2, 25, 1, 64), generator=g).float()
    lens = np.array([25, 11], np.int32)
    o1 = oracle.decode(q, K, V1, lens, 0.125)
    o2 = oracle.decode(q, K, V2, lens, 0.125)
    o3 = oracle.decode(q, K, 3 * V1 - V2, lens, 0.125)       # exact in fp32
    assert np.allclose(o3, 3 * o1 - o2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_poison_beyond_lens_is_never_read(dtype):
    q = rand((3, 8, 64), 120, dtype)
    K = rand((3, 40, 2, 64), 121, dtype)
    V = rand((3, 40, 2, 64), 122, dtype)
    lens = torch.tensor([40, 1, 17], dtype=torch.int32)
    o = oracle.decode(q, K, V, lens.numpy(), 0.125)
    Kp = workloads.poison_beyond(K, lens)
    Vp = workloads.poison_beyond(V, lens)
    assert torch.isnan(Kp.float()).any() and torch.isinf(Vp.float()).any()
    op = oracle.decode(q, Kp, Vp, lens.numpy(), 0.125)
    assert np.array_equal(o, op)


def test_empty_row_and_lens_clamp():
    q = rand((3, 4, 64), 130)
    K = rand((3, 10, 1, 64), 131)
    V = rand((3, 10, 1, 64), 132)
    o = oracle.decode(q, K, V, np.array([0, -5, 99], np.int32), 0.125)
    assert np.array_equal(o[0], np.zeros((4, 64))) and np.array_equal(o[1], np.zeros((4, 64)))
    o_full = oracle.decode(q, K, V, np.array([10, 10, 10], np.int32), 0.125)
    assert np.array_equal(o[2], o_full[2])                   # lens > m_cap reads m_cap rows


# ---------------------------------------------------------------- P11


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_append_is_a_bytewise_concat(dtype):
    b, m, G, dh = 4, 6, 2, 64
    K = rand((b, m, G, dh), 140, dtype)
    V = rand((b, m, G, dh), 141, dtype)
    kn = rand((b, G, dh), 142, dtype)
    vn = rand((b, G, dh), 143, dtype)
    lens = np.array([0, 3, 5, 6], np.int32)                   # last one is full
    Kr, _ = oracle._raw(K)
    Vr, _ = oracle._raw(V)
    Kr, Vr = Kr.copy(), Vr.copy()
    expK, expV = Kr.copy(), Vr.copy()
    knr, _ = oracle._raw(kn)
    vnr, _ = oracle._raw(vn)
    for bi, p in enumerate(lens):
        if p < m:
            expK[bi, p] = knr[bi]
            expV[bi, p] = vnr[bi]
    ln = lens.copy()
    over = oracle.kv_append(kn, vn, Kr, Vr, ln)
    assert over == 1
    assert np.array_equal(ln, [1, 4, 6, 6])
    assert Kr.tobytes() == expK.tobytes() and Vr.tobytes() == expV.tobytes()


# ---------------------------------------------------------------- beam reorder


def _beam_cache(dtype, seed, b=8, m=7, G=2, dh=64):
    K, _ = oracle._raw(rand((b, m, G, dh), seed, dtype))
    V, _ = oracle._raw(rand((b, m, G, dh), seed + 1, dtype))
    lens = np.random.default_rng(seed).integers(0, m + 1, size=b).astype(np.int32)
    return K.copy(), V.copy(), lens


def test_beam_reorder_identity_changes_nothing():
    K, V, lens = _beam_cache(torch.bfloat16, 150)
    K0, V0, l0 = K.copy(), V.copy(), lens.copy()
    for beam in (1, 2, 4, 8):
        assert oracle.kv_reorder(K, V, lens, np.arange(8) % beam, beam) == 0
        assert K.tobytes() == K0.tobytes() and V.tobytes() == V0.tobytes()
        assert np.array_equal(lens, l0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_beam_reorder_then_decode_equals_decode_of_gathered_rows(dtype):
    """Route 1: reorder in place, then decode.  Route 2: gather whole parent
    rows with numpy indexing and decode those.  Decode reads only j < L, so
    the two agree exactly iff the reorder moved every valid row and length."""
    b, beam, h, G, dh, m = 8, 4, 4, 2, 64, 7
    K, V, lens = _beam_cache(dtype, 152, b, m, G, dh)
    lens[lens == 0] = 1
    parent = np.array([3, 3, 0, 1, 2, 2, 2, 0], np.int32)   # duplicates, dropped beams
    src = (np.arange(b) // beam) * beam + parent
    q = rand((b, h, dh), 153, dtype)
    want = oracle.decode(q, K[src].copy(), V[src].copy(), lens[src].copy(), 0.125)
    assert oracle.kv_reorder(K, V, lens, parent, beam) == 0
    got = oracle.decode(q, K, V, lens, 0.125)
    assert np.array_equal(got, want)


def test_beam_reorder_leaves_positions_past_the_parent_length():
    K, V, lens = _beam_cache(torch.bfloat16, 154)
    K0, V0, l0 = K.copy(), V.copy(), lens.copy()
    parent = np.array([1, 0, 3, 3, 0, 0, 2, 1], np.int32)
    oracle.kv_reorder(K, V, lens, parent, 4)
    src = (np.arange(8) // 4) * 4 + parent
    for i in range(8):
        L = l0[src[i]]
        assert lens[i] == L
        assert K[i, L:].tobytes() == K0[i, L:].tobytes()
        assert V[i, L:].tobytes() == V0[i, L:].tobytes()
        assert K[i, :L].tobytes() == K0[src[i], :L].tobytes()


def test_beam_reorder_composes():
    """Reordering by p and then by r equals one reorder by p[r] (within the
    group), on every valid row and on lens."""
    b, beam = 8, 4
    K1, V1, l1 = _beam_cache(torch.float32, 156, b)
    K2, V2, l2 = K1.copy(), V1.copy(), l1.copy()
    g = np.random.default_rng(157)
    p = g.integers(0, beam, size=b).astype(np.int32)
    r = g.integers(0, beam, size=b).astype(np.int32)
    base = (np.arange(b) // beam) * beam
    oracle.kv_reorder(K1, V1, l1, p, beam)
    oracle.kv_reorder(K1, V1, l1, r, beam)
    oracle.kv_reorder(K2, V2, l2, p[base + r], beam)
    assert np.array_equal(l1, l2)
    for i in range(b):
        L = max(0, min(int(l1[i]), K1.shape[1]))
        assert K1[i, :L].tobytes() == K2[i, :L].tobytes()
        assert V1[i, :L].tobytes() == V2[i, :L].tobytes()


def test_beam_reorder_rejects_and_counts_bad_parents():
    K, V, lens = _beam_cache(torch.bfloat16, 158)
    K0, l0 = K.copy(), lens.copy()
    parent = np.array([0, 1, 4, -1, 0, 1, 2, 3], np.int32)   # rows 2, 3 invalid
    assert oracle.kv_reorder(K, V, lens, parent, 4) == 2
    assert K[2].tobytes() == K0[2].tobytes() and K[3].tobytes() == K0[3].tobytes()
    assert lens[2] == l0[2] and lens[3] == l0[3]
    with pytest.raises(ValueError):
        oracle.kv_reorder(K, V, lens, np.zeros(8, np.int32), 3)   # 3 does not divide 8


def test_append_then_attend_sees_new_token():
    """The concat precedes the logits (paper review section 3), so the new
    token attends to itself: with an empty cache the output is v_new."""
    q = rand((1, 4, 64), 150, mul=3.0)
    K = np.zeros((1, 4, 1, 64), np.float32)
    V = np.zeros((1, 4, 1, 64), np.float32)
    kn = rand((1, 1, 64), 151)
    vn = rand((1, 1, 64), 152)
    lens = np.array([0], np.int32)
    oracle.kv_append(kn, vn, K, V, lens)
    o = oracle.decode(q, K, V, lens, 0.125)
    for i in range(4):
        assert np.array_equal(o[0, i], f64(vn[0, 0]))


# ---------------------------------------------------------------- P12


def test_large_logits_are_shift_stable():
    """Adding a constant c to every logit leaves softmax unchanged.  Realised
    through an extra key dimension equal to 1 with a query entry c: with
    c*scale ~ 1e4 a softmax without the max-shift overflows even in fp64."""
    q = rand((2, 4, 63), 160, mul=20.0)                      # logits std ~ 20*sqrt(63)/8
    K = rand((2, 50, 1, 63), 161)
    V = rand((2, 50, 1, 63), 162)
    lens = np.array([50, 31], np.int32)
    o = oracle.decode(q, K, V, lens, 0.125)
    ref = bruteforce.decode(f64(q), f64(K), f64(V), lens, 0.125)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)
    c = 8.0e4
    q2 = torch.cat([q, torch.full((2, 4, 1), c)], dim=2)
    K2 = torch.cat([K, torch.ones(2, 50, 1, 1)], dim=3)
    V2 = torch.cat([V, torch.zeros(2, 50, 1, 1)], dim=3)
    o2 = oracle.decode(q2, K2, V2, lens, 0.125)
    assert np.isfinite(o2).all()
    # each logit now carries ~c*eps64 ~ 2e-11 of rounding from the +c term,
    # so agreement is to ~1e-10 relative, not to the last bit
    assert np.allclose(o2[..., :63], o, rtol=1e-9, atol=1e-10)


# ---------------------------------------------------------------- local window


@pytest.mark.parametrize("window", [1, 3, 32, 1000])
def test_local_window_against_bruteforce(window):
    """Local attention (study notes section 6.4): only the last `window` positions."""
    q = rand((2, 4, 8), 170)
    K = rand((2, 40, 2, 8), 171)
    V = rand((2, 40, 2, 8), 172)
    lens = np.array([40, 5], np.int32)
    o = oracle.decode(q, K, V, lens, 0.3, window=window)
    ref = bruteforce.decode(f64(q), f64(K), f64(V), lens, 0.3, window=window)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)
    if window == 1:
        for b in range(2):
            for i in range(4):
                assert np.array_equal(o[b, i], f64(V[b, lens[b] - 1, i // 2]))
    if window >= 40:
        assert np.array_equal(o, oracle.decode(q, K, V, lens, 0.3))


def test_oracle_rejects_bad_arguments():
    q = rand((1, 3, 8), 1)
    K = rand((1, 4, 2, 8), 2)
    with pytest.raises(ValueError):
        oracle.decode(q, K, K, np.array([4], np.int32), 1.0)  # G=2 does not divide h=3


# ---------------------------------------------------------------- attend (memory, mask)


def _memory_case(dtype, b=2, n=3, m=9, h=4, G=2, dh=64, seed=170):
    Q = rand((b, n, h, dh), seed, dtype)
    K = rand((b, m, G, dh), seed + 1, dtype)
    V = rand((b, m, G, dh), seed + 2, dtype)
    return Q, K, V


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_attend_with_mask_against_bruteforce(dtype):
    b, n, m, h = 2, 3, 9, 4
    Q, K, V = _memory_case(dtype)
    g = np.random.default_rng(171)
    mask = g.normal(0, 2, size=(b, h, n, m)).astype(np.float32)
    mask[0, 1, 2, :5] = -np.inf
    mask[1, 3, 0, :] = -np.inf                        # a fully hidden row
    got = oracle.attend(Q, K, V, 0.3, mask)
    want = bruteforce.memory(f64(Q), f64(K), f64(V), 0.3, mask)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)
    assert not got[1, 0, 3].any()
    got0 = oracle.attend(Q, K, V, 0.3)
    assert np.allclose(got0, bruteforce.memory(f64(Q), f64(K), f64(V), 0.3), rtol=1e-12,
                       atol=1e-13)


def test_attend_key_padding_mask_is_decode_with_lens():
    """n = 1 and -inf on keys j >= L_b (a [b, m] key-padding mask broadcast
    over heads and queries through zero strides) is decode over L_b rows."""
    b, m, h, G, dh = 3, 11, 4, 1, 64
    q = rand((b, h, dh), 175, torch.bfloat16)
    K = rand((b, m, G, dh), 176, torch.bfloat16)
    V = rand((b, m, G, dh), 177, torch.bfloat16)
    lens = np.array([11, 4, 1], np.int32)
    pad = np.where(np.arange(m)[None, :] < lens[:, None], 0.0, -np.inf).astype(np.float32)
    got = oracle.attend(q[:, None], K, V, 0.125, pad, strides=(m, 0, 0))
    want = oracle.decode(q, K, V, lens, 0.125)
    assert np.allclose(got[:, 0], want, rtol=1e-13, atol=1e-15)


def test_attend_causal_mask_is_prefill():
    b, n, h, G, dh = 2, 6, 4, 2, 64
    Q = rand((b, n, h, dh), 178, torch.bfloat16)
    K = rand((b, n, G, dh), 179, torch.bfloat16)
    V = rand((b, n, G, dh), 180, torch.bfloat16)
    causal = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], 0.0, -np.inf)
    mask = np.broadcast_to(causal.astype(np.float32), (b, h, n, n))
    got = oracle.attend(Q, K, V, 0.125, mask)
    assert np.allclose(got, oracle.prefill(Q, K, V, 0.125), rtol=1e-13, atol=1e-15)


def test_attend_hidden_key_equals_removed_key():
    Q, K, V = _memory_case(torch.float32)
    b, n, h = 2, 3, 4
    m = K.shape[1]
    mask = np.zeros((b, h, n, m), np.float32)
    mask[:, :, :, 4] = -np.inf
    keep = [j for j in range(m) if j != 4]
    got = oracle.attend(Q, K, V, 0.2, mask)
    want = oracle.attend(Q, K[:, keep].contiguous(), V[:, keep].contiguous(), 0.2)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)


def test_attend_mask_shift_invariance_and_one_hot():
    Q, K, V = _memory_case(torch.float32)
    b, n, h = 2, 3, 4
    m = K.shape[1]
    g = np.random.default_rng(181)
    # dyadic values, so that the shifted mask is exact in fp32
    mask = (g.integers(-16, 17, size=(b, h, n, m)) / 8.0).astype(np.float32)
    a = oracle.attend(Q, K, V, 0.2, mask)
    c = oracle.attend(Q, K, V, 0.2, mask + np.float32(37.0))
    assert np.allclose(a, c, rtol=1e-11, atol=1e-12)
    hot = np.zeros((b, h, n, m), np.float32)
    hot[:, :, :, 6] = 1e4                              # one key dominates completely
    o = oracle.attend(Q, K, V, 0.2, hot)
    Vd = f64(V)
    for i in range(h):
        assert np.array_equal(o[:, :, i], np.broadcast_to(Vd[:, None, 6, i // 2], o[:, :, i].shape))
