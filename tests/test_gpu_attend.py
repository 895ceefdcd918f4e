"""GPU parity of attention over a fixed memory (non-causal, additive mask)
against the fp64 oracle, on the same seeded inputs, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import announce, assert_parity
from query_decode_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import query_decode_attention_amd as mqa


def make_mask(kind, b, h, n, m, seed):
    """Returns (mask tensor broadcastable to [b,h,n,m] or None)."""
    g = torch.Generator("cpu").manual_seed(seed)
    if kind == "none":
        return None
    if kind == "pad":
        lens = torch.randint(1, m + 1, (b,), generator=g)
        mask = torch.zeros(b, 1, 1, m)
        for bi in range(b):
            mask[bi, 0, 0, int(lens[bi]):] = float("-inf")
        return mask
    mask = torch.randn(b, h, n, m, generator=g) * 2.0
    if kind == "full_inf":
        hide = torch.rand(b, h, n, m, generator=g) < 0.3
        mask[hide] = float("-inf")
        mask[0, h - 1, n - 1, :] = float("-inf")      # a row with every key hidden
    return mask


def oracle_ref(Q, K, V, scale, mask, rows=None):
    if mask is None:
        return oracle.attend(Q, K, V, scale, rows=rows)
    b, n, h = Q.shape[0], Q.shape[1], Q.shape[2]
    m = K.shape[1]
    full = mask.expand(b, h, n, m).contiguous()
    return oracle.attend(Q, K, V, scale, full.numpy(), rows=rows)


GRID = [
    # dtype, b, n, m, h, G, dh, mask
    (torch.bfloat16, 2, 5, 37, 8, 2, 64, "none"),
    (torch.bfloat16, 1, 17, 100, 32, 1, 128, "pad"),
    (torch.bfloat16, 3, 9, 64, 4, 4, 128, "full"),
    (torch.float32, 2, 33, 1, 32, 1, 64, "none"),
    (torch.float32, 2, 12, 70, 16, 2, 128, "full_inf"),
    (torch.bfloat16, 1, 40, 500, 32, 8, 128, "pad"),
    (torch.bfloat16, 2, 1, 300, 32, 1, 128, "full_inf"),
    (torch.float32, 1, 20, 45, 8, 1, 64, "pad"),
    (torch.bfloat16, 2, 20, 90, 8, 1, 64, "full"),      # d_h 64: V^T read transposed, padded chunks
    (torch.bfloat16, 1, 33, 165, 16, 4, 64, "pad"),
]


@pytest.mark.parametrize("dtype,b,n,m,h,G,dh,kind", GRID)
def test_attend_grid(dtype, b, n, m, h, G, dh, kind):
    what = f"attend {dtype} b={b} n={n} m={m} h={h} G={G} dh={dh} mask={kind}"
    announce(what)
    cfg = W.MemoryConfig("t", dtype, b, n, m, h, G, dh, m, m, 400 + n + m)
    inp = W.memory_inputs(cfg)
    mask = make_mask(kind, b, h, n, m, 401 + m)
    out = mqa.attend(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), cfg.scale,
                     mask=None if mask is None else mask.cuda())
    torch.cuda.synchronize()
    ref = oracle_ref(inp["Q"], inp["K"], inp["V"], cfg.scale, mask)
    assert_parity(out, ref, dtype, what)


def test_attend_with_causal_mask_matches_prefill():
    b, n, h, G, dh = 2, 70, 32, 1, 128
    cfg = W.MemoryConfig("t", torch.bfloat16, b, n, n, h, G, dh, n, n, 410)
    inp = W.memory_inputs(cfg)
    causal = torch.full((n, n), float("-inf")).triu(1)
    out = mqa.attend(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), cfg.scale,
                     mask=causal.cuda().view(1, 1, n, n))
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], cfg.scale)
    assert_parity(out, ref, torch.bfloat16, "attend with a causal mask vs prefill oracle")


def test_attend_encdec_full_size_sampled_rows():
    cfg = W.ENCDEC
    announce(f"attend {cfg.name} (sampled rows)")
    inp = W.memory_inputs(cfg)
    out = mqa.attend(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), cfg.scale,
                     mask=inp["mask"].cuda())
    torch.cuda.synchronize()
    g = np.random.default_rng(411)
    rows = np.concatenate([[0, cfg.n - 1, cfg.n, 2 * cfg.n - 1, cfg.b * cfg.n - 1],
                           g.integers(0, cfg.b * cfg.n, size=43)])
    ref = oracle.attend(inp["Q"], inp["K"], inp["V"], cfg.scale, inp["mask"].numpy(),
                        strides=(cfg.m, 0, 0), rows=rows)
    got = out.reshape(cfg.b * cfg.n, cfg.h, cfg.dh)[torch.as_tensor(rows).cuda()]
    assert_parity(got, ref, cfg.dtype, f"{cfg.name} sampled rows")


def test_attend_argument_errors_raise():
    Q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16, device="cuda")
    K = torch.zeros(1, 3, 1, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mqa.attend(Q, K, K, 1.0, mask=torch.zeros(1, 1, 1, 3, dtype=torch.float16, device="cuda"))
    Q96 = torch.zeros(1, 2, 4, 96, dtype=torch.bfloat16, device="cuda")
    K96 = torch.zeros(1, 3, 1, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mqa.MQAError):
        mqa.attend(Q96, K96, K96, 1.0)             # d_h = 96: rejected by the library


# Unmasked attention takes the folded softmax for a positive scale and the
# unfolded one for zero or a negative scale; masked attention never folds.
# Each instance is run with a scale <= 0 and with very large logits.
SCALE_GRID = [
    # dtype, b, n, m, h, G, dh, mask, scale
    (torch.bfloat16, 2, 9, 70, 32, 1, 128, "none", 0.0),
    (torch.bfloat16, 1, 30, 45, 8, 2, 64, "none", -0.25),
    (torch.float32, 2, 7, 100, 16, 1, 128, "none", 0.0),
    (torch.float32, 1, 12, 33, 32, 4, 64, "none", -0.1),
    (torch.bfloat16, 2, 6, 90, 32, 1, 128, "pad", 0.0),
    (torch.bfloat16, 1, 5, 64, 8, 8, 128, "full_inf", -0.2),
]


@pytest.mark.parametrize("dtype,b,n,m,h,G,dh,kind,scale", SCALE_GRID)
def test_attend_nonpositive_scale(dtype, b, n, m, h, G, dh, kind, scale):
    what = f"attend scale {scale} {dtype} b={b} n={n} m={m} h={h} G={G} dh={dh} mask={kind}"
    announce(what)
    cfg = W.MemoryConfig("t", dtype, b, n, m, h, G, dh, m, m, 420 + n + m)
    inp = W.memory_inputs(cfg)
    mask = make_mask(kind, b, h, n, m, 421 + m)
    out = mqa.attend(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), scale,
                     mask=None if mask is None else mask.cuda())
    torch.cuda.synchronize()
    ref = oracle_ref(inp["Q"], inp["K"], inp["V"], scale, mask)
    assert_parity(out, ref, dtype, what)
    if scale == 0.0 and kind == "none":
        # equal weights: every query row is the mean of the group's V rows
        mean = inp["V"].double().mean(dim=1, keepdim=True).repeat_interleave(h // G, dim=2)
        assert_parity(out, mean.expand(b, n, h, dh).numpy(), dtype, what + " = mean of V")


@pytest.mark.parametrize("kind", ["none", "pad", "full"])
@pytest.mark.parametrize("scale_sign", [1.0, -1.0])
def test_attend_large_logits(kind, scale_sign):
    """Q x 20 on every attend instance: folded (positive scale, no mask),
    unfolded (negative scale), per-key mask and general mask."""
    b, n, m, h, G, dh = 2, 21, 150, 32, 1, 128
    what = f"attend Q x 20 mask={kind} scale sign {scale_sign}"
    announce(what)
    cfg = W.MemoryConfig("t", torch.bfloat16, b, n, m, h, G, dh, m, m, 430 + len(kind))
    inp = W.memory_inputs(cfg)
    inp["Q"] = (inp["Q"].float() * 20).to(torch.bfloat16)
    mask = make_mask(kind, b, h, n, m, 431)
    scale = scale_sign * cfg.scale
    out = mqa.attend(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), scale,
                     mask=None if mask is None else mask.cuda())
    torch.cuda.synchronize()
    ref = oracle_ref(inp["Q"], inp["K"], inp["V"], scale, mask)
    assert_parity(out, ref, torch.bfloat16, what)


@pytest.mark.parametrize("kind", ["none", "pad", "full"])
def test_attend_logit_jump_past_the_reference(kind):
    """A key whose logit exceeds the first tile's maximum by far more than
    the bf16 kernel's fixed-reference slack (key 100 of 300, logit ~70.7):
    every workgroup takes the rescaling path, with each mask kind."""
    b, n, m, h, G, dh = 2, 19, 300, 32, 1, 128
    what = f"attend logit jump mask={kind}"
    announce(what)
    cfg = W.MemoryConfig("t", torch.bfloat16, b, n, m, h, G, dh, m, m, 440 + len(kind))
    inp = W.memory_inputs(cfg)
    inp["Q"][..., 0] = 20.0
    inp["K"][:, 100, :, 0] = 40.0
    mask = make_mask(kind, b, h, n, m, 441)
    if kind == "pad":
        mask[..., :150] = 0.0          # key 100 stays visible
    out = mqa.attend(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), cfg.scale,
                     mask=None if mask is None else mask.cuda())
    torch.cuda.synchronize()
    ref = oracle_ref(inp["Q"], inp["K"], inp["V"], cfg.scale, mask)
    assert_parity(out, ref, torch.bfloat16, what)


KEY_PAD_CASES = [
    # dtype, m, dh, G: visible keys per sequence below
    (torch.bfloat16, 300, 128, 1),
    (torch.bfloat16, 300, 64, 2),
    (torch.float32, 300, 128, 1),
]


@pytest.mark.parametrize("dtype,m,dh,G", KEY_PAD_CASES)
def test_attend_key_padding_edges(dtype, m, dh, G):
    """A key-padding mask whose last visible key falls at and around tile
    boundaries (32 keys), a sequence with every key hidden (zeros), keys
    visible only in the middle, and only the very last key visible.  The
    pipelined kernel stops each workgroup after the last tile with a visible
    key; the hidden tiles must add exactly nothing."""
    ends = [1, 31, 32, 33, 64, 65, 299, 300, 0]
    b, n, h = len(ends) + 2, 9, 32
    what = f"attend key padding edges {dtype} m={m} dh={dh} G={G}"
    announce(what)
    cfg = W.MemoryConfig("t", dtype, b, n, m, h, G, dh, m, m, 450 + dh + G)
    inp = W.memory_inputs(cfg)
    mask = torch.zeros(b, 1, 1, m)
    for bi, e in enumerate(ends):
        mask[bi, 0, 0, e:] = float("-inf")
    mask[len(ends), 0, 0, :100] = float("-inf")      # visible [100, 150) only
    mask[len(ends), 0, 0, 150:] = float("-inf")
    mask[len(ends) + 1, 0, 0, :m - 1] = float("-inf")  # only the last key visible
    out = mqa.attend(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), cfg.scale,
                     mask=mask.cuda())
    torch.cuda.synchronize()
    ref = oracle_ref(inp["Q"], inp["K"], inp["V"], cfg.scale, mask)
    assert_parity(out, ref, dtype, what)
    # the sequence with every key hidden gives exact zeros
    assert torch.count_nonzero(out[len(ends) - 1]).item() == 0
