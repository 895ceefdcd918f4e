"""GPU parity of the causal prefill against the fp64 oracle (full masked-row
route), plus its cache hand-off to decode."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import announce, assert_parity
from query_decode_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import query_decode_attention_amd as mqa


def make(dtype, b, n, h, G, dh, seed):
    cfg = W.PrefillConfig("t", dtype, b, n, h, G, dh, seed)
    return cfg, W.prefill_inputs(cfg)


CASES = [
    (torch.bfloat16, 2, 100, 32, 1, 128),   # MQA, ragged last tile
    (torch.bfloat16, 1, 257, 32, 4, 128),   # GQA h/G = 8 (4 rows per wave)
    (torch.bfloat16, 2, 70, 4, 4, 64),      # MHA h/G = 1 (32 rows per wave)
    (torch.bfloat16, 1, 64, 12, 1, 64),     # h/G = 12 padded to 16
    (torch.bfloat16, 1, 300, 32, 1, 64),    # d_h 64, ten key tiles in flight three ahead
    (torch.float32, 1, 90, 8, 2, 128),
    (torch.float32, 2, 33, 32, 1, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{str(c[0])[6:]}-b{c[1]}n{c[2]}h{c[3]}G{c[4]}d{c[5]}")
def test_prefill_parity_grid(case):
    dtype, b, n, h, G, dh = case
    announce(f"prefill grid {case}")
    cfg, inp = make(dtype, b, n, h, G, dh, seed=8000 + n + h + G)
    O = mqa.prefill_causal(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), cfg.scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], cfg.scale)
    assert_parity(O, ref, dtype, f"prefill {case}")


def test_prefill_first_row_is_first_value():
    announce("prefill row 0 exact")
    cfg, inp = make(torch.bfloat16, 2, 40, 32, 1, 128, seed=8100)
    O = mqa.prefill_causal(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), cfg.scale).cpu()
    for b in range(2):
        assert torch.equal(O[b, 0], inp["V"][b, 0, 0].expand(32, 128))


def test_c5_full_size_sampled_rows():
    """b=4, n=4096, h=32, G=1: the GPU computes everything; the oracle checks
    288 seeded rows including the first and last of every sequence."""
    announce("c5 full size, sampled rows")
    cfg = W.C5
    inp = W.prefill_inputs(cfg)
    O = mqa.prefill_causal(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), cfg.scale).cpu()
    g = torch.Generator().manual_seed(5)
    rows = set()
    for b in range(cfg.b):
        rows.update({b * cfg.n, b * cfg.n + cfg.n - 1, b * cfg.n + 31, b * cfg.n + 32})
    rows.update(torch.randint(0, cfg.b * cfg.n, (272,), generator=g).tolist())
    rows = sorted(rows)
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], cfg.scale, rows=rows)
    got = O.reshape(cfg.b * cfg.n, cfg.h, cfg.dh)[rows]
    assert_parity(got, ref, torch.bfloat16, f"c5 {len(rows)} rows")


def test_prefill_fills_cache_and_hands_off_to_decode():
    """Prefill writes K/V into the cache and sets lens = n; a decode step with
    query Q[:, t] over a cache of t+1 rows equals prefill row t."""
    announce("prefill -> cache -> decode")
    cfg, inp = make(torch.bfloat16, 2, 150, 32, 1, 128, seed=8200)
    m_cap = 200
    Kc = torch.full((2, m_cap, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    Vc = torch.full_like(Kc, float("nan"))
    lens = torch.zeros(2, dtype=torch.int32, device="cuda")
    Q, K, V = inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda()
    O = mqa.prefill_causal(Q, K, V, cfg.scale, cache_K=Kc, cache_V=Vc, lens=lens)
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == [150, 150]
    assert torch.equal(Kc[:, :150].cpu(), inp["K"]) and torch.equal(Vc[:, :150].cpu(), inp["V"])
    assert torch.isnan(Kc[:, 150:].float()).all()
    for t in (0, 31, 32, 149):
        lt = torch.full((2,), t + 1, dtype=torch.int32, device="cuda")
        o = mqa.decode(Q[:, t].contiguous(), Kc, Vc, lt, cfg.scale)
        ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], cfg.scale, rows=[t, 150 + t])
        assert_parity(o, ref, torch.bfloat16, f"decode row {t}")
        assert_parity(O[:, t], ref, torch.bfloat16, f"prefill row {t}")


# Instances chosen by the scale's sign: a positive scale folds the scale into
# the exponent (max over raw scores); zero or a negative scale takes the
# unfolded softmax.  Both must match the oracle on the same inputs.
SCALE_CASES = [
    # dtype, b, n, h, G, dh, scale
    (torch.bfloat16, 2, 75, 32, 1, 128, 0.0),
    (torch.bfloat16, 2, 75, 32, 1, 128, -0.3),
    (torch.bfloat16, 1, 130, 16, 2, 64, 0.0),     # h/G = 8: four rows per wave
    (torch.bfloat16, 1, 66, 4, 4, 128, -0.09),    # MHA: 32 rows per wave
    (torch.float32, 1, 70, 8, 1, 64, 0.0),
    (torch.float32, 2, 41, 32, 1, 128, -0.2),
]


@pytest.mark.parametrize("case", SCALE_CASES,
                         ids=lambda c: f"{str(c[0])[6:]}-n{c[2]}h{c[3]}G{c[4]}d{c[5]}-s{c[6]}")
def test_prefill_nonpositive_scale(case):
    dtype, b, n, h, G, dh, scale = case
    announce(f"prefill scale {scale} {case}")
    cfg, inp = make(dtype, b, n, h, G, dh, seed=8300 + n + h)
    O = mqa.prefill_causal(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], scale)
    assert_parity(O, ref, dtype, f"prefill scale {scale} {case}")
    if scale == 0.0:
        # every weight is equal: row t is the mean of V rows 0..t of its group
        Vd = inp["V"].double()
        csum = Vd.cumsum(dim=1) / torch.arange(1, n + 1, dtype=torch.float64).view(1, n, 1, 1)
        mean = csum.repeat_interleave(h // G, dim=2)
        assert_parity(O, mean.numpy(), dtype, "prefill scale 0 = running mean of V")


@pytest.mark.parametrize("scale_sign", [1.0, -1.0])
@pytest.mark.parametrize("dtype", [torch.bfloat16])
def test_prefill_large_logits(scale_sign, dtype):
    """Q x 20: logits with a standard deviation of ~20, so exp without the
    running max overflows fp32; both softmax instances (folded and not)."""
    announce(f"prefill Q x 20, scale sign {scale_sign}, {dtype}")
    cfg, inp = make(dtype, 2, 120, 32, 1, 128, seed=8400 + int(scale_sign))
    inp["Q"] = (inp["Q"].float() * 20).to(dtype)
    scale = scale_sign * cfg.scale
    O = mqa.prefill_causal(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], scale)
    assert_parity(O, ref, dtype, f"prefill Q x 20 scale {scale}")


@pytest.mark.parametrize("jump_at", [100, 5])
def test_prefill_logit_jump_past_the_reference(jump_at):
    """The bf16 kernel fixes each column's softmax reference at its first
    visible tile; a key whose logit exceeds it by more than the slack sends
    the workgroup to the rescaling path.  Q[..., 0] = 20 and K[jump_at, 0] =
    40 give that key a logit of ~70.7 against ~N(0, 1) elsewhere: at key 100
    (tile 3) the rows that see it take the rescaling path, at key 5 (tile 0)
    the reference already holds it."""
    announce(f"prefill logit jump at key {jump_at}")
    cfg, inp = make(torch.bfloat16, 2, 180, 32, 1, 128, seed=8500 + jump_at)
    inp["Q"][..., 0] = 20.0
    inp["K"][:, jump_at, :, 0] = 40.0
    O = mqa.prefill_causal(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), cfg.scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], cfg.scale)
    assert_parity(O, ref, torch.bfloat16, f"prefill logit jump at key {jump_at}")
