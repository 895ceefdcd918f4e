"""mqa_decode_noalloc (the decode variant that takes no workspace and
allocates nothing) against mqa_decode_ex with a caller workspace: the same
kernels, so the outputs, caches and lens must be bitwise equal, and both
within the oracle's tolerance.  Two calls in a row, the second with a smaller
input, so the second reuses the scratch the first left behind."""
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


CASES = [
    # (config of the first call, config of the second, smaller call)
    (W.DecodeConfig("na1", torch.bfloat16, 64, 32, 1, 128, 8448, 1, 8192, True, 9101),
     W.DecodeConfig("na2", torch.bfloat16, 7, 32, 1, 128, 600, 1, 599, True, 9102)),
    (W.DecodeConfig("na3", torch.bfloat16, 300, 16, 2, 64, 400, 0, 390, False, 9103),
     W.DecodeConfig("na4", torch.bfloat16, 20, 8, 2, 64, 100, 1, 90, False, 9104)),
    (W.DecodeConfig("na5", torch.float32, 9, 8, 1, 128, 700, 1, 690, True, 9105),
     W.DecodeConfig("na6", torch.float32, 3, 8, 1, 128, 70, 1, 60, True, 9106)),
]


@pytest.mark.parametrize("first,second", CASES, ids=lambda c: c.name)
def test_noalloc_equals_workspace_decode(first, second):
    for cfg in (first, second):
        announce(f"decode_noalloc {cfg}")
        inp = W.decode_inputs(cfg)
        d1 = {k: v.cuda() for k, v in inp.items()}
        d2 = {k: v.cuda() for k, v in inp.items()}
        kw1 = dict(k_new=d1["k_new"], v_new=d1["v_new"]) if cfg.append else {}
        kw2 = dict(k_new=d2["k_new"], v_new=d2["v_new"]) if cfg.append else {}
        out = torch.empty_like(d1["q"])
        mqa.decode_noalloc(d1["q"], d1["K"], d1["V"], d1["lens"], cfg.scale, out=out, **kw1)
        if cfg.append:
            ref = mqa.append_decode(d2["q"], d2["k_new"], d2["v_new"], d2["K"], d2["V"],
                                    d2["lens"], cfg.scale)
        else:
            ref = mqa.decode(d2["q"], d2["K"], d2["V"], d2["lens"], cfg.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{cfg.name}: output differs from the workspace decode"
        assert torch.equal(d1["lens"], d2["lens"]), f"{cfg.name}: lens"
        assert raw(d1["K"].cpu()).tobytes() == raw(d2["K"].cpu()).tobytes(), f"{cfg.name}: K"
        assert raw(d1["V"].cpu()).tobytes() == raw(d2["V"].cpu()).tobytes(), f"{cfg.name}: V"
        lens = inp["lens"].numpy().copy()
        K, V = inp["K"], inp["V"]
        if cfg.append:
            K, V = raw(inp["K"]), raw(inp["V"])
            oracle.kv_append(inp["k_new"], inp["v_new"], K, V, lens)
        expect = oracle.decode(inp["q"], K, V, lens, cfg.scale)
        assert_parity(out, expect, cfg.dtype, f"{cfg.name} noalloc vs oracle")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """b = 4.5M single-position sequences need an 18 MB schedule header, more
    than the 16 MiB scratch: refused on the host, nothing launched (every
    buffer is real, so even a launch would stay in bounds)."""
    b, h, dh = 4_500_000, 1, 64
    announce(f"decode_noalloc refuses b={b}")
    q = torch.zeros(b, h, dh, dtype=torch.bfloat16, device="cuda")
    K = torch.zeros(b, 1, 1, dh, dtype=torch.bfloat16, device="cuda")
    V = torch.zeros_like(K)
    lens = torch.ones(b, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(mqa.MQAError) as e:
        mqa.decode_noalloc(q, K, V, lens, 0.125, out=out)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool((out[:4096] == 7.0).all())        # nothing ran
