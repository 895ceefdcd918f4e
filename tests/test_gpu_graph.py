"""Decode steps replayed from a HIP graph (the way the serving loop and the
benchmark issue them) against the same steps issued eagerly and against the
fp64 oracle.  Each replay is checked, with eager work and synchronisation in
between, so a graph that only works once (or depends on state it does not
capture) fails here."""
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


@pytest.mark.parametrize("fused", [True, False])
def test_graph_replays_equal_eager_steps_and_oracle(fused):
    cfg = W.DecodeConfig("graph", torch.bfloat16, 6, 32, 1, 128, 400, 1, 300, True, 7600)
    inp = W.decode_inputs(cfg)
    steps_per_graph, replays = 3, 3
    dev = {k: v.cuda() for k, v in inp.items()}
    ref = {k: v.cuda().clone() for k, v in inp.items()}          # eager twin
    ws_g = mqa.workspace_for(cfg.h, dev["K"])
    ws_e = mqa.workspace_for(cfg.h, ref["K"])
    step_g = mqa.DecodeStep(dev["q"], dev["K"], dev["V"], dev["lens"], cfg.scale, workspace=ws_g,
                            k_new=dev["k_new"], v_new=dev["v_new"], fused=fused)
    step_e = mqa.DecodeStep(ref["q"], ref["K"], ref["V"], ref["lens"], cfg.scale, workspace=ws_e,
                            k_new=ref["k_new"], v_new=ref["v_new"], fused=fused)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(steps_per_graph):
                step_g()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # capturing records the steps without running them
    assert torch.equal(dev["lens"].cpu(), inp["lens"])

    Kr, Vr, lr = raw(inp["K"]), raw(inp["V"]), inp["lens"].numpy().copy()
    for rep in range(replays):
        announce(f"graph replay {rep} (fused={fused})")
        g.replay()
        for _ in range(steps_per_graph):                           # eager work in between
            step_e()
        torch.cuda.synchronize()
        assert torch.equal(step_g.out, step_e.out), f"replay {rep}: output differs from eager"
        assert torch.equal(dev["lens"], ref["lens"]), f"replay {rep}: lens"
        assert raw(dev["K"].cpu()).tobytes() == raw(ref["K"].cpu()).tobytes(), f"replay {rep}: K"
        assert raw(dev["V"].cpu()).tobytes() == raw(ref["V"].cpu()).tobytes(), f"replay {rep}: V"
        # the oracle's version of the same steps (the same new row every step)
        for _ in range(steps_per_graph):
            oracle.kv_append(inp["k_new"], inp["v_new"], Kr, Vr, lr)
        expect = oracle.decode(inp["q"], Kr, Vr, lr, cfg.scale)
        assert_parity(step_g.out, expect, cfg.dtype, f"graph replay {rep}")
        assert np.array_equal(dev["lens"].cpu().numpy(), lr)
