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


@pytest.mark.parametrize("window", [0, 7])
def test_serial_loop_graph_with_lens_reset(window):
    """The serial decoding loop as the benchmark issues it: one fill kernel
    resets the lens of every layer, then n tokens of fused append + decode
    through each layer, all captured in one graph.  Each token appends its own
    row, so after a replay layer l's cache holds rows 0..n-1 of its token
    sequence, lens is n, and the last output is the decode of the last
    token's query over those rows.  Replayed three times with eager work and
    synchronisation in between; every replay checked bytewise and against
    the oracle."""
    b, h, G, dh, n, layers = 48, 8, 1, 128, 40, 2
    gen = torch.Generator().manual_seed(7700 + window)
    rnd = lambda *s: torch.randn(*s, generator=gen).to(torch.bfloat16)
    Ks = [rnd(b, n + 8, G, dh) for _ in range(layers)]
    Vs = [rnd(b, n + 8, G, dh) for _ in range(layers)]
    qs = [rnd(n, b, h, dh) for _ in range(layers)]
    kns = [rnd(n, b, G, dh) for _ in range(layers)]
    vns = [rnd(n, b, G, dh) for _ in range(layers)]
    dK, dV = [k.cuda() for k in Ks], [v.cuda() for v in Vs]
    dq, dkn, dvn = [q.cuda() for q in qs], [k.cuda() for k in kns], [v.cuda() for v in vns]
    lens = torch.full((layers, b), 5, dtype=torch.int32, device="cuda")
    out = torch.empty(b, h, dh, dtype=torch.bfloat16, device="cuda")
    wss = [mqa.workspace_for(h, dK[l]) for l in range(layers)]
    steps = [[mqa.DecodeStep(dq[l][t], dK[l], dV[l], lens[l], 1.0 / dh ** 0.5, out=out,
                             workspace=wss[l], k_new=dkn[l][t], v_new=dvn[l][t], window=window)
              for l in range(layers)] for t in range(n)]

    def loop():
        lens.zero_()
        for t in range(n):
            for l in range(layers):
                steps[t][l]()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            loop()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(lens.cpu(), torch.full((layers, b), 5, dtype=torch.int32))

    # the oracle: layer l's cache rows 0..n-1 are its appended rows
    Kf, Vf = raw(Ks[-1]), raw(Vs[-1])
    Kf[:, :n] = raw(kns[-1].transpose(0, 1).contiguous())
    Vf[:, :n] = raw(vns[-1].transpose(0, 1).contiguous())
    expect = oracle.decode(qs[-1][n - 1], Kf, Vf, np.full(b, n, dtype=np.int32), 1.0 / dh ** 0.5,
                           window=window)
    twin = mqa.DecodeStep(dq[0][0].clone(), dK[0].clone(), dV[0].clone(),
                          torch.full((b,), 3, dtype=torch.int32, device="cuda"), 0.1)
    for rep in range(3):
        announce(f"serial loop graph replay {rep} (window={window})")
        g.replay()
        for _ in range(2):                                   # eager work in between
            twin()
        torch.cuda.synchronize()
        assert torch.equal(lens.cpu(), torch.full((layers, b), n, dtype=torch.int32))
        for l in range(layers):
            kc = raw(dK[l][:, :n].cpu().contiguous())
            assert kc.tobytes() == raw(kns[l].transpose(0, 1).contiguous()).tobytes(), f"K {l}"
            vc = raw(dV[l][:, :n].cpu().contiguous())
            assert vc.tobytes() == raw(vns[l].transpose(0, 1).contiguous()).tobytes(), f"V {l}"
        assert_parity(out, expect, torch.bfloat16, f"serial loop replay {rep} window {window}")
