"""GPU: the library's calls inside a captured HIP graph.

Every entry point only enqueues kernels on the caller's stream (no
allocation, no memset, no host synchronisation), so a caller can capture a
forward and backward (and a decode step) once and replay them.  The graph is
replayed several times with the program's own eager work and synchronisations
in between, and every replay must give the same bits as the eager calls on the
same inputs.  Calls given an explicit stream (not the current one) give the
same bits as on the current stream.
"""
import numpy as np
import pytest

from gpu_util import default_scale, inputs, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_self_attention_sdpa_amd as ga
    ga.load_library()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_backward_graph_replays_equal_eager(dtype):
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs = 2, 3, 200, (64 if dtype == "bf16" else 16)
    x = inputs(B, H, T, hs, dtype, seed=111, workload="graph")
    s = default_scale(hs)
    print(f"case graph {dtype} B={B} H={H} T={T} hs={hs}", flush=True)
    t = {n: to_dev(a, dtype) for n, a in x.items()}
    code = {"bf16": ga.BF16, "f32": ga.F32}[dtype]
    o, dq, dk, dv = (torch.empty_like(t["q"]) for _ in range(4))
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(ga.gattn_bwd_workspace_bytes(B, H, T, hs, code), dtype=torch.uint8,
                     device="cuda")

    def step():
        ga.gattn_fwd(t["q"], t["k"], t["v"], o, lse, s)
        ga.gattn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, dq, dk, dv, s, ws)

    step()
    torch.cuda.synchronize()
    eager = [a.clone() for a in (o, lse, dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for a in (o, lse, dq, dk, dv):  # eager work between replays: poison the outputs
            a.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), eager):
            assert torch.equal(a, b), f"replay {r}: {n} differs from the eager call"


def test_decode_step_graph_replays_equal_eager():
    """One decode step (a key split with its merge launch, so the workspace is
    used) captured once and replayed after the query changes in place."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, Tk, hs = 2, 3, 1000, 64
    x = inputs(B, H, Tk, hs, "bf16", seed=112, workload="graph-decode")
    s = default_scale(hs)
    k, v = to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16")
    q = to_dev(x["q"][:, :, Tk - 1:], "bf16")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, 1), dtype=torch.float32, device="cuda")
    nb = ga.gattn_fwd_decode_workspace_bytes(B, H, 1, Tk, hs, ga.BF16)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ga.gattn_fwd_decode(q, k, v, o, lse, s, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ga.gattn_fwd_decode(q, k, v, o, lse, s, ws)
    for r in range(3):
        q.copy_(to_dev(x["q"][:, :, Tk - 1 - r:Tk - r], "bf16"))  # a new query, same buffer
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = o.clone(), lse.clone()
        ga.gattn_fwd_decode(q, k, v, o, lse, s, ws)
        torch.cuda.synchronize()
        assert torch.equal(got_o, o) and torch.equal(got_l, lse), f"replay {r}"


def test_explicit_stream_argument_equals_default_stream():
    """The calls given a stream of their own (not the current one) enqueue there
    and give the same bits as on the current stream."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs = 2, 3, 150, 64
    x = inputs(B, H, T, hs, "bf16", seed=113, workload="stream")
    s = default_scale(hs)
    print(f"case explicit stream bf16 B={B} H={H} T={T} hs={hs}", flush=True)
    t = {n: to_dev(a, "bf16") for n, a in x.items()}

    def run(stream):
        o, lse = ga.attention_forward(t["q"], t["k"], t["v"], s, stream=stream)
        dq, dk, dv = ga.attention_backward(t["q"], t["k"], t["v"], o, t["do"], lse, s,
                                           stream=stream)
        od, ld, keep = ga.attention_forward_dropout(t["q"], t["k"], t["v"], 0.1, 7, 1, s,
                                                    stream=stream, return_keep=True)
        gd = ga.attention_backward_dropout(t["q"], t["k"], t["v"], od, t["do"], ld, 0.1, 7, 1, s,
                                           stream=stream, keep=keep)
        return (o, lse, dq, dk, dv, od, ld, *gd)

    ref = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = run(side)
    side.synchronize()
    for i, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a, b), i
