"""GPU backward metamorphic checks through the C ABI (bf16 path).

No kernel uses atomics: dq (the dQ kernel, one workgroup per query tile) and
dk, dv (the dK/dV kernel, one workgroup per key tile) each come from a fixed
order of operations, so determinism, causality and the head split are checked
bit for bit; a race or a lost or repeated tile in either kernel breaks one of
them.  Scaling V by 2 scales dS by 2, and dS enters the dq and dk products as
fp16, whose subnormal range (|dS| < 2^-14) rounds on a fixed grid that does
not scale: there dq and dk x 2 are held to one bf16 ulp, dv bit for bit."""
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


def run(t, scale, out=None):
    import torch
    import causal_self_attention_sdpa_amd as ga
    o, lse = ga.attention_forward(t["q"], t["k"], t["v"], scale)
    if out is None:
        dq, dk, dv = ga.attention_backward(t["q"], t["k"], t["v"], o, t["do"], lse, scale)
    else:
        dq, dk, dv = out
        B, H, T, hs = t["q"].shape
        ws = torch.empty(ga.gattn_bwd_workspace_bytes(B, H, T, hs, ga.BF16), dtype=torch.uint8,
                         device="cuda")
        ga.gattn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, dq, dk, dv, scale, ws)
    torch.cuda.synchronize()
    return dq, dk, dv


def dev_inputs(B, H, T, hs, seed):
    x = inputs(B, H, T, hs, "bf16", seed=seed, workload="bwd-meta")
    return {n: to_dev(a, "bf16") for n, a in x.items()}


@pytest.mark.parametrize("hs", [64, 32])
def test_bwd_causality(hs):
    """Changing rows < j of q and dO leaves dk, dv rows >= j bit-identical;
    changing rows > i of q, k, v, dO leaves dq rows <= i bit-identical."""
    import torch
    T = 333
    t = dev_inputs(2, 2, T, hs, 31)
    s = default_scale(hs)
    dq0, dk0, dv0 = run(t, s)
    for j in (1, 64, 128, 200):
        p = dict(t)
        p["q"] = t["q"].clone()
        p["do"] = t["do"].clone()
        p["q"][:, :, :j] = p["q"][:, :, :j] * 2 + 1
        p["do"][:, :, :j] = -p["do"][:, :, :j]
        _, dk1, dv1 = run(p, s)
        assert torch.equal(dk0[:, :, j:], dk1[:, :, j:]), j
        assert torch.equal(dv0[:, :, j:], dv1[:, :, j:]), j
    for i in (0, 100, 255):
        p = {n: t[n].clone() for n in t}
        for n in p:
            p[n][:, :, i + 1:] = p[n][:, :, i + 1:] * 3 - 1
        dq1, _, _ = run(p, s)
        assert torch.equal(dq0[:, :, :i + 1], dq1[:, :, :i + 1]), i


def test_bwd_value_scaling():
    """V x 2: dv unchanged bit for bit; dk x 2 and dq x 2 to one bf16 ulp
    (power-of-two scaling commutes with every rounding except that of fp16
    subnormal dS values)."""
    import torch
    t = dev_inputs(2, 3, 290, 64, 32)
    s = default_scale(64)
    dq0, dk0, dv0 = run(t, s)
    t2 = dict(t)
    t2["v"] = t["v"] * 2
    dq1, dk1, dv1 = run(t2, s)
    assert torch.equal(dv1, dv0)
    for a, b in ((dk1, dk0 * 2), (dq1, dq0 * 2)):
        a, b = a.float(), b.float()
        assert torch.all((a - b).abs() <= b.abs() * 2.0 ** -7 + 1e-6)
        assert (a != b).float().mean().item() < 0.01


def test_bwd_deterministic():
    import torch
    t = dev_inputs(3, 4, 777, 64, 33)
    s = default_scale(64)
    a = run(t, s)
    b = run(t, s)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for x in a:
        assert torch.isfinite(x).all()


def test_bwd_heads_split():
    """25 heads in one call: dq, dk, dv equal the single-head calls bit for bit."""
    import torch
    t = dev_inputs(1, 25, 200, 64, 34)
    s = default_scale(64)
    dq, dk, dv = run(t, s)
    for h in (0, 7, 24):
        th = {n: a[:, h:h + 1].contiguous() for n, a in t.items()}
        dqh, dkh, dvh = run(th, s)
        assert torch.equal(dkh, dk[:, h:h + 1]) and torch.equal(dvh, dv[:, h:h + 1]), h
        assert torch.equal(dqh, dq[:, h:h + 1]), h


def test_bwd_guard_bands_and_poison():
    """Outputs are fully overwritten (NaN poison gone) and nothing is written
    outside them (sentinels survive)."""
    import torch
    B, H, T, hs = 2, 2, 221, 64
    t = dev_inputs(B, H, T, hs, 35)
    s = default_scale(hs)
    n = B * H * T * hs
    pad = 2048
    bufs = [torch.full((n + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
            for _ in range(3)]
    for b in bufs:
        b[:pad] = 7.0
        b[pad + n:] = 7.0
    views = [b[pad:pad + n].view(B, H, T, hs) for b in bufs]
    dq, dk, dv = run(t, s, out=views)
    for b, vw in zip(bufs, views):
        assert torch.all(b[:pad] == 7.0) and torch.all(b[pad + n:] == 7.0)
        assert torch.isfinite(vw).all()
    ref = run(t, s)
    assert torch.equal(dq, ref[0]) and torch.equal(dk, ref[1]) and torch.equal(dv, ref[2])
