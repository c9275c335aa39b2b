"""GPU forward checks through the C ABI: parity of o and lse with the oracle,
and metamorphic properties that hold bit for bit on the bf16 MFMA path."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import check_close, default_scale, inputs, to_dev

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_self_attention_sdpa_amd as ga
    ga.load_library()


def fwd(q, k, v, scale, lse=True):
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs = q.shape
    o = torch.full_like(q, float("nan"))
    l = torch.full((B, H, T), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    ga.gattn_fwd(q, k, v, o, l, scale)
    torch.cuda.synchronize()
    return o, l


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _parity(B, H, T, hs, seed, qkv_scale=1.0, rel=0.0, slices=None):
    x = inputs(B, H, T, hs, "bf16", seed=seed, qkv_scale=qkv_scale, workload=f"fwd{B}.{H}.{T}.{hs}")
    s = default_scale(hs)
    print(f"case fwd bf16 B={B} H={H} T={T} hs={hs} x{qkv_scale} seed={seed}", flush=True)
    t = {n: to_dev(a, "bf16") for n, a in x.items()}
    o, l = fwd(t["q"], t["k"], t["v"], s)
    go, gl = np64(o), np64(l)
    if slices is None:
        ro, rl = oracle.attention_forward(x["q"], x["k"], x["v"], s)
    else:
        sel = lambda a: np.stack([a[b, h] for b, h in slices])[:, None]
        ro, rl = oracle.attention_forward(sel(x["q"]), sel(x["k"]), sel(x["v"]), s)
        go = np.stack([go[b, h] for b, h in slices])[:, None]
        gl = np.stack([gl[b, h] for b, h in slices])[:, None]
    return check_close((go, gl), (ro, rl), BF16_TOL, rel, names=("o", "lse"),
                       where=f"fwd {(B, H, T, hs)}")


@pytest.mark.parametrize("T", [1, 2, 17, 63, 64, 65, 127, 128, 129, 191, 256, 300, 513])
@pytest.mark.parametrize("hs", [64, 32])
def test_fwd_parity_lengths(T, hs):
    _parity(2, 3, T, hs, seed=T)


def test_fwd_parity_config_shapes():
    _parity(2, 6, 256, 64, seed=1)      # char-level GPT heads, reduced batch
    _parity(8, 12, 128, 32, seed=2)     # narrow heads, T=128
    _parity(8, 12, 256, 32, seed=3)     # narrow heads, T=256


def test_fwd_parity_full_size_sampled():
    _parity(12, 12, 1024, 64, 11, qkv_scale=0.5, slices=[(0, 0), (7, 3), (11, 11)])
    _parity(12, 12, 1024, 64, 11, qkv_scale=2.0, rel=2.0 ** -8, slices=[(0, 0), (5, 9), (11, 11)])
    _parity(12, 25, 1024, 64, 12, slices=[(0, 0), (6, 13), (11, 24)])
    _parity(64, 6, 256, 64, 13, slices=[(0, 0), (40, 2), (63, 5)])


def _dev_inputs(B, H, T, hs, seed):
    x = inputs(B, H, T, hs, "bf16", seed=seed, workload="meta")
    return x, {n: to_dev(a, "bf16") for n, a in x.items()}


@pytest.mark.parametrize("hs", [64, 32])
def test_fwd_causality_bit_exact(hs):
    """Changing rows > i of q, k, v leaves rows <= i of o and lse bit-identical
    (masked terms are exact zeros)."""
    import torch
    T = 300
    x, t = _dev_inputs(2, 3, T, hs, 21)
    s = default_scale(hs)
    o0, l0 = fwd(t["q"], t["k"], t["v"], s)
    for i in (0, 63, 64, 130, 299):
        pert = {n: t[n].clone() for n in ("q", "k", "v")}
        for n in pert:
            pert[n][:, :, i + 1:] = pert[n][:, :, i + 1:] * 3.0 + 1.0
        o1, l1 = fwd(pert["q"], pert["k"], pert["v"], s)
        assert torch.equal(o0[:, :, :i + 1], o1[:, :, :i + 1]), i
        assert torch.equal(l0[:, :, :i + 1], l1[:, :, :i + 1]), i


def test_fwd_value_scaling_exact():
    """V x 2 gives O x 2 exactly (power-of-two scaling commutes with every
    rounding); Q x 2 with K x 1/2 gives identical O and lse."""
    import torch
    x, t = _dev_inputs(2, 4, 333, 64, 22)
    s = default_scale(64)
    o0, l0 = fwd(t["q"], t["k"], t["v"], s)
    o1, l1 = fwd(t["q"], t["k"], t["v"] * 2, s)
    assert torch.equal(o1, o0 * 2)
    assert torch.equal(l1, l0)
    o2, l2 = fwd(t["q"] * 2, t["k"] * 0.5, t["v"], s)
    assert torch.equal(o2, o0)
    assert torch.equal(l2, l0)


def test_fwd_deterministic_and_lse_optional():
    import torch
    x, t = _dev_inputs(3, 5, 700, 64, 23)
    s = default_scale(64)
    a, la = fwd(t["q"], t["k"], t["v"], s)
    b, lb = fwd(t["q"], t["k"], t["v"], s)
    c, _ = fwd(t["q"], t["k"], t["v"], s, lse=False)
    assert torch.equal(a, b) and torch.equal(la, lb) and torch.equal(a, c)
    assert not torch.isnan(a).any() and not torch.isnan(la).any()


def test_fwd_heads_split_bit_identical():
    """25 heads in one call equal 25 single-head calls bit for bit."""
    import torch
    x, t = _dev_inputs(2, 25, 260, 64, 24)
    s = default_scale(64)
    o, l = fwd(t["q"], t["k"], t["v"], s)
    for h in range(25):
        sl = lambda a: a[:, h:h + 1].contiguous()
        oh, lh = fwd(sl(t["q"]), sl(t["k"]), sl(t["v"]), s)
        assert torch.equal(oh, o[:, h:h + 1]) and torch.equal(lh, l[:, h:h + 1]), h


def test_fwd_guard_bands_untouched():
    """Outputs written exactly in place: sentinels around o and lse survive."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs = 2, 3, 201, 64
    x, t = _dev_inputs(B, H, T, hs, 25)
    n = B * H * T * hs
    pad = 4096
    obuf = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * T + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + n].view(B, H, T, hs)
    l = lbuf[pad:pad + B * H * T].view(B, H, T)
    ga.gattn_fwd(t["q"], t["k"], t["v"], o, l, default_scale(hs))
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 7.0) and torch.all(obuf[pad + n:] == 7.0)
    assert torch.all(lbuf[:pad] == 7.0) and torch.all(lbuf[pad + B * H * T:] == 7.0)
    ref, _ = fwd(t["q"], t["k"], t["v"], default_scale(hs))
    assert torch.equal(o, ref)
