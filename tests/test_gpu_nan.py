"""NaN inputs reach the outputs that depend on them (16-bit and float32 paths).

The pages say nothing about non-finite inputs; the reading taken is that the
kernels do not sanitise them: IEEE arithmetic carries a NaN in a key, value or
incoming-gradient row into every result that mathematically depends on it.
A NaN key row j makes the scores S[i][j] of every query i >= j NaN, hence the
whole row i of o and lse[i]; a NaN value row j makes o[i] NaN for i >= j.  In
the backward a NaN row i of dO makes dq[i] NaN and reaches dk and dv of every
key j <= i.  Rows that never meet the NaN stay finite: every query row before
the 32-row block holding j (masked weights are exact zeros, but a masked
weight times a NaN value inside that block's MFMA is NaN, so rows of the same
block before j are not specified), and every other (b, h) slice.
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


def _run(x, dtype, scale):
    import torch
    import causal_self_attention_sdpa_amd as ga
    t = {n: to_dev(a, dtype) for n, a in x.items()}
    o, lse = ga.attention_forward(t["q"], t["k"], t["v"], scale)
    dq, dk, dv = ga.attention_backward(t["q"], t["k"], t["v"], o, t["do"], lse, scale)
    torch.cuda.synchronize()
    return [a.float().cpu().numpy() for a in (o, lse, dq, dk, dv)]


def _rows_nan(a, b, h, rows):
    r = a[b, h, rows]
    return np.isnan(r.reshape(len(rows), -1)).all(axis=1).all()


def _finite_except(a, b, h, rows_finite):
    """Every slice but (b, h) finite, and rows_finite of (b, h) finite."""
    m = np.ones(a.shape[:2], dtype=bool)
    m[b, h] = False
    return np.isfinite(a[m]).all() and np.isfinite(a[b, h, rows_finite]).all()


@pytest.mark.parametrize("dtype,hs", [("bf16", 64), ("bf16", 32), ("f16", 64), ("f32", 16)])
@pytest.mark.parametrize("j", [0, 70, 199])
def test_nan_key_row(dtype, hs, j):
    B, H, T = 2, 2, 200
    x = inputs(B, H, T, hs, dtype, seed=90 + j)
    x["k"][1, 0, j, 3] = np.nan
    print(f"case nan key dtype={dtype} hs={hs} j={j}", flush=True)
    o, lse, dq, dk, dv = _run(x, dtype, default_scale(hs))
    after = np.arange(j, T)
    before = np.arange(0, 32 * (j // 32))
    assert _rows_nan(o, 1, 0, after) and np.isnan(lse[1, 0, j:]).all()
    assert _finite_except(o, 1, 0, before) and _finite_except(lse, 1, 0, before)
    assert np.isnan(dq[1, 0, j:]).any(axis=-1).all()
    for g in (dq, dk, dv):
        assert _finite_except(g, 1, 0, np.arange(0, 0))


@pytest.mark.parametrize("dtype,hs", [("bf16", 64), ("f16", 32), ("f32", 16)])
@pytest.mark.parametrize("j", [5, 130])
def test_nan_value_row(dtype, hs, j):
    B, H, T = 2, 2, 200
    x = inputs(B, H, T, hs, dtype, seed=95 + j)
    x["v"][0, 1, j, :] = np.nan
    print(f"case nan value dtype={dtype} hs={hs} j={j}", flush=True)
    o, lse, dq, dk, dv = _run(x, dtype, default_scale(hs))
    assert _rows_nan(o, 0, 1, np.arange(j, T))
    assert _finite_except(o, 0, 1, np.arange(0, 32 * (j // 32)))
    assert np.isfinite(lse).all()


@pytest.mark.parametrize("dtype,hs", [("bf16", 64), ("f16", 64), ("f32", 16)])
def test_nan_grad_row(dtype, hs):
    B, H, T, i = 1, 3, 150, 100
    x = inputs(B, H, T, hs, dtype, seed=97)
    x["do"][0, 2, i, :] = np.nan
    print(f"case nan dO dtype={dtype} hs={hs} i={i}", flush=True)
    o, lse, dq, dk, dv = _run(x, dtype, default_scale(hs))
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert np.isnan(dq[0, 2, i]).all()
    assert np.isnan(dv[0, 2, :i + 1]).any(axis=-1).all()
    assert np.isnan(dk[0, 2, :i + 1]).any(axis=-1).all()
    for g in (dq, dk, dv):
        assert np.isfinite(g[0, :2]).all()
    assert np.isfinite(dq[0, 2, :32 * (i // 32)]).all()
    assert np.isfinite(dk[0, 2, 64 * ((i + 64) // 64):]).all()
    assert np.isfinite(dv[0, 2, 64 * ((i + 64) // 64):]).all()
