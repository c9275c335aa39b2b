"""GPU: attention dropout (gattn_fwd_dropout, gattn_bwd_dropout,
gattn_dropout_mask) against the float64 oracle of oracle/dropout.py with the
same seed and offset.

The keep decisions are integers, so they are compared exactly: the mask
kernel against the oracle's mask, and each attention kernel's own decisions
read out of its outputs with one-hot inputs (uniform weights from q = 0 or
k = 0, one-hot v, dO, k or q on a window of 64 rows), where a dropped weight
gives an exact zero (o, dv) or the other of two well separated values (dq,
dk).  The outputs on random inputs are then held to the bars of the path
without dropout: bf16 2e-2 + 2^-8 |ref| at unit variance, and the first-order
rounding bound of gpu_util.rounding_bound with the dropout multipliers (u =
2^-8 for bf16, 2^-11 for fp16); float32 1e-4.
"""
import numpy as np
import pytest

from gpu_util import (U_F16, check_bound, check_close, default_scale, inputs, pick,
                      rounding_bound, to_dev, torch_dtype)

pytestmark = pytest.mark.gpu

BF16_TOL, BF16_REL, F32_TOL = 2e-2, 2.0 ** -8, 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_self_attention_sdpa_amd as ga
    ga.load_library()


def _gpu_run(x, dtype, s, p, seed, off):
    """gattn_fwd_dropout then gattn_bwd_dropout; float64 (dq, dk, dv, o, lse)."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    t = {n: to_dev(a, dtype) for n, a in x.items()}
    o, lse = ga.attention_forward_dropout(t["q"], t["k"], t["v"], p, seed, off, scale=s)
    dq, dk, dv = ga.attention_backward_dropout(t["q"], t["k"], t["v"], o, t["do"], lse, p, seed,
                                               off, scale=s)
    torch.cuda.synchronize()
    return tuple(a.float().cpu().numpy().astype(np.float64) for a in (dq, dk, dv, o, lse))


def _oracle(x, s, p, seed, off, slices):
    from oracle import dropout as od
    r = od.attention_backward_dropout(x["q"], x["k"], x["v"], x["do"], s, p, seed, off,
                                      slices=slices)
    return tuple(a[:, None] for a in r)


def _z(x, p, seed, off, slices):
    from oracle import dropout as od
    B, H, T, _ = x["q"].shape
    m = od.keep_mask(B, H, T, p, seed, off, slices)
    return np.stack([m[bh] for bh in slices]) * od.keep_scale(p)


def _check(dtype, B, H, T, hs, p, slices=None, seed=0xC0FFEE, off=3, qkv_scale=1.0,
           stated_bar=True):
    x = inputs(B, H, T, hs, dtype, seed=101, workload="dropout", qkv_scale=qkv_scale)
    s = default_scale(hs)
    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    print(f"case dropout {dtype} B={B} H={H} T={T} hs={hs} p={p} slices={len(slices)}", flush=True)
    got = pick(_gpu_run(x, dtype, s, p, seed, off), slices)
    ref = _oracle(x, s, p, seed, off, slices)
    where = f"dropout {dtype} {(B, H, T, hs)} p={p}"
    if dtype == "f32":
        return check_close(got, ref, F32_TOL, where=where)
    if dtype == "bf16" and stated_bar:
        check_close(got, ref, BF16_TOL, BF16_REL, where=where)
    u, slack = (U_F16, 2e-4) if dtype == "f16" else (2.0 ** -8, 1e-3)
    bound = rounding_bound(x, s, slices, ref, u=u, slack=slack, z=_z(x, p, seed, off, slices))
    return check_bound(got, ref, bound, where=where)


# ------------------------------------------------------------ parity, random

@pytest.mark.parametrize("hs", [64, 32])
@pytest.mark.parametrize("T", [1, 17, 64, 65, 129, 200, 257])
def test_dropout_ragged_lengths(T, hs):
    _check("bf16", 2, 3, T, hs, 0.1)


@pytest.mark.parametrize("p", [0.5, 0.9])
def test_dropout_high_probability(p):
    _check("bf16", 2, 3, 190, 64, p, stated_bar=False)


def test_dropout_gpt2_small_shape():
    """B=12, H=12, T=1024, hs=64, p=0.1 (launch configuration of the bench),
    sampled slices."""
    _check("bf16", 12, 12, 1024, 64, 0.1, slices=[(0, 0), (5, 7), (11, 11)], qkv_scale=0.5)


def test_dropout_robgpt_shape():
    """The RobGPT model's attention (12 heads of 32, 256 tokens, dropout 0.1),
    batch 8, every slice."""
    _check("bf16", 8, 12, 256, 32, 0.1)


@pytest.mark.parametrize("T,hs", [(100, 64), (300, 32)])
def test_dropout_f16(T, hs):
    _check("f16", 2, 3, T, hs, 0.1)


@pytest.mark.parametrize("T,hs", [(1, 8), (8, 8), (45, 24)])
def test_dropout_f32(T, hs):
    _check("f32", 2, 3, T, hs, 0.2)


# ------------------------------------------------------- keep decisions, exact

def test_mask_kernel_equals_oracle():
    import torch
    import causal_self_attention_sdpa_amd as ga
    from oracle import dropout as od
    for (B, H, T, p, seed, off) in [(2, 3, 203, 0.1, 5, 0), (1, 2, 64, 0.5, 2**63 + 11, 7),
                                    (12, 12, 1024, 0.1, 1234, 42)]:
        keep = torch.empty((B, H, T, T), dtype=torch.uint8, device="cuda")
        ga.gattn_dropout_mask(keep, B, H, T, p, seed, off)
        torch.cuda.synchronize()
        sl = [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
        ref = od.keep_mask(B, H, T, p, seed, off, sl)
        for b, h in sl:
            assert np.array_equal(keep[b, h].cpu().numpy().astype(bool), ref[(b, h)]), (B, H, T, b, h)


def _onehot_window(T, hs, start):
    a = np.zeros((T, hs))
    n = min(hs, T - start)
    a[start:start + n, :n] = np.eye(n)
    return a


def _mask_ref(B, H, T, p, seed, off):
    from oracle import dropout as od
    return od.keep_mask(B, H, T, p, seed, off)


@pytest.mark.parametrize("T,win", [(300, 0), (300, 236), (1024, 960)])
def test_forward_keep_decisions_exact(T, win):
    """q = 0 (uniform weights), v one-hot on keys win..win+63: o[i][d] is 0
    exactly when weight (i, win + d) is dropped or lies above the diagonal."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, hs, p, seed, off = 2, 3, 64, 0.3, 77, 1
    q = torch.zeros((B, H, T, hs), dtype=torch.bfloat16, device="cuda")
    k = to_dev(inputs(B, H, T, hs, "bf16", seed=102, workload="dropout-mask")["k"], "bf16")
    v = to_dev(np.broadcast_to(_onehot_window(T, hs, win), (B, H, T, hs)), "bf16")
    o, _ = ga.attention_forward_dropout(q, k, v, p, seed, off, need_lse=False)
    kept = _mask_ref(B, H, T, p, seed, off)[:, :, :, win:win + hs]
    n = kept.shape[-1]
    vis = (win + np.arange(n))[None, :] <= np.arange(T)[:, None]
    got_nz = o.float().cpu().numpy()[..., :n] != 0
    assert np.array_equal(got_nz, kept & vis)


def _grad_setup(B, H, T, hs, which, win):
    """Inputs for reading the backward kernels' keep decisions (weights
    uniform, dO V^T = 2 everywhere):
      which = "dq": q = 0, k one-hot on keys win..: dq[i][d] = s dS[i][win+d];
      which = "dk": k = 0, q one-hot on queries win..: dk[j][d] = s dS[win+d][j];
      which = "dv": q = 0, dO one-hot on queries win..: dv[j][d] = (P Z)[win+d][j]."""
    x = inputs(B, H, T, hs, "bf16", seed=103, workload="dropout-grad")
    e0 = np.zeros((T, hs))
    e0[:, 0] = 1.0
    oh = np.broadcast_to(_onehot_window(T, hs, win), (B, H, T, hs))
    if which == "dq":
        return dict(q=np.zeros_like(x["q"]), k=oh, v=np.broadcast_to(e0, x["v"].shape),
                    do=np.broadcast_to(2 * e0, x["do"].shape))
    if which == "dk":
        return dict(q=oh, k=np.zeros_like(x["k"]), v=np.broadcast_to(e0, x["v"].shape),
                    do=np.broadcast_to(2 * e0, x["do"].shape))
    return dict(q=np.zeros_like(x["q"]), k=x["k"], v=x["v"], do=oh)


@pytest.mark.parametrize("which", ["dq", "dk", "dv"])
@pytest.mark.parametrize("T,win", [(300, 0), (300, 236), (1024, 960)])
def test_backward_keep_decisions_exact(which, T, win):
    from oracle import dropout as od
    B, H, hs, p, seed, off, s = 2, 3, 64, 0.3, 91, 5, 0.125
    x = _grad_setup(B, H, T, hs, which, win)
    print(f"case dropout keep read-out {which} T={T} win={win}", flush=True)
    dq, dk, dv, o, lse = _gpu_run(x, "bf16", s, p, seed, off)
    kept = _mask_ref(B, H, T, p, seed, off)
    zs = od.keep_scale(p)
    n = min(hs, T - win)
    i = np.arange(T)
    if which == "dv":
        # dv[j][d] = P[win+d][j] Z[win+d][j]: zero exactly when dropped or j > win + d
        ref = np.swapaxes(kept[:, :, win:win + n, :], 2, 3)   # (B, H, T_j, n)
        vis = i[:, None] <= (win + np.arange(n))[None, :]
        assert np.array_equal(dv[..., :n] != 0, ref & vis)
        return
    # dS = P (Z dP - D) with P = 1/(row+1), dP = 2, D from the kept count of the
    # row: kept gives P (2 zs - D), dropped -P D; classify by the midpoint.
    cnt = np.cumsum(kept, axis=-1)[..., i, i]                  # kept keys j <= i of row i
    D = 2 * zs * cnt / (i + 1)                                 # (B, H, T)
    if which == "dq":
        val = dq[..., :n] / s                                  # (B, H, T_i, n): dS[i][win+d]
        rows = np.broadcast_to(i[:, None], (T, n))
        cols = win + np.arange(n)[None, :]
        Drow = D[..., :, None]
        ref = kept[:, :, :, win:win + n]
    else:
        val = np.swapaxes(dk[..., :n] / s, 2, 3)               # (B, H, n, T_j): dS[win+d][j]
        rows = np.broadcast_to((win + np.arange(n))[:, None], (n, T))
        cols = i[None, :]
        Drow = D[..., win:win + n, None]
        ref = kept[:, :, win:win + n, :]
    vis = cols <= rows
    mid = (zs - Drow) / (rows + 1)                             # P (zs dP/2 - D), dP = 2
    got = val > mid
    assert np.array_equal(got & vis, ref & vis)
    assert np.all(val[..., ~vis] == 0)


# ---------------------------------------------------------------- properties

def test_p0_is_the_plain_path_bitwise():
    import torch
    import causal_self_attention_sdpa_amd as ga
    from gpu_util import gpu_fwd_bwd
    B, H, T, hs = 2, 3, 150, 64
    x = inputs(B, H, T, hs, "bf16", seed=104, workload="dropout-p0")
    s = default_scale(hs)
    got = _gpu_run(x, "bf16", s, 0.0, 5, 5)
    ref = gpu_fwd_bwd(x, "bf16", s)
    for n, a, b in zip(("dq", "dk", "dv", "o", "lse"), got, ref):
        assert np.array_equal(a, b), n


def test_same_seed_reproduces_other_offsets_differ():
    B, H, T, hs = 2, 2, 200, 64
    x = inputs(B, H, T, hs, "bf16", seed=105, workload="dropout-det")
    s = default_scale(hs)
    a = _gpu_run(x, "bf16", s, 0.1, 9, 1)
    b = _gpu_run(x, "bf16", s, 0.1, 9, 1)
    c = _gpu_run(x, "bf16", s, 0.1, 9, 2)
    for n in range(5):
        assert np.array_equal(a[n], b[n])
    assert not np.array_equal(a[3], c[3])
    assert np.array_equal(a[4], c[4])  # lse is that of the softmax before dropout


def test_fused_qkv_layout_equals_contiguous_bitwise():
    """Dropout through strided (B, T, 3C) / (B, T, C) views gives the same bits
    as the contiguous call."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs, p = 2, 4, 160, 64, 0.1
    x = inputs(B, H, T, hs, "bf16", seed=106, workload="dropout-fused")
    s = default_scale(hs)
    C = H * hs
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)
    qkv = dev(np.concatenate([x[n].transpose(0, 2, 1, 3).reshape(B, T, C)
                              for n in ("q", "k", "v")], axis=2))
    dy = dev(x["do"].transpose(0, 2, 1, 3).reshape(B, T, C))
    v4 = qkv.view(B, T, 3, H, hs)
    q, k, v = (v4[:, :, j].transpose(1, 2) for j in range(3))
    y = torch.empty((B, T, C), dtype=torch.bfloat16, device="cuda")
    y4 = y.view(B, T, H, hs).transpose(1, 2)
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    ga.gattn_fwd_dropout(q, k, v, y4, lse, s, p, 21, 4)
    dqkv = torch.empty_like(qkv)
    g4 = dqkv.view(B, T, 3, H, hs)
    ws = torch.empty(ga.gattn_bwd_workspace_bytes(B, H, T, hs, ga.BF16), dtype=torch.uint8,
                     device="cuda")
    ga.gattn_bwd_dropout(q, k, v, y4, dy.view(B, T, H, hs).transpose(1, 2), lse,
                         *(g4[:, :, j].transpose(1, 2) for j in range(3)), s, p, 21, 4, ws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    got = (f(g4[:, :, 0].transpose(1, 2)), f(g4[:, :, 1].transpose(1, 2)),
           f(g4[:, :, 2].transpose(1, 2)), f(y4), f(lse))
    ref = _gpu_run(x, "bf16", s, p, 21, 4)
    for n, a, b in zip(("dq", "dk", "dv", "o", "lse"), got, ref):
        assert np.array_equal(a, b), n
