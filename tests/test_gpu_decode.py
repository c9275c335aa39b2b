"""GPU: the forward of the newest Tq tokens against Tk >= Tq keys
(gattn_fwd_decode), and the pages' generate pattern (the whole forward
recomputed at every prefix length, lse not needed).

Bars: bf16 as the forward, 2e-2 + 2^-8 |ref| on o and 1e-3 on lse; fp16 the
first-order rounding bound of the output, u (|o| + sum_j p_ij |v_j|) + 2e-4
with u = 2^-11 (P is rounded to fp16 as an MFMA operand, o once when stored),
and 2e-4 on lse; float32 1e-4.
"""
import math

import numpy as np
import pytest

from gpu_util import check_close, default_scale, inputs, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

BF16_TOL, BF16_REL, LSE_BF16 = 2e-2, 2.0 ** -8, 1e-3
U_F16, F16_SLACK = 2.0 ** -11, 2e-4
F32_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_self_attention_sdpa_amd as ga
    ga.load_library()


def _kv_inputs(B, H, Tq, Tk, hs, dtype, seed):
    """q of the newest Tq tokens (the last Tq query rows of a Tk-token draw), k, v of all Tk."""
    x = inputs(B, H, Tk, hs, dtype, seed=seed, workload="decode")
    return x["q"][:, :, Tk - Tq:], x["k"], x["v"]


def _oracle(q, k, v, s):
    import oracle
    return oracle.attention_forward_kv(q, k, v, s)


def _f16_bound(q, k, v, s, o_ref, lse_ref):
    Tq, Tk = q.shape[2], k.shape[2]
    sc = np.einsum("bhid,bhjd->bhij", q, k) * s
    vis = np.arange(Tk)[None, :] <= (Tk - Tq + np.arange(Tq))[:, None]
    p = np.where(vis, np.exp(np.where(vis, sc, 0.0) - lse_ref[..., None]), 0.0)
    mag = np.einsum("bhij,bhjd->bhid", p, np.abs(v))
    return U_F16 * (np.abs(o_ref) + mag) + F16_SLACK


def _run(q, k, v, dtype, s, need_lse=True):
    import torch
    import causal_self_attention_sdpa_amd as ga
    tq, tk, tv = (to_dev(a, dtype) for a in (q, k, v))
    o, lse = ga.attention_decode(tq, tk, tv, s, need_lse=need_lse)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    return o, (lse.cpu().numpy().astype(np.float64) if lse is not None else None)


def _check(dtype, B, H, Tq, Tk, hs, seed=91):
    q, k, v = _kv_inputs(B, H, Tq, Tk, hs, dtype, seed)
    s = default_scale(hs)
    print(f"case decode {dtype} B={B} H={H} Tq={Tq} Tk={Tk} hs={hs}", flush=True)
    o, lse = _run(q, k, v, dtype, s)
    o_ref, lse_ref = _oracle(q, k, v, s)
    where = f"decode {dtype} {(B, H, Tq, Tk, hs)}"
    if dtype == "bf16":
        check_close((o,), (o_ref,), BF16_TOL, BF16_REL, names=("o",), where=where)
        check_close((lse,), (lse_ref,), LSE_BF16, names=("lse",), where=where)
    elif dtype == "f16":
        b = _f16_bound(q, k, v, s, o_ref, lse_ref)
        assert np.all(np.abs(o - o_ref) <= b), f"{where} o: worst ratio {np.max(np.abs(o - o_ref) / b)}"
        check_close((lse,), (lse_ref,), F16_SLACK, names=("lse",), where=where)
    else:
        check_close((o, lse), (o_ref, lse_ref), F32_TOL, names=("o", "lse"), where=where)


@pytest.mark.parametrize("hs", [64, 32])
@pytest.mark.parametrize("Tk", [1, 2, 63, 64, 65, 127, 200, 1024])
def test_decode_single_token(Tk, hs):
    _check("bf16", 2, 3, 1, Tk, hs)


@pytest.mark.parametrize("Tq,Tk", [(2, 2), (2, 9), (31, 31), (32, 40), (33, 100), (100, 100),
                                   (100, 290), (5, 1024)])
def test_decode_several_queries(Tq, Tk):
    _check("bf16", 2, 2, Tq, Tk, 64)


def test_decode_gpt2_small_shape():
    """One decode step of the GPT-2 124M shape: B=12, H=12, one new token, 1024 keys."""
    _check("bf16", 12, 12, 1, 1024, 64)


@pytest.mark.parametrize("Tq,Tk,hs", [(1, 300, 64), (7, 130, 32), (64, 64, 64)])
def test_decode_f16(Tq, Tk, hs):
    _check("f16", 2, 3, Tq, Tk, hs)


@pytest.mark.parametrize("Tq,Tk,hs", [(1, 40, 8), (3, 17, 24), (40, 40, 16)])
def test_decode_f32(Tq, Tk, hs):
    _check("f32", 2, 3, Tq, Tk, hs)


@pytest.mark.parametrize("Tq,Tk", [(4, 150), (1, 150), (1, 1000), (4, 1000)])
def test_decode_from_a_cache_view(Tq, Tk):
    """k, v as the first Tk rows of a (B, H, Tmax, hs) cache whose other rows
    hold NaN, q read from (B, Tq, H, hs) and o written into (B, Tq, H, hs + 8)
    with NaN poison: same values as the contiguous call, padding untouched.
    Tq = 1 runs the one-token kernel, Tq = 4 the MFMA kernel; Tk = 1000 splits
    the key range (a merge launch and the workspace)."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, Tmax, hs = 2, 3, 1024, 64
    print(f"case decode cache view Tq={Tq} Tk={Tk}", flush=True)
    q, k, v = _kv_inputs(B, H, Tq, Tk, hs, "bf16", 92)
    s = default_scale(hs)
    dt = torch.bfloat16
    kc = torch.full((B, H, Tmax, hs), float("nan"), dtype=dt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kc[:, :, :Tk] = to_dev(k, "bf16")
    vc[:, :, :Tk] = to_dev(v, "bf16")
    qb = to_dev(q.transpose(0, 2, 1, 3), "bf16").transpose(1, 2)  # (B, H, Tq, hs) view of (B, Tq, H, hs)
    ob = torch.full((B, Tq, H, hs + 8), float("nan"), dtype=dt, device="cuda")
    ov = ob[..., :hs].transpose(1, 2)
    ga.gattn_fwd_decode(qb, kc[:, :, :Tk], vc[:, :, :Tk], ov, None, s)
    torch.cuda.synchronize()
    assert torch.isnan(ob[..., hs:]).all(), "padding written"
    got = ov.float().cpu().numpy().astype(np.float64)
    ref, _ = _run(q, k, v, "bf16", s, need_lse=False)
    assert np.array_equal(got, ref)


def test_decode_matches_last_rows_of_forward():
    """The newest-Tq forward equals the last Tq rows of the causal forward over
    all Tk tokens (the pages' generate), within the bf16 bar."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs = 2, 4, 333, 64
    x = inputs(B, H, T, hs, "bf16", seed=93, workload="decode-vs-fwd")
    s = default_scale(hs)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    o_full, lse_full = ga.attention_forward(q, k, v, s)
    for Tq in (1, 17, 64):
        o, lse = ga.attention_decode(q[:, :, T - Tq:], k, v, s, need_lse=True)
        torch.cuda.synchronize()
        check_close((o.float().cpu().numpy(), lse.cpu().numpy()),
                    (o_full[:, :, T - Tq:].float().cpu().numpy(),
                     lse_full[:, :, T - Tq:].cpu().numpy()), BF16_TOL, BF16_REL,
                    names=("o", "lse"), where=f"decode Tq={Tq} vs forward")


def test_generate_every_prefix_length():
    """The pages' generate: the whole forward at every prefix length T = 1..256
    (B=1, 6 heads, hs 64: the character-level model's block size), without lse.
    Row i depends only on rows <= i and each row's arithmetic does not depend
    on T, so every prefix output equals the leading rows of the full forward
    bit for bit; a few prefix lengths are also checked against the oracle."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    import oracle
    B, H, Tmax, hs = 1, 6, 256, 64
    x = inputs(B, H, Tmax, hs, "bf16", seed=94, workload="generate")
    s = default_scale(hs)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    full, _ = ga.attention_forward(q, k, v, s, need_lse=False)
    full = full.float().cpu().numpy()
    for T in range(1, Tmax + 1):
        o = torch.empty((B, H, T, hs), dtype=torch.bfloat16, device="cuda")
        ga.gattn_fwd(q[:, :, :T].contiguous(), k[:, :, :T].contiguous(), v[:, :, :T].contiguous(),
                     o, None, s)
        got = o.float().cpu().numpy()
        assert np.array_equal(got, full[:, :, :T]), f"prefix {T} differs from the full forward"
        if T in (1, 2, 31, 100, 256):
            ref, _ = oracle.attention_forward(x["q"][:, :, :T], x["k"][:, :, :T], x["v"][:, :, :T], s)
            check_close((got,), (ref,), BF16_TOL, BF16_REL, names=("o",), where=f"generate T={T}")
