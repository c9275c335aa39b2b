"""GPU: the strided entry points (gattn_fwd_strided, gattn_bwd_strided) and
the fused-projection helpers built on them.

The attention of a GPT block reads q, k, v from the (B, T, 3C) output of one
projection and hands (B, T, C) to the output projection.  The strided entry
points read and write those layouts in place.  Checks:
  * the same kernels run, only the addressing differs, so every output is
    bit-identical to the contiguous entry points on the same values;
  * against the oracle, to the bars of the contiguous path (bf16 2e-2 +
    2^-8 |ref|, float32 1e-4);
  * nothing outside the addressed rows is written (padded rows keep their
    NaN poison) and every addressed element is written, ragged T included.
"""
import numpy as np
import pytest

from gpu_util import (check_close, default_scale, gpu_fwd_bwd, inputs, oracle_slices, pick,
                      to_dev, torch_dtype)

pytestmark = pytest.mark.gpu

BF16_TOL, BF16_REL, F32_TOL = 2e-2, 2.0 ** -8, 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_self_attention_sdpa_amd as ga
    ga.load_library()


def _fused(x, dtype):
    """(B, T, 3C) projection output holding q, k, v of x (heads side by side),
    and the (B, T, C) incoming gradient holding dO."""
    import torch
    B, H, T, hs = x["q"].shape
    qkv = np.concatenate([x[n].transpose(0, 2, 1, 3).reshape(B, T, H * hs)
                          for n in ("q", "k", "v")], axis=2)
    dy = x["do"].transpose(0, 2, 1, 3).reshape(B, T, H * hs)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch_dtype(dtype))
    return dev(qkv), dev(dy)


def _split_bthc(a: np.ndarray, H: int, parts: int):
    """(B, T, parts*C) -> `parts` arrays (B, H, T, hs)."""
    B, T, W = a.shape
    hs = W // (parts * H)
    r = a.reshape(B, T, parts, H, hs).transpose(2, 0, 3, 1, 4)
    return [r[j] for j in range(parts)]


@pytest.mark.parametrize("dtype,B,H,T,hs", [
    ("bf16", 2, 12, 256, 64),
    ("bf16", 3, 4, 200, 32),
    ("bf16", 1, 3, 77, 64),
    ("bf16", 3, 87, 70, 64),  # 261 heads: the grid pads them to 264
    ("f32", 2, 3, 40, 24),
])
def test_fused_qkv_matches_contiguous_bitwise_and_oracle(dtype, B, H, T, hs):
    import torch
    import causal_self_attention_sdpa_amd as ga
    x = inputs(B, H, T, hs, dtype, seed=71, workload="strided")
    s = default_scale(hs)
    print(f"case {dtype} fused qkv B={B} H={H} T={T} hs={hs}", flush=True)
    qkv, dy = _fused(x, dtype)
    y, lse = ga.attention_forward_qkv(qkv, H, s)
    dqkv = ga.attention_backward_qkv(qkv, y, dy, lse, H, s)
    torch.cuda.synchronize()
    got_o = _split_bthc(y.float().cpu().numpy().astype(np.float64), H, 1)[0]
    gq, gk, gv = _split_bthc(dqkv.float().cpu().numpy().astype(np.float64), H, 3)
    got = (gq, gk, gv, got_o, lse.cpu().numpy().astype(np.float64))
    # bit-identical to the contiguous entry points on the same values
    ref_c = gpu_fwd_bwd(x, dtype, s)
    for n, a, b in zip(("dq", "dk", "dv", "o", "lse"), got, ref_c):
        assert np.array_equal(a, b), f"{n} differs from the contiguous path"
    # and to the oracle
    import oracle
    ref = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], s)
    if dtype == "bf16":
        check_close(got, ref, BF16_TOL, BF16_REL, where=f"fused {dtype} {(B, H, T, hs)}")
    else:
        check_close(got, ref, F32_TOL, where=f"fused {dtype} {(B, H, T, hs)}")


@pytest.mark.parametrize("dtype,hs", [("bf16", 64), ("bf16", 32), ("f32", 16)])
def test_padded_rows_untouched_and_every_row_written(dtype, hs):
    """Outputs in (B, T, H, hs + pad) buffers with NaN poison: the padding keeps
    its poison, every addressed element is written, values equal the
    contiguous path.  Inputs come from (B, H, T + gap, hs) buffers read with a
    row stride and a head stride that skip rows."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T = 2, 5, 131
    pad = 8 if dtype == "bf16" else 4
    gap = 3
    x = inputs(B, H, T, hs, dtype, seed=72, workload="padded")
    s = default_scale(hs)
    tdt = torch_dtype(dtype)
    print(f"case {dtype} padded layouts B={B} H={H} T={T} hs={hs}", flush=True)

    def holder(a):  # (B, H, T + gap, hs) buffer, rows 0..T-1 hold the values
        buf = torch.full((B, H, T + gap, hs), float("nan"), dtype=tdt, device="cuda")
        buf[:, :, :T] = torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(tdt)
        return buf[:, :, :T]

    def out_buf():  # (B, T, H, hs + pad) poisoned buffer and its (B, H, T, hs) view
        buf = torch.full((B, T, H, hs + pad), float("nan"), dtype=tdt, device="cuda")
        return buf, buf[..., :hs].transpose(1, 2)

    q, k, v, do = (holder(x[n]) for n in ("q", "k", "v", "do"))
    ob, o = out_buf()
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    ga.gattn_fwd_strided(q, k, v, o, lse, s)
    # dO shares the layout of o: copy it into a poisoned (B, T, H, hs + pad) buffer
    gb, dO = out_buf()
    dO.copy_(torch.from_numpy(np.ascontiguousarray(x["do"])).to("cuda").to(tdt))
    bufs = [out_buf() for _ in range(3)]
    ws = torch.empty(ga.gattn_bwd_workspace_bytes(B, H, T, hs, ga.BF16 if dtype == "bf16" else ga.F32),
                     dtype=torch.uint8, device="cuda")
    ga.gattn_bwd_strided(q, k, v, o, dO, lse, *(b[1] for b in bufs), s, ws)
    torch.cuda.synchronize()
    for name, (buf, view) in zip(("o", "dq", "dk", "dv"), [(ob, o)] + bufs):
        assert torch.isnan(buf[..., hs:]).all(), f"{name}: padding was written"
        assert not torch.isnan(view).any(), f"{name}: an addressed element was not written"
    got = tuple(t.float().cpu().numpy().astype(np.float64)
                for t in (bufs[0][1], bufs[1][1], bufs[2][1], o, lse))
    ref_c = gpu_fwd_bwd(x, dtype, s)
    for n, a, b in zip(("dq", "dk", "dv", "o", "lse"), got, ref_c):
        assert np.array_equal(a, b), f"{n} differs from the contiguous path"


def test_fused_qkv_gpt2_small_shape_sampled():
    """B=12, H=12, T=1024, hs=64 through the fused-projection helpers (the
    launch configuration of a GPT-2 124M block), sampled slices against the
    oracle."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs = 12, 12, 1024, 64
    x = inputs(B, H, T, hs, "bf16", seed=73, workload="strided-gpt2", qkv_scale=0.5)
    s = default_scale(hs)
    print(f"case bf16 fused qkv B={B} H={H} T={T} hs={hs}", flush=True)
    qkv, dy = _fused(x, "bf16")
    y, lse = ga.attention_forward_qkv(qkv, H, s)
    dqkv = ga.attention_backward_qkv(qkv, y, dy, lse, H, s)
    torch.cuda.synchronize()
    got_o = _split_bthc(y.float().cpu().numpy().astype(np.float64), H, 1)[0]
    gq, gk, gv = _split_bthc(dqkv.float().cpu().numpy().astype(np.float64), H, 3)
    got = (gq, gk, gv, got_o, lse.cpu().numpy().astype(np.float64))
    sl = [(0, 0), (7, 5), (11, 11)]
    check_close(pick(got, sl), oracle_slices(x, s, sl), BF16_TOL, BF16_REL,
                where="fused bf16 gpt2-small")


def test_binding_rejects_mismatched_views():
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs = 1, 2, 16, 64
    q = torch.zeros((B, H, T, hs), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, T, H, hs), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o = torch.empty_like(q)
    with pytest.raises(ValueError):  # q and k with different strides
        ga.gattn_fwd_strided(q, k, q, o, None, 0.125)
    with pytest.raises(ValueError):  # head dimension not contiguous
        ga.gattn_fwd_strided(q, q, q, torch.empty((B, H, hs, T), dtype=torch.bfloat16,
                                                  device="cuda").transpose(2, 3), None, 0.125)
    with pytest.raises(ga.GattnError):  # row stride below hs: rejected by the library
        bad = torch.zeros(B * H * T * 32 + 64, dtype=torch.bfloat16, device="cuda")
        ov = bad.as_strided((B, H, T, hs), (H * T * 32, T * 32, 32, 1))
        ga.gattn_fwd_strided(q, q, q, ov, None, 0.125)


def test_size_one_dimensions_with_any_stride():
    """B = H = 1 tensors whose batch and head strides are 0 (as torch leaves a
    view of a broadcast array) give the same bits through the strided and
    dropout entry points as the canonical tensors."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs = 1, 1, 77, 64
    x = inputs(B, H, T, hs, "bf16", seed=74, workload="size-one")
    s = default_scale(hs)
    print(f"case size-one strides B={B} H={H} T={T} hs={hs}", flush=True)
    t = {n: to_dev(a, "bf16") for n, a in x.items()}
    z = {n: a.as_strided(a.shape, (0, 0, hs, 1)) for n, a in t.items()}

    def run(d):
        o = torch.empty_like(t["q"])
        lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
        ga.gattn_fwd_strided(d["q"], d["k"], d["v"], o, lse, s)
        n = ga.gattn_bwd_workspace_bytes(B, H, T, hs, ga.BF16)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        dq, dk, dv = (torch.empty_like(t["q"]) for _ in range(3))
        ga.gattn_bwd_strided(d["q"], d["k"], d["v"], o, d["do"], lse, dq, dk, dv, s, ws)
        od, ld = ga.attention_forward_dropout(d["q"], d["k"], d["v"], 0.2, 3, 1, s)
        gd = ga.attention_backward_dropout(d["q"], d["k"], d["v"], od, d["do"], ld, 0.2, 3, 1, s)
        torch.cuda.synchronize()
        return (o, lse, dq, dk, dv, od, ld, *gd)

    for i, (a, b) in enumerate(zip(run(z), run(t))):
        assert torch.equal(a, b), i
