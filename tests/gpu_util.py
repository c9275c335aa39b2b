"""Shared helpers for the GPU tests: run the library through the C ABI and the
oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import math

import numpy as np

import oracle
import synth_inputs as si

OUT_NAMES = ("dq", "dk", "dv", "o", "lse")


def torch_dtype(dtype: str):
    import torch
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]


def to_dev(a: np.ndarray, dtype: str):
    import torch
    a = np.ascontiguousarray(a)
    if not a.flags.writeable:  # a broadcast view: torch wants a writable array
        a = a.copy()
    return torch.from_numpy(a).to("cuda").to(torch_dtype(dtype))


def gpu_fwd_bwd(x: dict, dtype: str, scale: float, use_stages: bool = False,
                preprocess: bool = False):
    """Runs gattn_fwd then gattn_bwd; returns float64 numpy (dq, dk, dv, o, lse).
    use_stages: the backward as its two stages, gattn_bwd_dq then
    gattn_bwd_dkdv.  preprocess: the row terms from gattn_bwd_preprocess
    (D from the stored o), then gattn_bwd_dkdv, then gattn_bwd_dq."""
    import torch
    import causal_self_attention_sdpa_amd as ga
    t = {n: to_dev(a, dtype) for n, a in x.items()}
    B, H, T, hs = x["q"].shape
    o = torch.empty_like(t["q"])
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    ga.gattn_fwd(t["q"], t["k"], t["v"], o, lse, scale)
    code = {"bf16": ga.BF16, "f16": ga.F16, "f32": ga.F32}[dtype]
    ws = torch.empty(ga.gattn_bwd_workspace_bytes(B, H, T, hs, code), dtype=torch.uint8,
                     device="cuda")
    dq, dk, dv = (torch.empty_like(t["q"]) for _ in range(3))
    if preprocess:
        ga.gattn_bwd_preprocess(o, t["do"], lse, ws)
        ga.gattn_bwd_dkdv(t["q"], t["k"], t["v"], t["do"], dk, dv, scale, ws)
        ga.gattn_bwd_dq(t["q"], t["k"], t["v"], o, t["do"], lse, dq, scale, ws)
    elif use_stages:
        ga.gattn_bwd_dq(t["q"], t["k"], t["v"], o, t["do"], lse, dq, scale, ws)
        ga.gattn_bwd_dkdv(t["q"], t["k"], t["v"], t["do"], dk, dv, scale, ws)
    else:
        ga.gattn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, dq, dk, dv, scale, ws)
    torch.cuda.synchronize()
    return tuple(a.float().cpu().numpy().astype(np.float64) for a in (dq, dk, dv, o, lse))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def check_close(got, ref, tol: float, rel: float = 0.0, names=OUT_NAMES, where: str = ""):
    """Elementwise |got - ref| <= tol + rel*|ref| for every output."""
    report = {}
    for n, g, r in zip(names, got, ref):
        err = np.abs(g - r)
        bound = tol + rel * np.abs(r)
        report[n] = max_abs(g, r)
        bad = np.argwhere(~(err <= bound))
        assert bad.size == 0, (f"{where} {n}: {len(bad)} elements out of tolerance; first at "
                               f"{tuple(bad[0])}: got {g[tuple(bad[0])]}, ref {r[tuple(bad[0])]}, "
                               f"max abs err {report[n]}")
    return report


def inputs(B, H, T, hs, dtype, seed=1234, workload="test", layer=0, qkv_scale=1.0):
    return si.attention_inputs(B, H, T, hs, dtype, seed=seed, workload=workload, layer=layer,
                               qkv_scale=qkv_scale)


def oracle_slices(x: dict, scale: float, slices):
    """Oracle on selected (b, h) slices: returns outputs shaped (n, 1, T, hs)."""
    sel = {n: np.stack([a[b, h] for b, h in slices])[:, None] for n, a in x.items()}
    return oracle.attention_backward(sel["q"], sel["k"], sel["v"], sel["do"], scale)


def pick(got, slices):
    return tuple(np.stack([a[b, h] for b, h in slices])[:, None] for a in got)


U_BF16 = 2.0 ** -8  # unit roundoff of bfloat16 (8 significant bits)
U_F16 = 2.0 ** -11  # unit roundoff of IEEE binary16 (11 significant bits)


def rounding_bound(x: dict, scale: float, slices, ref, u: float = U_BF16, slack: float = 1e-3,
                   z=None, u_ds: float = U_F16):
    """First-order bound on the error of a 16-bit path, per element, for the
    selected (b, h) slices, derived from where that path rounds:
      o  = P V           P rounded to the input type (u) before the MFMA
      dv = P^T dO        P rounded (u)
      dk = s dS^T Q      dS rounded to fp16 (u_ds), with the exact row term D
      dq = s dS~ K       dS~ = P (dP - D~) rounded to fp16, D~ from the
                         16-bit-stored O (off by at most u sum |dO| |O|), and
                         the float32 correction s (D - D~) P K
    plus the rounding of the stored output itself (u |ref|).  Terms are
    float64 magnitudes built from the inputs and the oracle's lse:
    |err| <= u |ref| + u_o Mag + slack with Mag = sum of |operand products|
    (u_o = u for o and dv, u_ds for dq and dk); u is the unit roundoff of the
    16-bit type (bf16 2^-8, fp16 2^-11), `slack` covers the float32 arithmetic
    (and is the whole bound of lse, which is never rounded to 16 bits).  With
    attention dropout, z (n, T, T) holds the weight multipliers of each
    selected slice: P Z takes P's place in o and dv, and dS = P (Z dP - D)."""
    sel = {n: np.stack([a[b, h] for b, h in slices]) for n, a in x.items()}
    dq_r, dk_r, dv_r, o_r, lse_r = (a[:, 0] for a in ref)
    T = sel["q"].shape[1]
    causal = np.tril(np.ones((T, T), dtype=bool))
    s = np.einsum("nid,njd->nij", sel["q"], sel["k"]) * scale
    P = np.where(causal, np.exp(np.where(causal, s, 0.0) - lse_r[:, :, None]), 0.0)
    Z = np.ones_like(P) if z is None else np.asarray(z, dtype=np.float64)
    A = np.sum(np.abs(sel["do"]) * np.abs(o_r), axis=-1)          # |dO|.|O| per row
    D = np.sum(sel["do"] * o_r, axis=-1)
    dP = np.einsum("nid,njd->nij", sel["do"], sel["v"])
    dS = P * (Z * dP - D[:, :, None])
    W = np.abs(dS) + u * P * A[:, :, None]  # |dS~|
    mag = {
        "o": u * ((P * Z) @ np.abs(sel["v"])),
        "dv": u * (np.swapaxes(P * Z, 1, 2) @ np.abs(sel["do"])),
        "dk": u_ds * scale * (np.swapaxes(np.abs(dS), 1, 2) @ np.abs(sel["q"])),
        "dq": u_ds * scale * (W @ np.abs(sel["k"])),
    }
    out = []
    for n, r in zip(OUT_NAMES, (dq_r, dk_r, dv_r, o_r, lse_r)):
        if n == "lse":
            out.append(np.full(r.shape, slack)[:, None])
        else:
            out.append((u * np.abs(r) + mag[n] + slack)[:, None])
    return tuple(out)


def check_bound(got, ref, bound, names=OUT_NAMES, where: str = ""):
    """Elementwise |got - ref| <= bound; returns the largest err/bound ratio."""
    worst = {}
    for n, g, r, b in zip(names, got, ref, bound):
        ratio = np.abs(g - r) / b
        worst[n] = float(ratio.max())
        bad = np.argwhere(~(ratio <= 1.0))
        assert bad.size == 0, (f"{where} {n}: {len(bad)} elements above the rounding bound; "
                               f"worst ratio {worst[n]:.3f}")
    return worst


def default_scale(hs: int) -> float:
    return 1.0 / math.sqrt(hs)
