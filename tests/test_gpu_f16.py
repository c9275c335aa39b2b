"""GPU parity of the fp16 path (GATTN_F16) against the CPU oracle.

fp16 runs the same kernels as bf16 with the fp16 MFMA and conversions; the
pages offer it as the other half-precision option.  No tolerance for it is
given, so the bar is the first-order rounding bound of gpu_util.rounding_bound
with the unit roundoff of binary16 (u = 2^-11) in place of bf16's, derived
from where the path rounds (P, dS, the stored O and the outputs), plus 2e-4
for the float32 arithmetic; lse is never rounded to 16 bits and must be within
2e-4.  Inputs are the seeded draws rounded to fp16 (round to nearest even).
"""
import numpy as np
import pytest

from gpu_util import (U_F16, check_bound, default_scale, gpu_fwd_bwd, inputs, oracle_slices,
                      pick, rounding_bound)

pytestmark = pytest.mark.gpu

SLACK = 2e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_self_attention_sdpa_amd as ga
    ga.load_library()


def _check(B, H, T, hs, slices=None, qkv_scale=1.0, seed=81, workload="f16"):
    x = inputs(B, H, T, hs, "f16", seed=seed, workload=workload, qkv_scale=qkv_scale)
    s = default_scale(hs)
    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    print(f"case f16 B={B} H={H} T={T} hs={hs} x{qkv_scale} slices={len(slices)}", flush=True)
    got = pick(gpu_fwd_bwd(x, "f16", s), slices)
    ref = oracle_slices(x, s, slices)
    return check_bound(got, ref, rounding_bound(x, s, slices, ref, u=U_F16, slack=SLACK),
                       where=f"f16 {(B, H, T, hs)} x{qkv_scale}")


@pytest.mark.parametrize("hs", [64, 32])
@pytest.mark.parametrize("T", [1, 17, 64, 65, 129, 200, 257])
def test_f16_ragged_lengths(T, hs):
    _check(2, 3, T, hs)


def test_f16_gpt2_small_shape():
    """B=12, H=12, T=1024, hs=64, q/k/v x0.5: full launch, sampled slices."""
    _check(12, 12, 1024, 64, slices=[(0, 0), (5, 7), (11, 11)], qkv_scale=0.5)


def test_f16_gpt2_small_whole_layer():
    """B=12, H=12, T=1024, hs=64, q/k/v x0.5: every slice of the layer."""
    _check(12, 12, 1024, 64, qkv_scale=0.5)


def test_f16_softmax_range_stress():
    """q/k/v x2.0: scores up to ~±60, the weights span many orders of magnitude."""
    _check(12, 12, 1024, 64, slices=[(0, 0), (6, 4)], qkv_scale=2.0)


def test_f16_softmax_range_stress_whole_layer():
    """q/k/v x2.0 at B=12, H=12, T=1024, hs=64: every slice of the layer."""
    _check(12, 12, 1024, 64, qkv_scale=2.0, seed=84)


def test_f16_char_level_shape():
    _check(64, 6, 256, 64, slices=[(0, 0), (17, 3), (63, 5)])


def test_f16_more_accurate_than_bf16():
    """Same draws: the fp16 path's error against the oracle is well below the
    bf16 path's (8x smaller unit roundoff)."""
    B, H, T, hs = 2, 4, 300, 64
    s = default_scale(hs)
    errs = {}
    for dt in ("bf16", "f16"):
        x = inputs(B, H, T, hs, dt, seed=82, workload="f16-vs-bf16")
        sl = [(0, 0), (1, 3)]
        got = pick(gpu_fwd_bwd(x, dt, s), sl)
        ref = oracle_slices(x, s, sl)
        errs[dt] = float(np.max([np.max(np.abs(g - r)) for g, r in zip(got[:4], ref[:4])]))
    print(f"max abs error bf16 {errs['bf16']:.3g} f16 {errs['f16']:.3g}", flush=True)
    assert errs["f16"] < errs["bf16"] / 3


def test_f16_fused_layout_bitwise_equals_contiguous():
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs = 2, 4, 160, 64
    x = inputs(B, H, T, hs, "f16", seed=83, workload="f16-fused")
    s = default_scale(hs)
    C = H * hs
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.float16)
    qkv = dev(np.concatenate([x[n].transpose(0, 2, 1, 3).reshape(B, T, C)
                              for n in ("q", "k", "v")], axis=2))
    dy = dev(x["do"].transpose(0, 2, 1, 3).reshape(B, T, C))
    y, lse = ga.attention_forward_qkv(qkv, H, s)
    dqkv = ga.attention_backward_qkv(qkv, y, dy, lse, H, s)
    torch.cuda.synchronize()
    f = lambda t, k: t.float().cpu().numpy().astype(np.float64).reshape(B, T, k, H, hs)
    yo = f(y, 1)[:, :, 0].transpose(0, 2, 1, 3)
    g = f(dqkv, 3).transpose(2, 0, 3, 1, 4)
    ref_c = gpu_fwd_bwd(x, "f16", s)
    for n, a, b in zip(("dq", "dk", "dv", "o", "lse"),
                       (g[0], g[1], g[2], yo, lse.cpu().numpy().astype(np.float64)), ref_c):
        assert np.array_equal(a, b), f"{n} differs from the contiguous path"
