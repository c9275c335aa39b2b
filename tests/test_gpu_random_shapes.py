"""GPU parity over a seeded sweep of shapes, scales and input magnitudes.

The other parity tests pin the workloads' shapes and the tile edges one by
one; this sweep draws 24 cases from a fixed generator so that combinations
nobody listed by hand are covered too: dtype (bf16, fp16, float32), B 1..3,
H 1..5, T 1..700 (log-uniform, so short and ragged lengths are common), hs
32/64 for the 16-bit paths and 1..128 (including sizes that are not a
multiple of anything) for float32, and the backward either as one call or
as its stages; the 16-bit cases also draw a softmax scale from 0.3x to 2x
the 1/sqrt(hs) of the pages and inputs x0.5, x1 or x2.  Every element of
every slice is checked against the oracle:
  * 16-bit: the first-order rounding bound of gpu_util.rounding_bound (it
    scales with the inputs and the softmax scale, unlike a fixed bar), with
    the unit roundoff of the type and the slack of the fixed-shape tests;
  * float32: the 1e-4 max-abs bar, under the conditions it is stated for
    (unit-variance inputs, scale 1/sqrt(hs)), plus 2^-20 |ref| for the
    storage of large values.
"""
import numpy as np
import pytest

from gpu_util import (U_BF16, U_F16, check_bound, check_close, default_scale, gpu_fwd_bwd, inputs,
                      oracle_slices, rounding_bound)

pytestmark = pytest.mark.gpu

F32_TOL, F32_REL = 1e-4, 2.0 ** -20
SLACK = {"bf16": 1e-3, "f16": 2e-4}
U = {"bf16": U_BF16, "f16": U_F16}


def _cases(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = str(rng.choice(["bf16", "f16", "f32"], p=[0.4, 0.35, 0.25]))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 6))
        T = max(1, int(np.exp(rng.uniform(0.0, np.log(700.0)))))
        if dtype == "f32":
            hs = int(rng.choice([1, 3, 8, 16, 24, 40, 64, 100, 128]))
        else:
            hs = int(rng.choice([32, 64]))
        scale_mult = float(rng.uniform(0.3, 2.0))
        qkv_scale = float(rng.choice([0.5, 1.0, 2.0]))
        stages = bool(rng.integers(2))
        if dtype == "f32":  # the 1e-4 bar is stated for unit-variance inputs at 1/sqrt(hs)
            scale_mult, qkv_scale = 1.0, 1.0
        out.append((i, dtype, B, H, T, hs, scale_mult, qkv_scale, stages))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-{c[1]}-B{c[2]}H{c[3]}T{c[4]}d{c[5]}")
def test_random_shape_matches_oracle(case):
    import oracle
    i, dtype, B, H, T, hs, scale_mult, qkv_scale, stages = case
    s = default_scale(hs) * scale_mult
    x = inputs(B, H, T, hs, dtype, seed=5000 + i, workload="sweep", qkv_scale=qkv_scale)
    print(f"case sweep {i} {dtype} B={B} H={H} T={T} hs={hs} scale={s:.4f} x{qkv_scale} "
          f"stages={stages}", flush=True)
    got = gpu_fwd_bwd(x, dtype, s, use_stages=stages)
    where = f"sweep {i} {dtype} {(B, H, T, hs)} scale {s:.4f} x{qkv_scale}"
    if dtype == "f32":
        ref = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], s)
        check_close(got, ref, F32_TOL, F32_REL, where=where)
        return
    slices = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_slices(x, s, slices)
    got = tuple(np.stack([a[b, h] for b, h in slices])[:, None] for a in got)
    check_bound(got, ref, rounding_bound(x, s, slices, ref, u=U[dtype], slack=SLACK[dtype]),
                where=where)
