"""GPU: the largest problem the C ABI accepts.

B*H*T*hs must stay below 2^31 elements.  B=8191, H=64, T=64, hs=64 is 262144
elements short of that (4.29 GB per bf16 tensor): the launch grids have
524224 query or key tiles and every slice offset lies past 2^31 bytes for
most slices, so any 32-bit overflow in a grid index, slice offset or row
vector index shows up here.  Inputs are seeded draws made on the GPU (the
host generator would take minutes at this size); sampled slices, the first,
the last and others spread over the batch, are copied back and checked
against the oracle to the bf16 bar (2e-2 + 2^-8 |ref|).  One element more
per slice (T=65) is rejected before any launch.
"""
import numpy as np
import pytest

from gpu_util import check_close, default_scale

pytestmark = pytest.mark.gpu

BF16_TOL, BF16_REL = 2e-2, 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_self_attention_sdpa_amd as ga
    ga.load_library()


def test_largest_accepted_size():
    import torch
    import causal_self_attention_sdpa_amd as ga
    import oracle
    B, H, T, hs = 8191, 64, 64, 64
    assert B * H * T * hs < 2 ** 31 and B * H * T * hs + 2 ** 18 == 2 ** 31
    print(f"case largest size B={B} H={H} T={T} hs={hs}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(20241)
    mk = lambda: torch.randn((B, H, T, hs), device="cuda", generator=g, dtype=torch.float32
                             ).to(torch.bfloat16)
    q, k, v, do = mk(), mk(), mk(), mk()
    s = default_scale(hs)
    o, lse = ga.attention_forward(q, k, v, s)
    dq, dk, dv = ga.attention_backward(q, k, v, o, do, lse, s)
    torch.cuda.synchronize()
    slices = [(0, 0), (B - 1, H - 1), (B // 2, 17), (4096, 63), (8000, 1)]
    pick = lambda t: np.stack([t[b, h].float().cpu().numpy().astype(np.float64)
                               for b, h in slices])[:, None]
    x = {n: pick(t) for n, t in (("q", q), ("k", k), ("v", v), ("do", do))}
    ref = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], s)
    got = tuple(pick(t) for t in (dq, dk, dv, o, lse))
    check_close(got, ref, BF16_TOL, BF16_REL, where="largest size")
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_one_more_element_per_slice_is_rejected():
    import torch
    import causal_self_attention_sdpa_amd as ga
    B, H, T, hs = 8191, 64, 65, 64
    assert B * H * T * hs >= 2 ** 31
    lib = ga.load_library()
    p = torch.empty(16, dtype=torch.bfloat16, device="cuda").data_ptr()
    # pointers are never dereferenced: the shape check runs before any launch
    assert lib.gattn_fwd(p, p, p, p, None, B, H, T, hs, 0.125, ga.BF16, None) == 1
