"""GPU: gattn_bwd_noalloc (the backward on the library's static device
scratch, for callers that cannot allocate) against gattn_bwd (the same
kernels on a caller workspace), bit for bit, through the C ABI: two calls in
a row on the same GPU, the second on a smaller problem, so the second reads
row terms the first left in the scratch wherever it does not overwrite them
(it must overwrite every one it reads)."""
import math

import pytest

from gpu_util import inputs, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_self_attention_sdpa_amd as ga
    ga.load_library()


def _both(B, H, T, hs, dtype, seed):
    import torch
    import causal_self_attention_sdpa_amd as ga
    x = inputs(B, H, T, hs, dtype, seed=seed, workload="noalloc")
    t = {n: to_dev(a, dtype) for n, a in x.items()}
    scale = 1.0 / math.sqrt(hs)
    o = torch.empty_like(t["q"])
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    ga.gattn_fwd(t["q"], t["k"], t["v"], o, lse, scale)
    code = {"bf16": ga.BF16, "f16": ga.F16, "f32": ga.F32}[dtype]
    ws = torch.empty(ga.gattn_bwd_workspace_bytes(B, H, T, hs, code), dtype=torch.uint8,
                     device="cuda")
    ref = [torch.empty_like(t["q"]) for _ in range(3)]
    ga.gattn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, *ref, scale, ws)
    got = [torch.full_like(t["q"], float("nan")) for _ in range(3)]
    ga.gattn_bwd_noalloc(t["q"], t["k"], t["v"], o, t["do"], lse, *got, scale)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_workspace_backward_twice(dtype):
    import torch
    hs_big, hs_small = (64, 32) if dtype == "bf16" else (16, 8)
    for (B, H, T, hs, seed) in ((2, 3, 300, hs_big, 61), (1, 2, 129, hs_small, 62)):
        print(f"case noalloc {dtype} B={B} H={H} T={T} hs={hs}", flush=True)
        ref, got = _both(B, H, T, hs, dtype, seed)
        for n, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a, b), (dtype, (B, H, T, hs), n)


def test_noalloc_gpt2_shape():
    """The GPT-2 124M layer (B12 H12 T1024 hs64 bf16) fits the scratch."""
    import torch
    print("case noalloc bf16 B=12 H=12 T=1024 hs=64", flush=True)
    ref, got = _both(12, 12, 1024, 64, "bf16", 63)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
