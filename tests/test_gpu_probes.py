"""GPU: the two diagnostic entry points run and write what they promise.

gattn_probe_mfma_bf16 writes one float per wavefront (4 per workgroup) and
gattn_probe_issue one per wavefront (8 per workgroup); with MFMA loops only
(roles 1, 4, 5) every written value is finite, since the MFMA operands are
fixed bf16 constants.  Every kind and role combination of gattn_probe_issue
launches and returns success on the caller's stream.  Neither touches memory
beyond its sink: a guard band after the sink stays untouched.
"""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_self_attention_sdpa_amd as ga
    return ga.load_library()


def _sink(n, guard=64):
    import torch
    return torch.full((n + guard,), float("nan"), dtype=torch.float32, device="cuda")


def test_probe_mfma_writes_every_wavefront(lib):
    import torch
    blocks = 16
    s = _sink(4 * blocks)
    sp = torch.cuda.current_stream().cuda_stream
    print(f"case probe mfma blocks={blocks}", flush=True)
    assert lib.gattn_probe_mfma_bf16(s.data_ptr(), blocks, 8, sp) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(s[: 4 * blocks]).all()
    assert torch.isnan(s[4 * blocks:]).all()


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_probe_issue_every_role(lib, kind):
    import torch
    blocks = 8
    sp = torch.cuda.current_stream().cuda_stream
    for roles in range(1, 16):
        s = _sink(8 * blocks)
        print(f"case probe issue kind={kind} roles={roles}", flush=True)
        assert lib.gattn_probe_issue(s.data_ptr(), blocks, 4, 4, kind, roles, sp) == 0
        torch.cuda.synchronize()
        assert not torch.isnan(s[: 8 * blocks]).any()  # every wavefront wrote its float
        assert torch.isnan(s[8 * blocks:]).all()
        if roles in (1, 4, 5):
            assert torch.isfinite(s[: 8 * blocks]).all()
