"""GPU: the library called from plain C (tests/c_abi/gattn_c_roundtrip.c).

The program allocates device memory with the HIP runtime, runs the causal
forward and backward through the C ABI on float32 and bf16 inputs (the tiny
4x4x8x8 shape, a ragged float32 shape, bf16 at hs 64 and 32 with ragged T),
and compares every output with the float64 oracle library on the same
inputs, to the float32 (1e-4) and bf16 (2e-2 + 2^-8 |ref|) bars; it also
checks that an invalid call is rejected before any launch.  The binary is
built by build() (gcc, host code only) and rebuilt here only if absent.
"""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _binary():
    import importlib.util
    path = os.path.join(HERE, "c_abi", "build.py")
    spec = importlib.util.spec_from_file_location("gattn_c_abi_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.BINARY if os.path.exists(mod.BINARY) else mod.build()


def test_plain_c_caller_matches_oracle():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = _binary()
    print(f"case plain C caller {exe}", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, f"exit status {r.returncode}:\n{r.stdout}\n{r.stderr}"
    assert "all cases within their bars" in r.stdout
