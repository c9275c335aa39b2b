"""GPU: the Python binding in a fresh interpreter that loads the library before
torch has been imported.

libgattn.so asks for the HIP runtime by its soname; load_library() imports
torch first so that this resolves to torch's own runtime.  Without that, the
process would hold two HIP runtimes and the library's launches would reject
torch's streams (GATTN_ERR_HIP on the first call).  The child computes the
forward and backward of one small bf16 case and compares them with a float32
softmax-attention reference of plain torch ops (on the GPU, no batched
products) within the bf16 bar 2e-2 + 2^-8 |ref|.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import causal_self_attention_sdpa_amd as ga
ga.load_library()
import math
import torch
g = torch.Generator(device="cuda"); g.manual_seed(5)
B, H, T, hs = 2, 3, 77, 64
mk = lambda: torch.randn(B, H, T, hs, device="cuda", generator=g).to(torch.bfloat16)
q, k, v, do = mk(), mk(), mk(), mk()
o, lse = ga.attention_forward(q, k, v)
dq, dk, dv = ga.attention_backward(q, k, v, o, do, lse)
torch.cuda.synchronize()
qf, kf, vf, dof = (t.float().requires_grad_(True) for t in (q, k, v, do))
s = (qf.unsqueeze(3) * kf.unsqueeze(2)).sum(-1) / math.sqrt(hs)
s = s.masked_fill(torch.ones(T, T, device="cuda").triu(1).bool(), float("-inf"))
p = torch.softmax(s, dim=-1)
ref_o = (p.unsqueeze(-1) * vf.unsqueeze(2)).sum(3)
gq, gk, gv = torch.autograd.grad(ref_o, (qf, kf, vf), dof.detach())
for name, got, ref in (("o", o, ref_o), ("dq", dq, gq), ("dk", dk, gk), ("dv", dv, gv)):
    err = (got.float() - ref.detach()).abs()
    bar = 2e-2 + 2.0 ** -8 * ref.detach().abs()
    assert bool((err <= bar).all()), (name, float(err.max()))
print("load order ok")
"""


def test_library_loaded_before_torch():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("case binding in a fresh interpreter, library loaded before torch", flush=True)
    env = dict(os.environ, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    print(r.stdout, r.stderr[-2000:], flush=True)
    assert r.returncode == 0, f"exit status {r.returncode}:\n{r.stdout}\n{r.stderr[-2000:]}"
    assert "load order ok" in r.stdout
