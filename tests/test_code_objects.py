"""CPU checks of the GPU code the library ships: every device code object in
libgattn.so is built for gfx950 and holds none of the instructions the build
rules out.

* Packed float32 vector ops (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32): every
  HIP file is compiled with the packed-fp32 target feature off, so none may
  appear.
* Writes through the scalar data cache (scalar stores and atomics, its
  write-back or discard): the kernels write through vector stores only.

The code objects are taken out of the library with llvm-objdump --offloading
and disassembled with llvm-objdump -d (the library is this repository's own
build)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "causal_self_attention_sdpa_amd", "libgattn.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
SCALAR_WRITE = re.compile(r"\bs_(store|buffer_store|scratch_store|atomic|buffer_atomic|"
                          r"dcache_wb|dcache_discard)\w*")


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not found")
    if not os.path.exists(LIB):
        pytest.skip("libgattn.so not built")
    d = tmp_path_factory.mktemp("code_objects")
    shutil.copy(LIB, d / "libgattn.so")
    subprocess.run([OBJDUMP, "--offloading", "libgattn.so"], cwd=d, check=True,
                   capture_output=True)
    bundles = sorted(p for p in os.listdir(d) if "amdgcn" in p)
    out = {}
    for b in bundles:
        r = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", b], cwd=d, check=True,
                           capture_output=True, text=True)
        out[b] = r.stdout
    return out


def test_every_device_code_object_is_gfx950(disassembly):
    assert disassembly, "no device code objects in the library"
    for name in disassembly:
        assert name.endswith("--gfx950"), name


def test_no_packed_fp32_ops(disassembly):
    for name, text in disassembly.items():
        hits = PACKED_F32.findall(text)
        assert not hits, f"{name}: {len(hits)} packed fp32 instructions"


def test_no_writes_through_the_scalar_cache(disassembly):
    for name, text in disassembly.items():
        hits = sorted(set(m.group(0) for m in SCALAR_WRITE.finditer(text)))
        assert not hits, f"{name}: {hits}"


def test_the_mfma_kernels_are_there(disassembly):
    n = sum(len(re.findall(r"\bv_mfma_f32_32x32x16_(bf16|f16)\b", t)) for t in disassembly.values())
    assert n > 1000
