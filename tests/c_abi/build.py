"""Builds gattn_c_roundtrip, the plain-C caller of the library (gcc, host
code only), next to its source.  It links libgattn.so, the CPU oracle
(oracle/libgattn_ref.so) and the HIP runtime, with run paths relative to the
binary, so the built tree can move."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(os.path.dirname(_HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BINARY = os.path.join(_HERE, "gattn_c_roundtrip")


def build(verbose: bool = False, out: str = BINARY) -> str:
    src = os.path.join(_HERE, "gattn_c_roundtrip.c")
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(_ROOT, "include"), "-I", os.path.join(ROCM, "include"), src,
           "-o", tmp,
           "-L", os.path.join(_ROOT, "causal_self_attention_sdpa_amd"), "-lgattn",
           "-L", os.path.join(_ROOT, "oracle"), "-lgattn_ref",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../causal_self_attention_sdpa_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
