"""Build libpa_verify.so (gfx950) in-tree with hipcc."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libpa_verify.so")
SOURCES = [os.path.join(CSRC, "pa_plan.cpp"), os.path.join(CSRC, "pa_kernels.hip"),
           os.path.join(CSRC, "pa_append.hip"), os.path.join(CSRC, "pa_verdict.hip"),
           os.path.join(CSRC, "pa_noalloc.hip"), os.path.join(CSRC, "pa_stream_floor.hip")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Packed fp32 arithmetic stays off: the compiler must not form
    # v_pk_{add,mul,fma}_f32 from scalar or float2 code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every source into the shared library, replacing any old one."""
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
