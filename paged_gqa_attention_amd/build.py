"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_gqa_attention_amd.build        # or __graft_entry__.build()

The library is one shared object holding the HIP kernels and the C-ABI host
code; it links the HIP runtime by its soname (libamdhip64.so.7), so in a
process that has already loaded torch it shares torch's runtime.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["decode_kernels.hip", "mq_kernels.hip", "kv_write.hip", "prologue.hip", "api.cpp"]
HEADERS = ["launch.h", "device_common.h"]

ARCH = "gfx950"
# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 are generated (the host pass
# warns that it does not know the feature; that warning is harmless).
# -amdgpu-mfma-vgpr-form: MFMA accumulators live in ordinary VGPRs, not the
# accumulation registers: the multi-query kernel's rarely taken rescale
# branch otherwise made the compiler copy every accumulator out of them on
# each iteration (measured on MI355X: wide257 110 -> 96 us, decode unchanged).
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def build(verbose: bool = False) -> str:
    """Compile every source into LIB_PATH (always recompiles). Returns the path."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc(), *COMMON_FLAGS, "-shared", "-Wl,-rpath,/opt/rocm/lib",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
