"""Build the HIP library libpa.so in-tree for gfx950 with hipcc.

    python -m paged_kv_gqa_write_amd.build          # always recompiles

The library is a plain shared object exporting the C ABI of include/pa.h;
the Python binding loads it with ctypes.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libpa.so")
SOURCES = ["pa_api.hip", "write_kv.hip", "decode.hip", "prefill.hip", "copy.hip",
           "noalloc.hip", "prefix_index.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Packed fp32 instructions stay off: plain fp32 math only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # The first kernel arguments arrive in SGPRs at wave launch instead of
    # through a scalar load; the kernels list first what their first memory
    # loads need.
    "-mllvm", "-amdgpu-kernarg-preload-count=11",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build_library(out_path: str = LIB_PATH, verbose: bool = False) -> str:
    """Compile all HIP sources into one shared library (atomically replaced)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(prefix="libpa.", suffix=".so.tmp", dir=os.path.dirname(out_path))
    os.close(fd)
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{os.path.join(ROOT, 'include')}", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out_path


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv[1:]))
