"""Build liblightning_attn.so for gfx950 with hipcc, in-tree.

    python -m long_context_attn_amd.build        (or build() from Python)

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled, and linked with the host API into one shared library next to this
file.  The C ABI is declared in include/lightning_attn.h.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblightning_attn.so")
SOURCES = ["api.cpp", "plan_scan_norm.hip", "valu.hip", "mfma.hip", "state_mfma.hip",
           "decode.hip", "backward.hip", "backward_mfma.hip", "gemm_hipblaslt.cpp", "gemm.hip",
           "softmax_attn.hip"]
ARCH = "gfx950"
# hipBLASLt: the projection GEMMs of the layer entry point
LIBS = ["-L" + os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib"), "-lhipblaslt"]


def source_sha() -> str:
    """Short hash of the HIP/C++ sources: ties a committed profile to the kernels it measured."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", "-x", "hip", "--offload-arch=" + ARCH,
            "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + INCLUDE, "-I" + CSRC, "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, jobs: int = 8) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, src.rsplit(".", 1)[0] + ".o")
        cmd = [cc] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
        if verbose:
            print(" ".join(cmd))
        return obj

    with ThreadPoolExecutor(max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + LIBS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
