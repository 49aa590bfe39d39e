"""Build libjl.so (the C-ABI library) in-tree for gfx950 with hipcc.

    python -m encoder_transformer_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
prints a harmless warning that it does not know that feature.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libjl.so")
SOURCES = ["jl_kernels.hip", "jl_layer.hip", "jl_head.hip", "jl_embed.hip", "jl_api.cpp", "jl_router.cpp", "jl_serve.cpp"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -amdgpu-mfma-vgpr-form keeps matrix-core accumulators in ordinary VGPRs:
# otherwise the compiler may place them in AGPRs, and every vector operation
# on them (the attention kernel's online-softmax rescale) then costs a copy
# out and back.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _quiet(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops' is not a recognized" not in l)


def build(verbose: bool = False) -> str:
    """Compile every source and link libjl.so; returns its path. Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    objs = []
    for src, obj, p in procs:
        out, _ = p.communicate()
        out = _quiet(out)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if out.strip() and verbose:
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + _quiet(r.stdout))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
