"""Build the HIP library libmoe_latent.so for gfx950, in-tree.

Device code is compiled without floating-point contraction (every fused multiply-add in
the kernels is written out), with correctly rounded fp32 division, with denormals kept,
and with packed-fp32 instructions disabled.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_latent.so")
SOURCES = ["layer_kernels.hip", "prefill_kernels.hip", "moe_latent_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


OBJ = os.path.join(PKG, "_build")


def build(extra=(), lib=LIB, obj=OBJ):
    """Compile every source to an object (in parallel), then link the library.

    `extra` flags go to every compile and to the link; `lib` and `obj` place another build
    of the same sources (the CPU sanitizer tests build one with instrumented host code).
    """
    os.makedirs(obj, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs, objs = [], []
    for s in SOURCES:
        o = os.path.join(obj, os.path.splitext(s)[0] + ".o")
        objs.append(o)
        procs.append(subprocess.Popen([HIPCC, *FLAGS, *extra, *inc, "-c", os.path.join(CSRC, s), "-o", o]))
    bad = [s for s, p in zip(SOURCES, procs) if p.wait() != 0]
    if bad:
        raise subprocess.CalledProcessError(1, f"hipcc -c {' '.join(bad)}")
    subprocess.run([HIPCC, *FLAGS, *extra, "-shared", *objs, "-o", lib + ".tmp"], check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(sys.argv[1:]))
