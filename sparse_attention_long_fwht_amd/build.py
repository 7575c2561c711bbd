"""Build libadamas.so (HIP, gfx950 only) in-tree with hipcc.

Flags: -ffp-contract=off (no silent fma contraction: the key/query encode must
round each add once, exactly as specified), denormals kept
(-fno-gpu-flush-denormals-to-zero), packed fp32 instructions disabled, and
kernel-argument preloading: the leading scalar arguments of a kernel (up to
16 dwords) arrive in SGPRs when its waves start, so a block issues its first
loads without first fetching its arguments from memory (the decode kernels
take the values their first loads need as leading arguments).
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libadamas.so")
SOURCES = [os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "decode.hip")]
# the decoder stack's fused elementwise kernels (include/llama_glue.h), a library of their own
GLUE_LIB = os.path.join(PKG, "libllama_glue.so")
GLUE_SOURCES = [os.path.join(CSRC, "llama_glue.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    _build_one(LIB, SOURCES, verbose)
    _build_one(GLUE_LIB, GLUE_SOURCES, verbose)
    return LIB


def _build_one(lib, sources, verbose):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that
    # line is expected and harmless, everything else is shown.
    noise = "packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if msg.strip() and verbose:
        print(msg)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))
