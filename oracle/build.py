"""Compile the C oracle (test infrastructure) into oracle/liboracle.so with gcc.

No FMA contraction and no fast-math: the fp32 transform must round each add/sub
once, in the written order.  OpenMP is used only to run independent heads in
parallel when a caller asks for more than one thread.

build(sanitize=True) makes a second library, liboracle_san.so, instrumented
with AddressSanitizer and UndefinedBehaviorSanitizer (host code only; any
report aborts).  The oracle's Python front end loads it instead of the plain
one when ADAMAS_ORACLE_LIB names it (the sanitizer test does this in a child
process with the ASan runtime preloaded).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "adamas_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-Wall", "-Wextra", "-Werror"]
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *(SAN_FLAGS if sanitize else []), SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
