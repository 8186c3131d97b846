"""Build the CPU oracle (test infrastructure only) with gcc.

IEEE fp32 semantics of the quantizers depend on these flags: no FMA
contraction and no fast-math, so every fp32 operation rounds to nearest even.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkvc_ref.so")
SRC = os.path.join(HERE, "kvc_ref.c")
FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
         "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", *FLAGS, SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
