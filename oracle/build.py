"""Compile the fp64 oracle (plain C, OpenMP) into liboracle.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build():
    src = os.path.join(HERE, "oracle.c")
    out = os.path.join(HERE, "liboracle.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                           "-Wall", "-o", out, src, "-lm"])
    return out


if __name__ == "__main__":
    print(build())
