"""Compile the oracle (plain C, fp64, OpenMP).  Test infrastructure only."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path():
    return os.path.join(_HERE, "libsqa_oracle.so")


def build(verbose=False):
    out = lib_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
           os.path.join(_HERE, "sqa_oracle.c"), "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out
