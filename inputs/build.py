"""Compile the input generator (plain C, OpenMP) into a shared library."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path():
    return os.path.join(_HERE, "libsqa_inputs.so")


def build(verbose=False):
    out = lib_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
           os.path.join(_HERE, "gen.c"), "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out
