"""Builds the oracle's C library with gcc (plain C11, fp64, OpenMP; no fast-math)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(HERE, "libmala_oracle.so")


def build() -> str:
    src = os.path.join(HERE, "mala_oracle.c")
    out = lib_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
