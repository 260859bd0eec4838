"""Build the fp64 oracle library (test infrastructure) with the host g++."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dma_oracle.cpp")
LIB_PATH = os.path.join(HERE, "libdma_oracle.so")


def build(verbose=False):
    out = LIB_PATH
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", SRC, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
