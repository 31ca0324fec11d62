"""Build the CPU oracle shared library (plain C, gcc, OpenMP).

Test infrastructure: the oracle is the checker, never part of the product
path.  ``build()`` always recompiles.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dwconv_oracle.c")
LIB = os.path.join(HERE, "libdwconv_oracle.so")


def build(verbose: bool = False) -> str:
    # -O2 without -march=native: the library is built here and run on other
    # hosts; -ffp-contract=off keeps every multiply and add a separate
    # double-precision rounding, as the source reads.
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_timing(out_dir: str, verbose: bool = False) -> str:
    """The CPU timing baseline: the same source with single-precision
    accumulation (-DDWO_ACC_T=float), -O3 -march=native, OpenMP.  Built on
    the host that runs it (the instruction set follows that CPU), into
    `out_dir`; not used for parity."""
    lib = os.path.join(out_dir, "libdwconv_oracle_f32.so")
    cmd = ["gcc", "-std=c99", "-O3", "-march=native", "-fopenmp", "-fPIC", "-shared",
           "-DDWO_ACC_T=float", "-o", lib, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
