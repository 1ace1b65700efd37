"""Build liboracle.so (the fp64 CPU oracle; test infrastructure only)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # -ffp-contract=off: the only fused multiply-adds are the explicit fma() calls
    # whose order the oracle fixes; -mfma lets those calls use the hardware FMA.
    cmd = ["gcc", "-O2", "-std=c11", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
