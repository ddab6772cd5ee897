"""Compile the CPU oracle (test infrastructure) into two shared libraries.

liboracle_f32.so: `real` = float, the precision the pages train in.
liboracle_f64.so: `real` = double, for finite-difference gradient checks.

Plain gcc, -O2, OpenMP.  No -ffast-math: every sum keeps source order.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gpt2_oracle.c")
LIBS = {
    "f32": os.path.join(HERE, "liboracle_f32.so"),
    "f64": os.path.join(HERE, "liboracle_f64.so"),
}


def build(verbose: bool = False) -> None:
    for kind, out in LIBS.items():
        cmd = ["gcc", "-O2", "-std=gnu99", "-fopenmp", "-fPIC", "-shared",
               "-fvisibility=hidden", "-Wall", "-Wno-unknown-pragmas"]
        if kind == "f64":
            cmd.append("-DORACLE_FP64")
        cmd += [SRC, "-o", out + ".tmp", "-lm"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
