"""Compile the CPU oracle (test infrastructure) into oracle/liblo32.so and
oracle/liblo64.so with gcc.  Plain C99; OpenMP only parallelises the seeded
input generator's fill loops, never the oracle's arithmetic."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ld_oracle.c")
LIBS = {
    "f32": (os.path.join(HERE, "liblo32.so"), []),
    "f64": (os.path.join(HERE, "liblo64.so"), ["-DLO_REAL=double", "-DLO_REAL_IS_DOUBLE=1"]),
}
CFLAGS = ["-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose=False):
    for name, (out, defs) in LIBS.items():
        tmp = out + ".tmp"
        cmd = ["gcc"] + CFLAGS + defs + [SRC, "-o", tmp, "-lm"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return [v[0] for v in LIBS.values()]


def built():
    return all(os.path.exists(v[0]) for v in LIBS.values())


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
