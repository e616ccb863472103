"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Plain x86-64 code (no -march), -ffp-contract=off so every a*b+c is two fp32 roundings,
no fast-math, OpenMP over rows.  build(sanitize=True) writes oracle/liboracle_san.so instead,
the same source under AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts),
for a test run with the sanitizer runtime preloaded."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "h3dit_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
LIB_SAN = os.path.join(HERE, "liboracle_san.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = LIB_SAN if sanitize else LIB
    opt = SAN_FLAGS if sanitize else ["-O3"]
    cmd = ["gcc"] + opt + ["-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
