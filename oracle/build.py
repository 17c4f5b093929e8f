"""Compile the CPU oracle (moe_oracle.c) into oracle/libmoe_oracle.so.

Test infrastructure only: the oracle checks the HIP path and is never part of it.

``build(sanitize=True)`` writes oracle/libmoe_oracle_san.so instead, built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc's runtimes; a process that
loads it needs gcc's libasan first in LD_PRELOAD).  ``oracle`` loads that copy
when MOEQ_ORACLE_SANITIZE=1.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")
SAN_LIB = os.path.join(HERE, "libmoe_oracle_san.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
          "-Wall", "-Wno-unknown-pragmas"]
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    cmd = ["gcc", *CFLAGS, *(SAN_FLAGS if sanitize else []), SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv)
    sys.exit(0)
