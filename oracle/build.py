"""Build the fp64 CPU oracle (test infrastructure) with gcc.

`build(out, mutation=0)` compiles oracle/gqa_oracle.c into a shared library.
A non-zero `mutation` plants one known mistake (the ORC_MUTATE hooks in the C
source); the test suite builds those variants into a temporary directory to
show that its pins catch each mistake.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gqa_oracle.c")
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")


# AddressSanitizer + UndefinedBehaviorSanitizer build of the oracle (host
# code only; the caller preloads gcc's libasan and libubsan).
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def build(out=DEFAULT_LIB, mutation=0, verbose=False, sanitize=None):
    if sanitize is None:
        sanitize = os.environ.get("ORACLE_SANITIZE", "") not in ("", "0")
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-std=c11", "-Wall", "-Wno-unused-function",
           "-DORC_MUTATE=%d" % int(mutation)] + (SANITIZE_FLAGS if sanitize else []) + \
          [SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    print("built", DEFAULT_LIB)
    sys.exit(0)
