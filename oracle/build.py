"""Build the fp64 CPU oracle (oracle/liboracle.so) with gcc.

Test infrastructure only: the oracle is what the GPU library is checked
against, never part of the product path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "xl_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


# AddressSanitizer and UndefinedBehaviorSanitizer build (for a process that
# preloads gcc's libasan and libubsan): every out-of-bounds access or
# undefined operation in the oracle then aborts the run with a report.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = ["gcc", "-O1" if sanitize else "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", *(SANITIZE if sanitize else []), SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
