"""Build the CPU oracle (test infrastructure only) into oracle/liboracle.so.

Plain gcc, -O2 without fast-math so that every operation keeps its IEEE double
meaning; OpenMP only splits independent (sequence, head) pairs over threads.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pkv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if os.environ.get("PKV_SANITIZE", "") == "1":
        # AddressSanitizer and UndefinedBehaviorSanitizer (load with the
        # runtimes preloaded, as paged_kv_cache_101_amd/build.py describes)
        cmd[1:1] = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-g"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
