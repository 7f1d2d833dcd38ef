"""Build the CPU oracle (test infrastructure only) into oracle/libgdn_oracle.so.

Plain gcc, no fast-math, no FMA contraction, so that float expressions are
IEEE binary32 and double expressions IEEE binary64.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")
# the same code with AddressSanitizer and UndefinedBehaviorSanitizer (any
# report aborts); loaded in place of LIB when GDN_ORACLE_LIB names it and the
# process preloads the sanitizer runtimes
SAN_LIB = os.path.join(HERE, "libgdn_oracle_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", *(SAN_FLAGS if sanitize else []),
           SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
