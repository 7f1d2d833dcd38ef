"""Build the HIP library fp8_state_qat_amd/libgdn.so for gfx950 with hipcc.

Every source under csrc/ goes into one shared object that exports the C ABI
declared in include/gdn.h.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgdn.so")
# the same library with its host code (the C ABI's checks, layouts and
# launches) under AddressSanitizer and UndefinedBehaviorSanitizer, device code
# unchanged; loaded in place of LIB when GDN_LIB names it and the process
# preloads the sanitizer runtimes
SAN_LIB = os.path.join(HERE, "libgdn_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # IEEE fp32 division and square root (the QDQ scale and x / s are IEEE divisions)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    "-ffp-contract=fast",
    # no packed fp32 ALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-I", INCLUDE, "-I", CSRC, *sources(),
           "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
