"""The CPU oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; the GPU code is not instrumented).

- The oracle (plain C) is built with gcc's -fsanitize=address,undefined and
  its pins run against that build in a child process that preloads gcc's
  sanitizer runtimes; a read past an undersized buffer must abort that
  process (the instrumentation is live).
- The HIP library is built with the sanitizers on its host code (argument
  checks, workspace layouts, launch set-up; -Xarch_host) and the C-ABI and
  binding tests run against it in a child process that preloads clang's
  ASan runtime (it carries the UBSan handlers).  That build takes a minute
  or two and is kept, keyed by a hash of the sources, for later runs.
Any sanitizer report aborts its child process and fails the test.
"""
import hashlib
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG_ASAN = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


def _gcc_runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def _child(preload, env_extra, args, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", **env_extra)
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = ["timeout", "-k", "10", str(timeout), "env", f"LD_PRELOAD={preload}", sys.executable, *args]
    return subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True)


def test_oracle_under_asan_ubsan():
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    lib = ob.build(sanitize=True)
    pre = f"{asan}:{ubsan}"
    r = _child(pre, {"GDN_ORACLE_LIB": lib},
               ["-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x", "-p", "no:cacheprovider"])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    # a QDQ tile of 128 values over a 64-value buffer reads past its end
    probe = ("import ctypes, numpy as np; L = ctypes.CDLL(%r); x = np.ones(64, np.float32); "
             "o = np.zeros(128, np.float32); s = np.zeros(1, np.float32); "
             "fp = ctypes.POINTER(ctypes.c_float); "
             "L.orc_qdq_tile_f32(x.ctypes.data_as(fp), ctypes.c_int64(128), o.ctypes.data_as(fp), "
             "s.ctypes.data_as(fp), None)") % lib
    r = _child(pre, {}, ["-c", probe], timeout=120)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]


def _sources_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "fp8_state_qat_amd", "csrc", "*")) +
                    glob.glob(os.path.join(ROOT, "include", "*.h")) +
                    [os.path.join(ROOT, "fp8_state_qat_amd", "build.py")]):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def test_host_abi_under_asan():
    if not CLANG_ASAN:
        pytest.skip("clang's ASan runtime is not installed")
    sys.path.insert(0, ROOT)
    from fp8_state_qat_amd import build as fb
    stamp = fb.SAN_LIB + ".sources"
    want = _sources_hash()
    if not (os.path.exists(fb.SAN_LIB) and os.path.exists(stamp) and open(stamp).read() == want):
        fb.build(sanitize=True)
        with open(stamp, "w") as f:
            f.write(want)
    r = _child(CLANG_ASAN[-1], {"GDN_LIB": fb.SAN_LIB},
               ["-m", "pytest", "tests/test_abi_cpu.py", "tests/test_api_cpu.py", "-q", "-x", "-m", "not gpu",
                "-p", "no:cacheprovider"])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
