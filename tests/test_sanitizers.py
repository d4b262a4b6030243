"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU (no GPU).

* The oracle, built with g++ and both sanitizers, runs its pin and
  losslessness tests (tests/test_oracle_pins.py, tests/test_oracle_lossless.py).
* The library, built with both sanitizers on its host code only (device code
  is unchanged), runs the C-ABI tests of tests/test_abi_cpu.py: every entry
  point's argument validation, workspace sizing, switches and strings.

Each run is a subprocess of its own with the matching sanitizer runtime
preloaded (the oracle uses GCC's runtime, the library clang's; one process
cannot hold both).  UBSan does not recover, so any finding ends the run with
a nonzero status; the output is also searched for sanitizer reports.  Leak
detection is off: the Python interpreter and the HIP runtime keep
allocations until exit by design.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "_build", "san")
REPORT_MARKERS = ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer")


def _run(env_extra, tests, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    # -s: a sanitizer report goes to the real stderr (a capture would be lost
    # when the report ends the process)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m", "not gpu", "-p",
           "no:cacheprovider"] + tests
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    found = [m for m in REPORT_MARKERS if m in out]
    assert r.returncode == 0 and not found, f"rc={r.returncode} reports={found}\n{out[-6000:]}"
    return out


def _newer(target, sources):
    return os.path.exists(target) and all(os.path.getmtime(target) >= os.path.getmtime(s)
                                          for s in sources)


def test_oracle_under_asan_ubsan():
    src = os.path.join(ROOT, "oracle", "dspark_oracle.cpp")
    lib = os.path.join(SAN_DIR, "liboracle_asan_ubsan.so")
    os.makedirs(SAN_DIR, exist_ok=True)
    if not _newer(lib, [src]):
        subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer", "-shared", "-fPIC", src, "-o", lib],
                       check=True, timeout=300)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("GCC's AddressSanitizer runtime is not installed")
    _run({"LD_PRELOAD": asan, "DSPARK_ORACLE_LIB": lib},
         ["tests/test_oracle_pins.py", "tests/test_oracle_lossless.py"], timeout=1200)


def _clang_asan_runtime():
    for pat in ("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    return None


def test_library_host_code_under_asan_ubsan():
    sys.path.insert(0, ROOT)
    from draft_verify_sampling_head_amd import build as B
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    lib = os.path.join(SAN_DIR, "libdspark_asan_ubsan.so")
    srcs = glob.glob(os.path.join(B.CSRC, "*")) + glob.glob(os.path.join(B.INCLUDE, "*.h"))
    if not _newer(lib, srcs):
        host = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                "-fno-omit-frame-pointer", "-g"]
        flags = tuple(f for h in host for f in ("-Xarch_host", h))
        B.build(lib_path=lib, objdir=os.path.join(SAN_DIR, "obj"), extra_flags=flags)
    _run({"LD_PRELOAD": rt, "DSPARK_LIB_PATH": lib}, ["tests/test_abi_cpu.py"], timeout=600)
