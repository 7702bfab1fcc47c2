"""The C ABI's host validation layer under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed).

spec_verify.cpp (argument checks, workspace planning, dispatch) is compiled
with both sanitizers on its host code and linked with the library's other
objects and tests/sanitize/abi_checks.cpp, which calls every entry point with
arguments the validation must reject (sizes whose products reach 2^31,
misaligned pointers, NULLs, undersized workspaces) and with empty problems.
The run must print "all checks passed" with no sanitizer report.  (It found
one: out-of-range values of the C enums were undefined in C++, since the types
spanned only their enumerators; they now span every int32.)
"""
import os
import subprocess


from verify_pass_rejection_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "abi_checks_sanitized")
# Each sanitizer flag applies to host code only (after -Xarch_host): the
# device code is compiled as usual.
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_validation_layer_under_asan_and_ubsan():
    objs = [os.path.join(B.BUILD, s + ".o") for s in B.SOURCES if s != "spec_verify.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build_library(verbose=False)
    host_obj = os.path.join(B.BUILD, "spec_verify_sanitized.o")
    flags = [f for f in B.CFLAGS if f != "-O3"] + ["-O1", "-g"]
    cmd = [B.HIPCC, *flags, *SAN, "-x", "hip", "-c", os.path.join(B.CSRC, "spec_verify.cpp"),
           "-o", host_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    driver_obj = os.path.join(B.BUILD, "abi_checks_sanitized.o")
    cmd = [B.HIPCC, *flags, *SAN, "-x", "hip", "-c",
           os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"), "-o", driver_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", *SAN, driver_obj, host_obj, *objs, "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    syms = subprocess.run(["nm", host_obj], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_handle_" in syms      # the checks are compiled in
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([OUT], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
