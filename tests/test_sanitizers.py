"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. The CPU oracle (oracle/oracle.c) built with gcc and both sanitizers runs
   every one of its functions on small inputs with edge cases
   (tests/sanitize/oracle_driver.c); its checksum must equal the one an
   uninstrumented build prints.
2. libw4a8 built with both sanitizers on its host code (device code as
   usual) runs every entry point's host-side validation, the plan and
   workspace arithmetic and the status strings (tests/sanitize/abi_driver.cpp);
   valid calls stop at the HIP runtime, which finds no GPU here.

Any sanitizer report or failed check fails the test.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(SAN, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def _clean(out):
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in out, out


@pytest.fixture(scope="module")
def build_dir():
    os.makedirs(BUILD, exist_ok=True)
    return BUILD


def test_oracle_under_sanitizers(build_dir):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    srcs = [os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c")]
    common = ["-fopenmp", "-std=c11", "-ffp-contract=off"]
    san = os.path.join(build_dir, "oracle_driver_san")
    plain = os.path.join(build_dir, "oracle_driver_plain")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", *common, *srcs, "-o", san, "-lm"])
    _run(["gcc", "-O2", *common, *srcs, "-o", plain, "-lm"])
    a = subprocess.run([san], capture_output=True, text=True, env=ENV)
    _clean(a.stdout + a.stderr)
    assert a.returncode == 0, a.stdout + a.stderr
    b = _run([plain])
    assert a.stdout.strip() == b.stdout.strip() and "oracle driver ok" in a.stdout


def test_abi_validation_under_sanitizers(build_dir):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    csrc = os.path.join(ROOT, "w4a8_quantized_gemm_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]
    # host code instrumented, device code built as usual (each sanitizer
    # flag applies to the host compilation only)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", *host_san]
    objs, procs = [], []
    for src in sorted(glob.glob(os.path.join(csrc, "*.hip"))):
        obj = os.path.join(build_dir, os.path.basename(src) + ".san.o")
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc, *flags, *inc, "-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out
    lib = os.path.join(build_dir, "libw4a8_san.so")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san, *objs, "-o", lib])
    drv = os.path.join(build_dir, "abi_driver_san")
    _run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
          os.path.join(SAN, "abi_driver.cpp"), lib, f"-Wl,-rpath,{build_dir}",
          f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
          "-o", drv])
    r = subprocess.run([drv], capture_output=True, text=True, env=ENV, timeout=300)
    _clean(r.stdout + r.stderr)
    assert r.returncode == 0 and "0 failures" in r.stdout, r.stdout + r.stderr
