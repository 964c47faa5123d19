"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU needed).

The three library sources are compiled for the host side only (the GPU code
object is replaced by an empty one: no kernel runs here) with the sanitizers
on the host compilation, and linked with ``tests/host_abi_check.cpp``, which
drives every entry point through its argument checks: bad pointers, formats,
shapes, alignments, zero-sized calls and extreme sizes whose products
overflow 64-bit arithmetic.  Each call must return its documented status
before any HIP call; any sanitizer report fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "scaled_quantize_fp8_amd", "csrc")
SOURCES = ["scale.hip", "quantize.hip", "gemm.hip"]
ROCM = "/opt/rocm"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tools():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not found")
    return hipcc, clang


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError(f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}")
    return r


def test_host_code_under_asan_and_ubsan(tmp_path):
    hipcc, clang = _tools()
    empty = tmp_path / "empty.hipfb"
    empty.write_bytes(b"")
    objs = []
    for src in SOURCES:
        obj = tmp_path / (src + ".o")
        _run([hipcc, "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC", "-w",
              "-Xclang", "-fcuda-include-gpubinary", "-Xclang", str(empty), *SAN,
              "-c", os.path.join(CSRC, src), "-o", str(obj)])
        objs.append(str(obj))
    drv = tmp_path / "host_abi_check"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    _run([clang, "-x", "c++", "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
          f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", *san,
          "-c", os.path.join(ROOT, "tests", "host_abi_check.cpp"), "-o", str(tmp_path / "drv.o")])
    _run([clang, *san, str(tmp_path / "drv.o"), *objs, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib", "-o", str(drv)])
    env = dict(os.environ)
    # the HIP runtime's own allocations at exit are not this library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([str(drv)], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ok" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
