"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

api.cpp is rebuilt with the sanitizers on its host code (-Xarch_host), linked
with the library's other objects into tests/asan/abi_driver.c, and run: every
call the driver makes is decided on the host, so no GPU is needed, and any
out-of-bounds access, leak or undefined behaviour in the argument checks fails
the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_space_retrieval_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN = ["address", "undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    return r.returncode, out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not found")
def test_abi_layer_under_asan_and_ubsan(tmp_path):
    from attention_space_retrieval_amd import build_lib
    others = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in build_lib.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in others):
        build_lib.build(verbose=False)
    san_host = [f for s in SAN for f in ("-Xarch_host", f"-fsanitize={s}")]
    api_o = str(tmp_path / "api_asan.o")
    rc, out = _run([HIPCC, "-x", "hip", f"--offload-arch={build_lib.ARCH}", "-O1", "-g", "-std=c++17",
                    "-Xarch_host", "-fno-omit-frame-pointer", *san_host,
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o])
    assert rc == 0, out
    drv_o = str(tmp_path / "abi_driver.o")
    san = "-fsanitize=" + ",".join(SAN)
    rc, out = _run([CLANG, "-O1", "-g", san, "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(ROOT, "tests", "asan", "abi_driver.c"), "-o", drv_o])
    assert rc == 0, out
    exe = str(tmp_path / "abi_driver")
    rc, out = _run([CLANGXX, san, "-o", exe, drv_o, api_o, *others, "-L", os.path.join(ROCM, "lib"),
                    "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    rc, out = _run([exe], env=env, timeout=120)
    assert rc == 0 and "0 failed checks" in out, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
