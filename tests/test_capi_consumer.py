"""The library used from plain C: tests/capi/kvs_c_consumer.c includes only
kvs.h and the HIP runtime header, takes device memory from hipMalloc and runs
an IntentKV rule turn and a KVMEM Mean-K step through the C ABI, checking the
invariants that hold exactly (sums, forced sets, valid top-C* selections, the
slot map, index means, bit-exact V pages, K pair norms, determinism).  The
CPU test compiles and links it with warnings as errors; the GPU test runs it.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "attention_space_retrieval_amd")
SRC = os.path.join(ROOT, "tests", "capi", "kvs_c_consumer.c")
ROCM = "/opt/rocm"
CC = shutil.which("gcc") or shutil.which("cc")


def _compile(out):
    lib = os.path.join(PKG, "libkvs.so")
    if not os.path.exists(lib):
        from attention_space_retrieval_amd import build_lib
        build_lib.build(verbose=False)
    cmd = [CC, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", out,
           "-L", PKG, "-lkvs", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


@pytest.mark.skipif(CC is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="C compiler or HIP headers not found")
def test_c_consumer_compiles_against_the_header(tmp_path):
    exe = _compile(str(tmp_path / "kvs_c_consumer"))
    assert os.path.exists(exe)


@pytest.mark.gpu
def test_c_consumer_runs_rule_turn_and_meank_step(tmp_path):
    exe = _compile(str(tmp_path / "kvs_c_consumer"))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    out = r.stdout + r.stderr
    print(out)
    assert r.returncode == 0 and "0 failed checks" in out, out
