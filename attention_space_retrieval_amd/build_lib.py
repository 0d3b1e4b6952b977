"""Build libkvs.so (HIP kernels + C ABI) for gfx950 with hipcc.

    python -m attention_space_retrieval_amd.build_lib [--jobs N] [--debug]

Objects go to _build/ at the repository root, the library to
attention_space_retrieval_amd/libkvs.so.  Every call rebuilds.
"""

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvs.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [
    "api.cpp",
    "qmem.hip",
    "rule_score.hip",
    "topk.hip",
    "meank_build.hip",
    "meank_score.hip",
    "workset.hip",
    "rerope_scatter.hip",
]

# Packed fp32 VALU forms are switched off for every HIP translation unit.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src, debug):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + (["-g"] if debug else []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature flag: drop that notice
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    return src, obj, r.returncode, err


def build(jobs=None, debug=False, verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, debug), SOURCES))
    failed = [r for r in results if r[2] != 0]
    for src, _, rc, err in results:
        if err.strip() and (verbose or rc):
            print(f"--- {src}\n{err}", file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(r[0] for r in failed))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [r[1] for r in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.debug))


if __name__ == "__main__":
    main()
