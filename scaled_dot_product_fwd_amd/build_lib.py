"""Build libsdpa_fwd.so (HIP kernels + C ABI) in-tree for gfx950.

    python -m scaled_dot_product_fwd_amd.build_lib [--incremental] [--resource-usage]

Objects go to ``_build/`` at the repository root, the shared library next to
this file.  Each kernel-instantiation unit compiles separately so the build
runs in parallel.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsdpa_fwd.so")
ARCH = "gfx950"

HIP_SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")) + ["sdpa_api.cpp"]
CXX_SOURCES = ["plan.cpp"]
HEADERS = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + [
    os.path.join(ROOT, "include", "sdpa.h")]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


# -packed-fp32-ops keeps the compiler from forming packed fp32 VALU ops.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # keep MFMA accumulators in ordinary VGPRs: the softmax rescales
             # them with VALU ops, which would otherwise copy them out of and
             # back into the accumulation registers every block
             "-mllvm", "-amdgpu-mfma-vgpr-form=1",
             "-I", os.path.join(ROOT, "include")]


# Per-unit extra flags.  The large-head-dim prefill kernels and the decode
# kernels run one wave per SIMD, so nothing but the instruction schedule hides
# LDS and MFMA latency; the iterative ILP scheduler measures 15-20% faster for
# the former and 1-3% for the latter (and no better for the small-dim prefill
# and short-query units, which keep the default).
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
UNIT_FLAGS = {f"inst_{t}_{k}{m}.hip": _ILP for t in ("bf16", "f16", "f32")
              for k in ("prefill_large", "decode") for m in ("", "_mask")}


def _needs(obj: str, src: str) -> bool:
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(p) > t for p in [src] + HEADERS)


def _compile(cmd, label):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    return label, r.returncode, out


def build(incremental: bool = False, resource_usage: bool = False, jobs: int | None = None) -> str:
    """Compile every source for gfx950 and link the shared library.  Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = jobs or min(8, os.cpu_count() or 1)
    work = []
    objs = []
    for f in HIP_SOURCES:
        src = os.path.join(CSRC, f)
        obj = os.path.join(BUILD, f + ".o")
        objs.append(obj)
        if incremental and not _needs(obj, src):
            continue
        flags = list(HIP_FLAGS) + UNIT_FLAGS.get(f, [])
        if resource_usage and f.endswith(".hip"):
            flags.append("-Rpass-analysis=kernel-resource-usage")
        lang = ["-x", "hip"] if f.endswith(".cpp") else []
        work.append(([hipcc] + flags + lang + ["-c", src, "-o", obj], f))
    for f in CXX_SOURCES:
        src = os.path.join(CSRC, f)
        obj = os.path.join(BUILD, f + ".o")
        objs.append(obj)
        if incremental and not _needs(obj, src):
            continue
        work.append((["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"),
                      "-c", src, "-o", obj], f))
    failed = []
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for label, rc, out in ex.map(lambda w: _compile(*w), work):
            if out.strip():
                print(f"--- {label}\n{out}", file=sys.stderr)
            if rc != 0:
                failed.append(label)
    if failed:
        raise RuntimeError("compile failed: " + ", ".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--incremental", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    args = ap.parse_args()
    print(build(args.incremental, args.resource_usage, args.jobs))


if __name__ == "__main__":
    main()
