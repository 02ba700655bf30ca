"""Build libmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m quantized_moe_expert_sigmoid_amd.build [--force]

Every source under csrc/ is compiled to an object with hipcc for gfx950 and
linked into quantized_moe_expert_sigmoid_amd/libmoe.so. Floating point is
compiled without fast-math and without contraction (every fused multiply-add
is written out), so the library's fp32 steps are the ones its header states.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
# host code under AddressSanitizer + UndefinedBehaviorSanitizer (device code
# unchanged): the pool's bookkeeping and the argument checks, run on a host
# without a GPU with the clang ASan runtime preloaded
SANITIZED_LIB = os.path.join(PKG, "libmoe_asan.so")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fno-fast-math",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source device flags. The matrix-core FFN keeps its MFMA accumulators in
# ordinary VGPRs: with the default accumulation registers the compiler rotates
# the loop-carried accumulators between them every K slice (about two
# register moves per MFMA), which left the vector ALU as busy as the matrix
# cores.
FILE_FLAGS = {
    "ffn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def file_flags(src: str) -> list[str]:
    return FILE_FLAGS.get(os.path.basename(src), [])


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def headers():
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    return hs + [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + (".asan.o" if sanitize else ".o"))
    cmd = [HIPCC, *FLAGS, *file_flags(src), *(SANITIZE_FLAGS if sanitize else []), "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(force: bool = True, jobs: int | None = None, sanitize: bool = False) -> str:
    """Compile every HIP source and link libmoe.so (sanitize: libmoe_asan.so,
    host code under ASan + UBSan). Always recompiles when force."""
    lib = SANITIZED_LIB if sanitize else LIB
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    if not force and os.path.exists(lib):
        newest = max(os.path.getmtime(p) for p in srcs + headers())
        if os.path.getmtime(lib) >= newest:
            return lib
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found: cannot build the HIP library")
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    tmp = lib + ".tmp%d" % os.getpid()
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"] \
        if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    args = ap.parse_args()
    print(build(force=True if args.force else False))
    sys.exit(0)
