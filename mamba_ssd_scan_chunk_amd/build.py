"""Build libssd.so (the C-ABI HIP library) in-tree for gfx950.

    python -m mamba_ssd_scan_chunk_amd.build

Each csrc/*.hip file is compiled to an object with hipcc, in parallel, and
linked into mamba_ssd_scan_chunk_amd/libssd.so.  Packed-fp32 instructions are
disabled for all device code (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libssd.so")
OBJDIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the prefill kernels rescale them with VALU
    # instructions between MFMAs, which AGPR accumulators would turn into
    # v_accvgpr_read/write round trips
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    subprocess.check_call([HIPCC, *COMMON, "-c", src, "-o", obj])
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


# Host-side sanitizers for the library's argument checks: AddressSanitizer and
# UndefinedBehaviorSanitizer on the host half of every source only (each flag
# behind -Xarch_host; the device code is built as usual).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]


def build_host_sanitized(outdir: str) -> str:
    """libssd.so with sanitized host code, in `outdir`; load it by setting
    SSD_LIB_PATH, with clang's ASan runtime (asan_runtime()) preloaded."""
    objdir = os.path.join(outdir, "objs")
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def comp(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        subprocess.check_call([HIPCC, *COMMON, *SANITIZE_HOST, "-c", src, "-o", obj],
                              stderr=subprocess.DEVNULL)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    lib = os.path.join(outdir, "libssd.so")
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE_HOST, "-o", lib, *objs])
    return lib


def asan_runtime() -> str:
    """clang's shared AddressSanitizer runtime (with UBSan), for LD_PRELOAD."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


if __name__ == "__main__":
    build()
