"""Build libzebra.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

    python -m linear_hybrid_attention_zebra_amd.build

compiles every source under ``csrc/`` for gfx950 into ``_build/`` at the
repository root and links ``linear_hybrid_attention_zebra_amd/libzebra.so``.
The library is linked against the HIP runtime by soname; at run time it binds
to the runtime already loaded by torch (import torch first).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libzebra.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # never let the compiler form packed fp32 ops (v_pk_fma_f32 and friends).
    # The feature exists only for the gfx950 device pass; the x86 host pass of
    # the same hipcc line reports it as unknown and ignores it (the warning is
    # filtered below). tests/test_build_flags.py checks the device assembly.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in arch VGPRs: the softmax reads them with VALU ops, and
    # the AGPR form costs a v_accvgpr_read/write per element
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libzebra")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc()] + COMMON_FLAGS + ["-x", "hip", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    # the host pass's notice about the device-only feature above (nothing else)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    warn = "\n".join(l for l in res.stderr.splitlines() if noise not in l).strip()
    if warn:
        print(warn, file=sys.stderr)
    return obj


def device_asm(src: str, out: str) -> str:
    """gfx950 assembly of one source, compiled with the library's own flags."""
    cmd = [hipcc()] + COMMON_FLAGS + ["--cuda-device-only", "-S", "-o", out]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    res = subprocess.run(cmd + [src], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{res.stderr}")
    return out


ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB_PATH = os.path.join(ASAN_DIR, "libzebra_asan.so")


def asan_runtime() -> str:
    """Path of the host AddressSanitizer runtime of the ROCm compiler."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    return res.stdout.strip()


def build_asan(jobs: int = 8) -> str:
    """A copy of the library whose HOST code is built with AddressSanitizer
    (the gfx950 device code is built as usual): for the host-side ABI tests,
    which exercise argument validation and launch nothing. Needs the ASan
    runtime preloaded into the process that loads it."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    flags = COMMON_FLAGS + ["-Xarch_host", "-fsanitize=address", "-Xarch_host",
                            "-fno-omit-frame-pointer", "-g"]

    def one(src):
        obj = os.path.join(ASAN_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc()] + flags + (["-x", "hip"] if src.endswith(".cpp") else []) + \
            ["-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc (asan) failed on {src}:\n{res.stderr}")
        return obj

    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(one, srcs))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan",
           "-Xarch_host", "-fsanitize=address", "-o", ASAN_LIB_PATH] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"asan link failed:\n{res.stderr}")
    return ASAN_LIB_PATH


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every kernel source for gfx950 and link libzebra.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--asan":
        print(build_asan())
    else:
        build(verbose=True)
