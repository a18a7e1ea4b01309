"""Build libuq.so (the HIP kernels and the C ABI of include/uq_paged.h) in-tree for gfx950.

Usage: python -m quantized_paged_attention_amd.build
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libuq.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

SOURCES = ["uq_abi.cpp", "decode_fp8.hip", "decode_fp4.hip", "reduce.hip", "index_score.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in device code
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_host_sanitized(out_dir: str) -> str:
    """libuq.so with AddressSanitizer and UndefinedBehaviorSanitizer in its host code (the
    C ABI: argument checks, planning, workspace layout), linked with the kernel objects of
    the last build().  Device code is built exactly as in build(): every -fsanitize= flag
    applies to the host side only.  Load it with clang's ASan runtime preloaded."""
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES[1:]]
    if not all(os.path.exists(o) for o in objs):
        build(verbose=False)
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    obj = os.path.join(out_dir, "uq_abi_san.o")
    cmd = [HIPCC, "-O1", "-g", *COMMON[1:], *DEVICE_FLAGS, *san, "-x", "hip", "-c",
           os.path.join(CSRC, "uq_abi.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for uq_abi.cpp (sanitized):\n{r.stderr}")
    lib = os.path.join(out_dir, "libuq_san.so")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan",
           "-o", lib, obj, *objs]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return lib


def asan_runtime() -> str:
    """Path of the ASan runtime that build_host_sanitized() links against."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


if __name__ == "__main__":
    build()
