"""Build librtp.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m head_wise_sparse_amd.build          # compiles head_wise_sparse_amd/lib/librtp.so

Every HIP source under csrc/ is compiled to an object under _build/ (in parallel)
and linked into one shared library next to the Python binding.

build_host_sanitized(out_dir) makes a second copy whose host code (argument checks,
workspace layout, launch set-up) carries AddressSanitizer and UndefinedBehaviorSanitizer
checks; the device code is built as usual.  It is loaded with the ASan runtime
preloaded (asan_runtime()) by the CPU tests, never shipped.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "librtp.so")
ARCH = "gfx950"

# Packed-fp32 instructions stay off: hipcc must not form v_pk_{add,mul,fma}_f32.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I" + INCLUDE,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-parameter"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build librtp")


# host-only sanitizer flags: each -fsanitize= applies to the host pass alone
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """The ASan runtime of hipcc's clang (to LD_PRELOAD into a process that loads the
    host-sanitized library)."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root), reverse=True) if os.path.isdir(root) else []:
        p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError(f"no libclang_rt.asan-x86_64.so under {root}")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc()] + HIP_FLAGS + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)      # the host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def device_asm(src: str, out_path: str) -> str:
    """gfx950 assembly of one source's device code, with the library's flags (for checks
    of the generated instruction stream)."""
    cmd = [hipcc()] + HIP_FLAGS + ["--cuda-device-only", "-S", src, "-o", out_path]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stdout}{r.stderr}")
    return out_path


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


def build_host_sanitized(out_dir: str) -> str:
    """librtp.so with ASan + UBSan on its host code, under out_dir (returns its path)."""
    obj_dir = os.path.join(out_dir, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, False, obj_dir, SAN_FLAGS), srcs))
    path = os.path.join(out_dir, "librtp_san.so")
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}"] + SAN_FLAGS + ["-o", path] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    return path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
