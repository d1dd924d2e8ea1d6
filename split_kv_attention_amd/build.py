"""Build libsplitkv.so (HIP, gfx950) in-tree.

Every call recompiles: each translation unit under csrc/ goes to an object
file in _build/, then they are linked into split_kv_attention_amd/libsplitkv.so.
Usage:  python -m split_kv_attention_amd.build   (or __graft_entry__.build()).

build_checked() makes libsplitkv_checked.so, whose forward kernels guard every
global index (compile flag SK_CHECKED, reported by sk_check_violations).
build_c_client() compiles tests/c_client/sk_client.c, a plain C99 client of
the ABI, with gcc against the built library.
build_asan() makes a copy of the library whose HOST code is built with
AddressSanitizer (device code unchanged) in _build/asan/; a process that loads
it must preload the sanitizer runtime (asan_runtime()).  It exists for the
host-side tests of argument checking and dispatch.
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
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libsplitkv.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed f32 VALU ops.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: a ROCm toolchain is required to build libsplitkv")
    return path


def sources():
    return sorted(
        os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip") or f.endswith(".cpp")
    )


def _compile(src: str, extra: list[str], out_dir: str = BUILD) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *HIP_FLAGS, *extra, *lang, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _build_lib(path: str, flags: list[str], out_dir: str) -> str:
    """Compile every source with `flags` into out_dir and link `path`."""
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, flags, out_dir), srcs))
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)
    return path


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source and link libsplitkv.so; returns the library path."""
    _build_lib(LIB_PATH, list(extra_flags or []), BUILD)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB_PATH = os.path.join(ASAN_DIR, "libsplitkv_asan.so")
# Host-only instrumentation: each sanitizer flag applies to the host pass only.
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """Path of the AddressSanitizer runtime of the compiler hipcc drives."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "lib", "clang")
    if not os.path.isdir(llvm):
        llvm = "/opt/rocm/llvm/lib/clang"
    for ver in sorted(os.listdir(llvm), reverse=True):
        p = os.path.join(llvm, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return os.path.realpath(p)
    raise RuntimeError("AddressSanitizer runtime (libclang_rt.asan-x86_64.so) not found")


def build_asan() -> str:
    """Compile every source with the host pass under AddressSanitizer and link
    _build/asan/libsplitkv_asan.so; returns its path.  The shared library
    leaves the sanitizer's symbols to the preloaded runtime."""
    return _build_lib(ASAN_LIB_PATH, ASAN_HOST_FLAGS, ASAN_DIR)


CHECKED_LIB_PATH = os.path.join(PKG, "libsplitkv_checked.so")


def build_checked() -> str:
    """Compile every source with -DSK_CHECKED=1 (the forward kernels test
    every global index they derive and count the failures, which
    sk_check_violations reports) and link
    split_kv_attention_amd/libsplitkv_checked.so beside the normal library;
    returns its path."""
    return _build_lib(CHECKED_LIB_PATH, ["-DSK_CHECKED=1"], os.path.join(BUILD, "checked"))


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_client", "sk_client.c")
C_CLIENT_PATH = os.path.join(ROOT, "tests", "c_client", "sk_client")


def rocm_root() -> str:
    return os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))


def build_c_client() -> str:
    """Compile the plain C99 client of the ABI (tests/c_client/sk_client.c)
    with gcc against the in-tree libsplitkv.so and the HIP runtime; returns
    its path.  It finds the library beside the package at run time."""
    rocm = rocm_root()
    tmp = C_CLIENT_PATH + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
           f"-I{rocm}/include", C_CLIENT_SRC, f"-L{PKG}", "-lsplitkv", f"-L{rocm}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../split_kv_attention_amd", f"-Wl,-rpath,{rocm}/lib", "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C client build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, C_CLIENT_PATH)
    return C_CLIENT_PATH


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
