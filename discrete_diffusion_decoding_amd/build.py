"""Build libdg.so (HIP, gfx950) in-tree with hipcc.

Every .hip under csrc/ is compiled to an object in parallel and linked into
discrete_diffusion_decoding_amd/libdg.so.  Always rebuilds (a few seconds per
file once the headers are cached by the compiler).

build_host_asan() builds the same sources with AddressSanitizer on the host
half of the compilation only (the GPU code is compiled as usual) into
_build_asan/libdg_asan.so, for CPU tests of the host runtime: it is loaded
with the sanitizer runtime preloaded and never ships."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdg.so")
ARCH = os.environ.get("DG_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-I", INCLUDE, "-I", CSRC,
    # packed fp32 instructions stay off (hipcc would otherwise form them itself)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    # a variable read before it is set (e.g. a macro-local shadowing its
    # argument) is an error, not a warning
    "-Wall", "-Werror=uninitialized", "-Werror=sometimes-uninitialized",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: ROCm is required to build libdg")
    return p


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# host-side AddressSanitizer: each -fsanitize= goes to the host compilation only
HOST_ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile(src: str, obj_dir: str, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _build(obj_dir: str, out: str, extra=(), verbose: bool = True) -> str:
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build(verbose: bool = True) -> str:
    return _build(os.path.join(PKG, "_build"), LIB, (), verbose)


def build_host_asan(verbose: bool = True) -> str:
    """The library with AddressSanitizer on its host code.  The sanitizer
    runtime is not linked in: load the library into a process started with
    asan_runtime() in LD_PRELOAD."""
    d = os.path.join(PKG, "_build_asan")
    return _build(d, os.path.join(d, "libdg_asan.so"), HOST_ASAN_FLAGS, verbose)


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime."""
    base = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm", "lib", "clang")
    for root in (base, "/opt/rocm/llvm/lib/clang"):
        if os.path.isdir(root):
            for v in sorted(os.listdir(root), reverse=True):
                p = os.path.join(root, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
                if os.path.exists(p):
                    return p
    raise RuntimeError("the clang AddressSanitizer runtime (libclang_rt.asan-x86_64.so) was not found")


if __name__ == "__main__":
    build()
