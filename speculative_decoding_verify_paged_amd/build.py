"""Build libpa_verify.so in-tree with hipcc for gfx950.

Every HIP source under csrc/ is compiled to an object in parallel, then
linked into ``speculative_decoding_verify_paged_amd/libpa_verify.so``.
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
LIB = os.path.join(PKG, "libpa_verify.so")
MEMBENCH_SRC = os.path.join(PKG, "membench", "membench.hip")
MEMBENCH_LIB = os.path.join(PKG, "libpa_membench.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-command-line-argument",
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(extra_flags=(), verbose: bool = False) -> str:
    """Build libpa_verify.so (the attention library) and libpa_membench.so
    (the read-ceiling and copy reference kernels the benchmark uses)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources() + [MEMBENCH_SRC]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], MEMBENCH_LIB)
    if verbose:
        print(f"built {LIB} and {MEMBENCH_LIB}")
    return LIB


# The host-side sanitizers for the checked build below: each flag goes to the
# host compilation only (the kernels are built as usual).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all"]


def build_host_checked(out_dir: str) -> str:
    """A copy of libpa_verify.so whose host code (argument checks, planner,
    launch set-up: csrc/pa_verify.hip) is built with AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the kernel objects of the regular
    build (which must exist: run build() first).  Load it only in a process
    that preloads clang's ASan runtime (``asan_runtime()``).  Returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    host = os.path.join(CSRC, "pa_verify.hip")
    kernels = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in sources() if s != host]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        raise RuntimeError(f"regular build objects missing ({missing[0]}): run build() first")
    obj = os.path.join(out_dir, "pa_verify_checked.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    r = subprocess.run([hipcc(), *flags, *HOST_SANITIZE, "-c", host, "-o", obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {host}:\n{r.stderr}")
    out = os.path.join(out_dir, "libpa_verify_checked.so")
    _link([obj] + kernels, out)
    return out


def asan_runtime() -> str:
    """clang's shared ASan runtime (it carries the UBSan handlers too)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for base in (os.path.join(root, "llvm"), root, "/opt/rocm/llvm"):
        hits = sorted(glob.glob(os.path.join(base, "lib", "clang", "*", "lib", "linux",
                                             "libclang_rt.asan-x86_64.so")))
        if hits:
            return hits[-1]
    raise RuntimeError("clang's ASan runtime not found")


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)
