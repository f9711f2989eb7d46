"""Builds libtq.so (host C++ + gfx950 HIP kernels) in-tree with hipcc, and a
host-sanitizer build of the same library for the CPU tests."""
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
KERNELS_OBJ = os.path.join(HERE, "tq_kernels.o")   # kept for the sanitizer build
HOST_OBJ = os.path.join(HERE, "tq_host.o")

# Device code is built for gfx950 only, without packed-fp32 instructions.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for tq_host.cpp
# (the host code only: every -fsanitize flag is behind -Xarch_host).
SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


def hipcc_path():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _compile(src, obj, extra=(), verbose=False):
    tmp = obj + ".tmp"
    _run([hipcc_path(), *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src),
          "-o", tmp], verbose)
    os.replace(tmp, obj)


def build(verbose: bool = False) -> str:
    _compile("tq_kernels.hip", KERNELS_OBJ, verbose=verbose)
    _compile("tq_host.cpp", HOST_OBJ, verbose=verbose)
    tmp = LIB + ".tmp"
    _run([hipcc_path(), *FLAGS, "-shared", HOST_OBJ, KERNELS_OBJ, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def sanitizer_runtime() -> str:
    """The compiler's AddressSanitizer runtime, to preload into the process
    that loads the sanitizer build."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/*/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found")
    return hits[-1]


def build_sanitized(out_dir: str, verbose: bool = False) -> str:
    """libtq with tq_host.cpp built under ASan + UBSan (device code as in
    build()), written to out_dir/libtq_asan.so."""
    if not os.path.exists(KERNELS_OBJ):
        _compile("tq_kernels.hip", KERNELS_OBJ, verbose=verbose)
    host = os.path.join(out_dir, "tq_host_asan.o")
    _compile("tq_host.cpp", host, extra=SANITIZE, verbose=verbose)
    lib = os.path.join(out_dir, "libtq_asan.so")
    _run([hipcc_path(), *FLAGS, *SANITIZE, "-shared", host, KERNELS_OBJ, "-o", lib], verbose)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
