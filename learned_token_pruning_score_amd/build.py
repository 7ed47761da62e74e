"""Build libtokengate.so in-tree with hipcc for gfx950.

Usage: ``python -m learned_token_pruning_score_amd.build`` (or call
``build_library()``).  Every call recompiles every source.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libtokengate.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["tg_api.hip", "gate.hip", "select.hip", "compact.hip", "attn.hip", "attn_bwd.hip", "proj.hip", "gate_bwd.hip", "decode.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 vector ops stay off: the compiler must not form them.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libtokengate.so)")


def _compile(src: str, verbose: bool, build_dir: str, extra) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build_library(verbose: bool = False, extra_flags=(), out_path: str = LIB_PATH) -> str:
    """Compile every HIP source and link the shared library; returns its path.

    ``extra_flags`` are passed to every compile (e.g. ``-g``);
    ``out_path`` places the library elsewhere (objects go next to it).
    """
    build_dir = BUILD_DIR if out_path == LIB_PATH else os.path.splitext(out_path)[0] + "_obj"
    os.makedirs(build_dir, exist_ok=True)
    extra = list(extra_flags)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    tmp = out_path + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, out_path)
    return out_path


# Host code built with AddressSanitizer and UndefinedBehaviorSanitizer: every
# flag applies to the host compilation only (the device code is built as
# usual, without them), and undefined behaviour aborts instead of continuing.
SANITIZE_HOST_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-sanitize-recover=undefined "
                       "-Xarch_host -fno-omit-frame-pointer").split()
SANITIZED_DIR = os.path.join(PKG_DIR, "_build_san")


def build_host_sanitized(out_dir: str = SANITIZED_DIR) -> str:
    """Build the library's host code (argument checks, planning, workspace
    sizes, launch set-up) with ASan and UBSan into ``out_dir``; returns the
    path of the shared library.  It exists to run the host-side tests under
    the sanitizers; load it with the ASan runtime preloaded
    (``asan_runtime()``)."""
    os.makedirs(out_dir, exist_ok=True)
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             *SANITIZE_HOST_FLAGS]

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [_hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"sanitized host build failed for {src}:\n{' '.join(cmd)}\n"
                               f"{res.stdout}{res.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    out = os.path.join(out_dir, "libtokengate_san.so")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
           *SANITIZE_HOST_FLAGS[:4], "-shared-libsan", "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return out


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload into a process
    that loads the sanitized library)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    for pat in (os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"),
                os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    raise RuntimeError("shared ASan runtime not found next to hipcc")


if __name__ == "__main__":
    print(build_library(verbose=True))
