"""Build the gfx950 latent-cache library in-tree: mla_latent_kv_cache_amd/libmla_latent.so.

    python -m mla_latent_kv_cache_amd.build        (or call build())

Every HIP translation unit is compiled with hipcc for gfx950 only, with packed-fp32 instruction
selection disabled, and linked into one shared library exposing the C ABI of include/mla.h.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla_latent.so")

SOURCES = ["api.cpp", "append.hip", "decode.hip", "prefill.hip"]
# the streaming-read ceiling kernel that bench.py measures HBM with, in a library of its own
BW_SOURCE = "bandwidth.hip"
BW_LIB = os.path.join(PKG, "libmla_bandwidth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same sources (device code is built as
# usual, only the host code is instrumented): the C ABI's argument validation runs under the sanitizers in the
# CPU test suite, with the sanitizer runtime preloaded.
SAN_BUILD = os.path.join(BUILD, "host_sanitized")
SAN_LIB = os.path.join(SAN_BUILD, "libmla_latent_hostsan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + [BW_SOURCE]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], BW_LIB)
    if verbose:
        print(f"built {LIB} and {BW_LIB}")
    return LIB


def build_host_sanitized(verbose: bool = True) -> str:
    """The library with its host code built under ASan + UBSan (SAN_LIB); load it only in a process whose
    sanitizer runtime is preloaded (sanitizer_runtime())."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, SAN_BUILD, SAN_FLAGS), SOURCES))
    _link(objs, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def sanitizer_runtime() -> str:
    """The compiler's shared ASan runtime (it also carries the UBSan handlers), to LD_PRELOAD."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the ASan runtime of the ROCm compiler was not found")
    return path


if __name__ == "__main__":
    build()
