"""Compiles libbsa.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

    python -m block_sparse_attention_avg_amd._build

Objects go to ``_build/`` next to this file; the shared library is written
into the package directory, where the binding loads it from.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbsa.so")
PROBE = os.path.join(PKG, "mfma_probe")
ARCH = "gfx950"

SOURCES = ["api.cpp", "pool.hip", "select.hip", "attn_fwd.hip", "attn_fwd_1w.hip", "attn_bwd.hip",
           "diag.hip", "permute.hip", "kmeans.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-source flags. The attention kernels assume finite inputs: without NaN
# semantics their running row maxima need no quieting of the MFMA results
# (one v_max_f32 per score fewer).
EXTRA = {"attn_fwd.hip": ["-fno-honor-nans"], "attn_fwd_1w.hip": ["-fno-honor-nans"]}


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the whole
# library (device code is built as usual): the argument checks, descriptor
# conversions and host functions of the C ABI run instrumented on the CPU.
SAN_OUT = os.path.join(OUT, "san")
SAN_LIB = os.path.join(OUT, "libbsa_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile(src: str, sanitize: bool = False) -> str:
    out = SAN_OUT if sanitize else OUT
    obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *EXTRA.get(src, []), *(SAN_FLAGS if sanitize else []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build_sanitized(verbose: bool = False) -> str:
    """Builds _build/libbsa_san.so (host code under ASan + UBSan). It needs the
    sanitizer runtime preloaded (asan_runtime()) in the process that loads it."""
    os.makedirs(SAN_OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 6)) as ex:
        objs = list(ex.map(lambda src: _compile(src, True), SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime."""
    r = subprocess.run([os.path.join(os.path.dirname(_hipcc()), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("shared AddressSanitizer runtime not found")
    return path


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 6)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    # measurement helper for bench.py (a program, not part of the library)
    cmd = [_hipcc(), *FLAGS, "-x", "hip", os.path.join(CSRC, "mfma_probe.hip"), "-o", PROBE + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for mfma_probe.hip:\n{r.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    if verbose:
        print(f"built {LIB} and {PROBE}")
    return LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
