"""Builds libpkv.so in place with hipcc for gfx950.

    python -m paged_kv_chunked_amd.build

Every translation unit is compiled (in parallel) to an object under
``paged_kv_chunked_amd/_build`` and linked into
``paged_kv_chunked_amd/libpkv.so``.  Device code is built with packed-fp32
instructions disabled (``-packed-fp32-ops``); the host pass warns that it does
not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")
ARCH = "gfx950"
SOURCES = ["host.cpp", "api.hip", "append.hip", "decode.hip", "chunk.hip", "mixed.hip",
           "generic.hip", "copy.hip", "stream.hip"]
# Per-file device flags.  The chunk kernel never lets a NaN reach a max (masked
# scores are replaced by -inf with a select, V past the sequence is zeroed as
# integers), so its device code may drop the quieting of max operands.  The
# mixed-batch kernel runs the same chunk code and is built the same way; its
# work-queue atomic must stay a plain atomic whose result is awaited only where
# it is used (the compiler's wave aggregation of atomics would wait at once);
# that backend option is passed to the compiler as is.
EXTRA_DEVICE_FLAGS = {"chunk.hip": ["-fno-honor-nans"], "mixed.hip": ["-fno-honor-nans"]}
EXTRA_FLAGS = {"mixed.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


HEADER = os.path.join(os.path.dirname(HERE), "include", "pkv.h")


def source_files():
    """Every file the library is built from: the kernel sources and the C header."""
    names = sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".h", ".cpp")))
    return [os.path.join(CSRC, n) for n in names] + [HEADER]


def source_hash() -> str:
    """SHA-256 of the sources (name and bytes of each file) and of the flag set;
    embedded in the library as pkv_source_hash() and checked when it loads."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    flags = {"arch": ARCH, "sources": SOURCES, "common": _flag_set(),
             "device": EXTRA_DEVICE_FLAGS, "extra": EXTRA_FLAGS}
    h.update(repr(sorted(flags.items())).encode())
    return h.hexdigest()


def _flag_set():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv)")


def common_flags():
    return _flag_set() + ["-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + common_flags()
    cmd.append(f'-DPKV_SOURCE_HASH="{digest}"')
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    for f in EXTRA_DEVICE_FLAGS.get(src, []):
        cmd += ["-Xarch_device", f]
    cmd += EXTRA_FLAGS.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    digest = source_hash()
    with cf.ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, digest), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp, f"--offload-arch={ARCH}"] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
