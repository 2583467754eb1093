"""Builds the gfx950 HIP library ``liblora_mi355x.so`` in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 instructions
disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "liblora_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
DIGEST_PATH = LIB_PATH + ".digest"   # digest of the sources the library was built from
SOURCES = ["lora_single.hip", "lora_multi.hip"]
HEADERS = ["lora_device.hpp", "lora_host.hpp"]

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the LoRA HIP library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def source_digest() -> str:
    """Digest of every source, header and compiler flag the library is built
    from (contents, not file times: a copied tree keeps it)."""
    h = hashlib.sha256(" ".join(HIPCC_FLAGS).encode())
    deps = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [os.path.join(ROOT, "include", "lora.h")]
    for d in deps:
        h.update(os.path.basename(d).encode())
        with open(d, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def built_digest():
    """The digest recorded by the last build, or None."""
    try:
        with open(DIGEST_PATH) as f:
            return f.read().strip()
    except OSError:
        return None


def build(verbose: bool = False) -> str:
    """Compile all sources and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    digest = source_digest()
    os.replace(tmp, LIB_PATH)
    with open(DIGEST_PATH, "w") as f:
        f.write(digest + "\n")
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


def is_stale() -> bool:
    """True when the library is missing or was built from other sources than
    the ones in the tree now."""
    return not os.path.exists(LIB_PATH) or built_digest() != source_digest()


if __name__ == "__main__":
    build(verbose=True)
