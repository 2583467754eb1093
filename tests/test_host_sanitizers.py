"""The library's host code (argument checks, schedule planning, workspace
sizing) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

A copy of the library whose host half is instrumented (its GPU code is built
as usual and never runs here) is loaded in a child process with the sanitizer
runtime preloaded, and the host ABI tests run against it there: every
argument check, including sizes at the limits of what an operand can span.
A sanitizer finding ends the child with an error. The copy lives under the
build folder and is rebuilt only when a source, header or flag changes."""
import hashlib
import os
import subprocess
import sys

import pytest
import torch

from lora_rank_adapter_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(B.BUILD_DIR, "host-sanitize")
SAN_LIB = os.path.join(SAN_DIR, B.LIB_NAME)
# host-only instrumentation: each sanitizer flag applies to the host pass
SAN_FLAGS = [f for f in B.HIPCC_FLAGS if f != "-O3"] + [
    "-O1",
    "-Xarch_host", "-g",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
]

pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="host-only checks (fake device pointers)")


def _asan_runtime():
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        return None
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(cand):
            res = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = res.stdout.strip()
            if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    return None


def _digest():
    h = hashlib.sha256(" ".join(SAN_FLAGS).encode())
    for f in B.SOURCES + B.HEADERS:
        with open(os.path.join(B.CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    with open(os.path.join(ROOT, "include", "lora.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()


def _build_sanitized():
    stamp = os.path.join(SAN_DIR, "digest")
    digest = _digest()
    if os.path.exists(SAN_LIB) and os.path.exists(stamp) and open(stamp).read().strip() == digest:
        return SAN_LIB
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = []
    procs = []
    for src in B.SOURCES:
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [B.hipcc(), *SAN_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(B.CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for src, p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, f"sanitized build of {src} failed:\n{out}\n{err}"
    res = subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs, "-o", SAN_LIB],
                         capture_output=True, text=True)
    assert res.returncode == 0, f"sanitized link failed:\n{res.stdout}\n{res.stderr}"
    with open(stamp, "w") as fh:
        fh.write(digest + "\n")
    return SAN_LIB


RUNNER = """
import sys
import lora_rank_adapter_amd.build as b
b.LIB_PATH = sys.argv[1]
b.is_stale = lambda: False
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", sys.argv[2]]))
"""


def test_host_abi_checks_under_asan_and_ubsan():
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("no hipcc, or no AddressSanitizer runtime next to its clang")
    lib = _build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PYTHONPATH": ROOT + os.pathsep + env.get("PYTHONPATH", ""),
    })
    res = subprocess.run([sys.executable, "-c", RUNNER, lib, os.path.join(ROOT, "tests", "test_abi_host.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in res.stdout and " failed" not in res.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
