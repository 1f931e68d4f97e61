"""Build the gfx950 HIP library in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled to an object twice, in parallel: once
for the release library ``paged_kv_decode_reshape_amd/libpkv.so`` and once
with ``PKV_DEBUG=1`` for ``libpkv_debug.so``, whose kernels check the values
they read from caller buffers (block ids, context lengths, slots, chunk
bounds) before forming addresses from them. Objects go to ``_build/``.

``build_sanitized()`` links a third, CPU-test-only library,
``_build/sanitize/libpkv_sanitize.so``: the host code of ``host.hip`` (the
C-ABI argument checks, layouts and workspace sizing) compiled with
AddressSanitizer and UndefinedBehaviorSanitizer, the device code and the other
objects as in the release build. It is loaded with the sanitizer runtime
preloaded, on the CPU only.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBS = {"release": os.path.join(PKG, "libpkv.so"), "debug": os.path.join(PKG, "libpkv_debug.so")}
LIB = LIBS["release"]
SANITIZED_LIB = os.path.join(BUILD, "sanitize", "libpkv_sanitize.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU ops are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-command-line-argument"] + DEVICE_FLAGS
VARIANT_FLAGS = {"release": [], "debug": ["-DPKV_DEBUG=1"]}
# Host-only sanitizers: each -fsanitize= is preceded by -Xarch_host, so the
# device code is built exactly as in the release library.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _obj(variant: str, src: str) -> str:
    return os.path.join(BUILD, variant, os.path.basename(src) + ".o")


def build(verbose: bool = False, variants=("release", "debug")) -> str:
    """Compile and link the given library variants; returns the release library's path."""
    sources = _sources()
    jobs = []
    for v in variants:
        os.makedirs(os.path.join(BUILD, v), exist_ok=True)
        jobs += [(v, s) for s in sources]

    def compile_one(job):
        v, src = job
        cmd = [HIPCC, *COMMON, *VARIANT_FLAGS[v], "-c", src, "-o", _obj(v, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)

    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(compile_one, jobs))
    for v in variants:
        out = LIBS[v]
        tmp = out + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[_obj(v, s) for s in sources], "-o", tmp])
        os.replace(tmp, out)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """host.hip with host-side ASan + UBSan, linked with the release objects of
    the kernel sources (build() must have run). CPU tests only."""
    os.makedirs(os.path.dirname(SANITIZED_LIB), exist_ok=True)
    host_src = os.path.join(CSRC, "host.hip")
    host_obj = os.path.join(os.path.dirname(SANITIZED_LIB), "host.hip.o")
    cmd = [HIPCC, *COMMON, *SANITIZE_FLAGS, "-c", host_src, "-o", host_obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    others = [_obj("release", s) for s in _sources() if os.path.basename(s) != "host.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"release objects missing ({missing}): run build() first")
    tmp = SANITIZED_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE_FLAGS, host_obj, *others, "-o", tmp])
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose=True))
