"""Compile the HIP kernels and host code into libkvpaged.so (gfx950), and
the plain-read measurement kernel into libkvprobe.so.

Every call recompiles. Objects go to ``_build/`` next to this file; the
libraries are written next to this file so they travel with the source tree.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
SOURCES = ["host.cpp", "prefix_cache.cpp", "vcache.cpp", "cache_ops.hip",
           "decode.hip", "decode_noalloc.hip", "prefill.hip"]
LIB = os.path.join(HERE, "libkvpaged.so")
# measurement only (the benchmark's read ceiling), not the attention API
PROBE_SOURCES = ["read_probe.hip"]
PROBE_LIB = os.path.join(HERE, "libkvprobe.so")
ARCH = os.environ.get("KVPAGED_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-Wall",
          "-Wno-unused-function"]
# Packed fp32 VALU ops are disabled for all device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]


def _compile(src: str, obj: str, extra=()) -> None:
    path = os.path.join(HERE, "csrc", src)
    cmd = [HIPCC] + COMMON + list(extra)
    if src.endswith(".hip"):
        cmd += ["-x", "hip"] + DEVICE
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n"
                           f"{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines()
             if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    shutil.move(tmp, lib)


def build(verbose: bool = False) -> str:
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in srcs]
    with ThreadPoolExecutor(len(srcs)) as ex:
        list(ex.map(lambda p: _compile(*p), zip(srcs, objs)))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB}")
        print(f"built {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
