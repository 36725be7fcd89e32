"""Build libavsg.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libavsg.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_LIB = "/opt/rocm/lib"
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libavsg.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + [
        "-L" + ROCM_LIB, "-lrocprofiler-sdk-roctx", "-Wl,-rpath," + ROCM_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


NATIVE_SRC = os.path.join(HERE, "..", "tests", "native", "avsg_native_steps.cpp")
NATIVE_BIN = os.path.join(HERE, "..", "tests", "native", "avsg_native_steps")


def build_native_test(verbose: bool = False) -> str:
    """Compile the test program that calls libavsg through its C ABI alone
    (linked against the in-tree library, found through its rpath)."""
    tmp = NATIVE_BIN + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-O2", "-std=c++17", "-o", tmp, NATIVE_SRC,
           "-L" + HERE, "-lavsg", "-Wl,-rpath,$ORIGIN/../../device_buffer_reuse_amd"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("native test build failed:\n%s" % r.stderr)
    os.replace(tmp, NATIVE_BIN)
    if verbose:
        print("built", os.path.normpath(NATIVE_BIN))
    return NATIVE_BIN


def needs_build() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    srcs = glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(HERE, "..", "include", "*.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


if __name__ == "__main__":
    build(verbose=True)
