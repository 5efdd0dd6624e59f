"""Build libmsm.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m selective_state_space_msm_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmsm.so")
# (source, extra flags): the recurrence kernels are built once per (bf16 I/O, variant) pair --
# variant 0 plain, 1 fused extras, 2 fused extras with the zero-order hold -- all in parallel
_PARTS = [("-DMSM_IO_BF16=%d" % io, "-DMSM_EXT=%d" % ext) for io in (0, 1) for ext in (0, 1, 2)]
SOURCES = ([("msm_api.cpp", ()), ("msm_launch.hip", ()), ("msm_bwd_wide.hip", ()),
            ("msm_step.hip", ()), ("msm_cfwd.hip", ()), ("msm_cbwd.hip", ())]
           + [("msm_fwd.hip", f) for f in _PARTS] + [("msm_bwd.hip", f) for f in _PARTS])

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed FP32 (v_pk_*_f32) is disabled for every HIP file this library compiles.
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-Wall", "-Wno-unused-command-line-argument"]


def _compile(src: str, flags) -> tuple[subprocess.Popen, str]:
    tag = "".join(f.split("=")[-1] for f in flags)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + (("." + tag) if tag else "") + ".o")
    cmd = [HIPCC, *COMMON, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libmsm.so.  Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    t0 = time.time()
    procs = [_compile(src, flags) for src, flags in SOURCES]
    objs, failed = [], []
    for (proc, obj), (src, flags) in zip(procs, SOURCES):
        out, _ = proc.communicate()
        # the host pass does not know the packed-fp32 target feature; that warning is harmless
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l]
        if proc.returncode != 0:
            failed.append((src + " " + " ".join(flags), "\n".join(lines)))
        elif verbose and lines:
            print("\n".join(lines))
        objs.append(obj)
    if failed:
        msg = "\n".join("%s:\n%s" % f for f in failed)
        raise RuntimeError("hipcc failed:\n" + msg)
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print("built %s in %.1fs" % (LIB, time.time() - t0))
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
