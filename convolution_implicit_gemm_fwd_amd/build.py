"""Build libconvimg.so (HIP, gfx950) in-tree.

``python -m convolution_implicit_gemm_fwd_amd.build`` compiles the HIP
translation units with hipcc for gfx950 only (each with its own extra flags)
and links them into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libconvimg.so")
# (source, extra hipcc flags): the weight-backward kernel keeps its MFMA
# accumulators in VGPRs (fewer register copies in its loop, measured)
UNITS = [(os.path.join(CSRC, "conv2d_fwd.hip"), []),
         (os.path.join(CSRC, "conv2d_wgrad.hip"), ["-mllvm", "-amdgpu-mfma-vgpr-form"])]
SOURCES = [u[0] for u in UNITS]
DEPENDS = SOURCES + [os.path.join(CSRC, h) for h in ("igemm_common.hpp", "igemm_regs.hpp", "igemm_pipe.hpp", "igemm_patch.hpp", "igemm_strip.hpp", "igemm_window.hpp", "igemm_resident.hpp", "igemm_image.hpp", "igemm_dgrad.hpp", "igemm_wgrad.hpp", "igemm_layout.hpp")] + [os.path.join(INCLUDE, "convimg.h")]

ARCH = "gfx950"
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 instructions stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile the library (always) and return its path."""
    tag = "%d" % os.getpid()
    objs = []
    # the host pass does not know the packed-fp32 feature and says so
    noise = "'-packed-fp32-ops' is not a recognized feature"

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))

    try:
        # the translation units compile in parallel
        procs = []
        for src, flags in UNITS:
            obj = os.path.join(PKG, os.path.basename(src) + ".%s.o" % tag)
            objs.append(obj)
            flags_c = [f for f in HIPCC_FLAGS if f != "-shared"]
            cmd = [hipcc(), *flags_c, *flags, *extra_flags, "-I", INCLUDE, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                          text=True))
        failed = []
        for p in procs:
            out, _ = p.communicate()
            msgs = [ln for ln in out.splitlines() if noise not in ln]
            if p.returncode != 0:
                failed.append("\n".join(msgs))
            elif verbose and msgs:
                print("\n".join(msgs))
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        tmp = LIB + ".tmp" + tag
        run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra_flags=sys.argv[1:]))
