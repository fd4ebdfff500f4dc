"""Host code under AddressSanitizer and UBSan (CPU only).

The oracle is built with gcc and the library's host pass with hipcc, each
with -fsanitize=address,undefined, and driven by a small C / C++ program
(tests/asan/): the oracle on seeded small shapes, the library's planner on
thousands of seeded shapes and every forced plan, and the argument checks of
every entry point.  No device is used.  A sanitizer report aborts the
driver, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, "%s\n%s%s" % (" ".join(cmd), res.stdout[-3000:], res.stderr[-3000:])
    return res.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-O1", "-g", "-fopenmp", *SAN, os.path.join(HERE, "asan", "oracle_driver.c"),
         os.path.join(ROOT, "oracle", "conv_ref.c"), "-lm", "-o", exe])
    out = run([exe], env=dict(ENV, OMP_NUM_THREADS="2"))
    assert "shapes" in out


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="hipcc is not installed")
def test_library_host_code_under_sanitizers(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    csrc = os.path.join(ROOT, "convolution_implicit_gemm_fwd_amd", "csrc")
    host_san = []
    for f in SAN:                       # host pass only: the device code is not instrumented
        host_san += ["-Xarch_host", f]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    objs = []
    for src, extra in (("conv2d_fwd.hip", []),
                       ("conv2d_wgrad.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"])):
        obj = str(tmp_path / (src + ".o"))
        run([hipcc, *common, *host_san, *extra, "-c", os.path.join(csrc, src), "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_driver.o")
    run([hipcc, *common, *host_san, "-c", os.path.join(HERE, "asan", "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    run([hipcc, "--offload-arch=gfx950", *host_san, drv, *objs, "-o", exe])
    out = run([exe], env=ENV)
    assert "0 unexpected statuses" in out
