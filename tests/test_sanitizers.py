"""Sanitizer builds of the CPU-side code (no GPU needed):

* the fp64 oracle (oracle/conv_oracle.c) with AddressSanitizer and
  UndefinedBehaviorSanitizer, driven over a grid of small 1-D/2-D/3-D
  problems through every entry point, each buffer allocated at its exact
  size (tests/sanitize/oracle_driver.c);
* the host code of the HIP library (descriptor validation, extents, the
  selector, plan creation for every configuration, chain and backward plans,
  and the argument checks of every run call) built with the same sanitizers
  on its host side only, driven by tests/sanitize/capi_driver.c, which
  launches nothing.

A sanitizer report makes the driver exit non-zero (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"   # the sanitizer runtime must be the one hipcc's host pass used
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=timeout)
    return r.returncode, r.stdout


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-ffp-contract=off"] + SAN +
                   ["-o", exe, os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "conv_oracle.c"),
                    "-lm"])
    assert rc == 0, out
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1")
    rc, out = _run([exe], env=env)
    assert rc == 0 and "oracle sanitize ok" in out, out[-4000:]


def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    if not os.path.exists(HIPCC) or not os.path.exists(CLANGXX):
        pytest.skip("hipcc or ROCm's clang++ not available")
    so = str(tmp_path / "libconvfwd_hostsan.so")
    # the sanitizers apply to the host pass only (each flag after -Xarch_host);
    # the gfx950 device code is built as usual
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san +
                   ["-I" + os.path.join(ROOT, "include"), "-o", so,
                    os.path.join(ROOT, "convolution_forward_implicit_amd", "csrc", "conv_fwd.hip")], timeout=900)
    assert rc == 0, out[-4000:]
    exe = str(tmp_path / "capi_driver")
    rc, out = _run([CLANGXX, "-O1", "-g", "-x", "c++"] + SAN + ["-I" + os.path.join(ROOT, "include"), "-o", exe,
                    os.path.join(HERE, "capi_driver.c"), "-x", "none", so, "-Wl,-rpath," + str(tmp_path)])
    assert rc == 0, out[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", HIP_VISIBLE_DEVICES="")
    rc, out = _run([exe], env=env)
    assert rc == 0 and "capi sanitize ok" in out, out[-4000:]
