"""Builds the HIP library libconvfwd.so (gfx950) in the package directory.

    python -m convolution_forward_implicit_amd.build

Flags: -O3 for gfx950 only; packed-fp32 instruction selection is switched
off (-packed-fp32-ops), so the compiler emits no v_pk_*_f32 on its own.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "conv_fwd.hip")]
LIB = os.path.join(HERE, "libconvfwd.so")
# peak-rate probes (measured roofline denominators for the benchmark)
PROBE_SOURCES = [os.path.join(HERE, "csrc", "peak_probe.hip")]
PROBE_LIB = os.path.join(HERE, "libconvprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _compile(sources, lib, verbose):
    cmd = [HIPCC] + FLAGS + ["-o", lib + ".tmp"] + sources
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the gfx950-only feature and says so
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if out.strip():
        print(out, file=sys.stderr)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d)" % r.returncode)
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False) -> str:
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    _compile(SOURCES, LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
