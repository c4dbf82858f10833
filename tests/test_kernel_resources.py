"""CPU build checks of the direct-to-LDS kernels (no GPU):
representative instantiations of every code path (wide-N tiles, four and
two reduction groups, front-loaded loads, 16x16 and 32x32 bf16 blocks,
fp32 blocks over two sub-slices; with and without the bias + GELU
epilogue; and the patch kernels' configurations) are compiled for gfx950
and must use no scratch memory.  A helper
lambda that the compiler leaves as a call passes its captures through
scratch, which made such kernels 10-100x slower; an array of uint4 kept
across the epilogue's LDS reads and stores landed there too; register
spills show up the same way."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_forward_implicit_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# <DT, BM, BN, WM, WN, NS, MF, KSUB, KG, FL>
INSTANCES = [
    "1, 192, 384, 2, 4, 2, 32, 1, 1, 4",
    "1, 256, 256, 2, 4, 2, 32, 1, 1, 4",
    "0, 48, 48, 1, 1, 2, 16, 1, 4, 0",
    "0, 32, 32, 2, 2, 2, 16, 2, 2, 0",
    "0, 32, 32, 2, 2, 2, 16, 2, 1, 0",
    "0, 32, 64, 1, 4, 2, 16, 2, 1, 0",
    "1, 256, 64, 4, 1, 2, 32, 1, 1, 0",
    "1, 128, 64, 2, 2, 2, 16, 1, 1, 0",
    "1, 128, 128, 2, 2, 3, 32, 1, 1, 0",
]


# <TH, TW, BN, CC, NS, PHMAX, PWMAX, TAPMAX, PAD>
PATCH_INSTANCES = [
    "16, 32, 32, 16, 2, 20, 36, 9, 0",
    "8, 32, 64, 16, 2, 10, 34, 9, 1",
    "8, 32, 64, 16, 3, 10, 34, 9, 0",
    "8, 32, 64, 32, 2, 10, 34, 9, 0",
]


# <TH, TW, BN, CC, NS, FY, FX, DH, DW, NW, PM, RA, RR>
PFIX_INSTANCES = [
    "28, 32, 32, 16, 2, 3, 3, 2, 2, 4, 1, 1, 1",
    "16, 32, 32, 16, 2, 3, 3, 2, 2, 4, 0, 1, 1",
    "16, 28, 32, 16, 2, 3, 3, 2, 2, 2, 1, 1, 0",
    "8, 56, 64, 16, 2, 3, 3, 1, 1, 4, 1, 1, 0",
    "4, 56, 64, 16, 2, 3, 3, 1, 1, 4, 1, 1, 0",
    "8, 56, 64, 16, 2, 3, 3, 1, 1, 7, 1, 1, 0",
    "28, 32, 32, 16, 2, 3, 3, 2, 2, 14, 1, 1, 1",
    "28, 28, 32, 16, 2, 3, 3, 2, 2, 13, 1, 1, 0",
]


def _resource_usage(header, kernel, params, instances):
    lines = ['#include "%s"' % header, "namespace convfwd {"]
    for inst in instances:
        for ep in ("true, true", "false, false"):
            lines.append("template __global__ void %s<%s, %s>(%s);" % (kernel, inst, ep, params))
    lines.append("}")
    d = tempfile.mkdtemp()
    try:
        src = os.path.join(d, "inst.hip")
        with open(src, "w") as f:
            f.write("\n".join(lines) + "\n")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-c", "--cuda-device-only",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I" + CSRC, "-I" + os.path.join(ROOT, "include"),
               "-Rpass-analysis=kernel-resource-usage", src, "-o", os.path.join(d, "inst.o")]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
        assert r.returncode == 0, r.stdout[-3000:]
    finally:
        shutil.rmtree(d, ignore_errors=True)
    names = re.findall(r"Function Name: (\S+)", r.stdout)
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stdout)]
    spills = [int(v) for v in re.findall(r"VGPRs Spill: (\d+)", r.stdout)]
    assert len(names) == 2 * len(instances) == len(scratch) == len(spills), r.stdout[-2000:]
    return [(n, s, v) for n, s, v in zip(names, scratch, spills) if s or v]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_dma_kernels_use_no_scratch():
    bad = _resource_usage("igemm_dma.h", "igemm_dma_kernel", "DmaParams", INSTANCES)
    assert not bad, bad


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_patch_kernels_use_no_scratch():
    bad = _resource_usage("patch_kernel.h", "patch_conv_kernel", "PatchParams", PATCH_INSTANCES)
    assert not bad, bad


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_fixed_filter_patch_kernels_use_no_scratch():
    bad = _resource_usage("patch_fixed.h", "patch_fixed_kernel", "PatchFixedParams", PFIX_INSTANCES)
    assert not bad, bad
