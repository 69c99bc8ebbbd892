"""Resource checks on the built kernels (CPU only): the code-object metadata
of libfa2.so, read with ROCm's llvm tools.

Each kernel family is sized for a number of waves per SIMD; a register count
over that budget halves the occupancy, and spills put scratch traffic in the
loop.  Both change performance without changing results, so no parity test
sees them; this does.  The budgets: two waves per SIMD (at most 256 VGPRs,
architectural plus accumulation registers) for every kernel; LDS within the
160 KiB a workgroup may use.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from flashattention_forward_tile_amd import _build

LLVM = "/opt/rocm/llvm/bin"
OBJDUMP = os.path.join(LLVM, "llvm-objdump")
READELF = os.path.join(LLVM, "llvm-readelf")
LDS_LIMIT = 160 * 1024

NAME = re.compile(r"fa2_fwd_kernelILi(\d+)ELb(\d)ELi(\d)ELb(\d)ELi(\d)ELb(\d)ELb(\d)ELb(\d)E")


def field(entry, key):
    m = re.search(r"\.%s:\s+(\d+)" % key, entry)
    return int(m.group(1)) if m else 0


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(_build.LIB):
        pytest.skip("libfa2.so is not built")
    if not (os.access(OBJDUMP, os.X_OK) and os.access(READELF, os.X_OK)):
        pytest.skip("ROCm llvm tools not found")
    tmp = tempfile.mkdtemp()
    try:
        lib = os.path.join(tmp, "libfa2.so")
        shutil.copy(_build.LIB, lib)
        subprocess.run([OBJDUMP, "--offloading", lib], cwd=tmp, check=True,
                       capture_output=True)
        objs = [f for f in os.listdir(tmp) if f.endswith("gfx950")]
        assert len(objs) == 1, objs
        notes = subprocess.run([READELF, "--notes", os.path.join(tmp, objs[0])],
                               check=True, capture_output=True, text=True).stdout
    finally:
        shutil.rmtree(tmp)
    out = {}
    for entry in re.split(r"\n\s+- \.agpr_count:", notes)[1:]:
        name = re.search(r"\.name:\s+(\S+)", entry).group(1)
        m = NAME.search(name)
        if not m:
            continue
        d, fp16, mode, causal, q8, short, persist, split = (int(x) for x in m.groups())
        out[(d, fp16, mode, causal, q8, short, persist, split)] = {
            "agpr": int(entry.split("\n", 1)[0].strip()),
            "vgpr": field(entry, "vgpr_count"),
            "vgpr_spill": field(entry, "vgpr_spill_count"),
            "scratch": field(entry, "private_segment_fixed_size"),
            "lds": field(entry, "group_segment_fixed_size"),
        }
    return out


def test_every_kernel_is_present(kernels):
    # per (d, cache (0 none, 1 INT8, 2 FP8), half-height, persistent, key
    # splits): 2 dtypes x 3 scale-sign modes, with and without the mask
    families = {(64, 0, 0, 0, 0): 12, (64, 0, 0, 1, 0): 6, (128, 0, 0, 0, 0): 12,
                (128, 0, 1, 0, 0): 12, (128, 0, 0, 1, 0): 12, (128, 1, 0, 0, 0): 12,
                (128, 2, 0, 0, 0): 12, (256, 0, 0, 0, 0): 12,
                (64, 0, 0, 0, 1): 12, (128, 0, 1, 0, 1): 12, (256, 0, 0, 0, 1): 12,
                (128, 1, 1, 0, 1): 12, (128, 2, 1, 0, 1): 12,
                (64, 1, 0, 0, 0): 12, (64, 2, 0, 0, 0): 12, (64, 1, 1, 0, 1): 12,
                (64, 2, 1, 0, 1): 12, (256, 1, 0, 0, 0): 12, (256, 2, 0, 0, 0): 12,
                (256, 1, 1, 0, 1): 12, (256, 2, 1, 0, 1): 12}
    count = {}
    for (d, fp16, mode, causal, q8, short, persist, split) in kernels:
        key = (d, q8, short, persist, split)
        count[key] = count.get(key, 0) + 1
    assert count == families


def test_lds_fits_a_workgroup(kernels):
    for k, r in kernels.items():
        assert 0 < r["lds"] <= LDS_LIMIT, (k, r)


def test_two_waves_per_simd(kernels):
    """Every kernel fits two waves per SIMD (at most 256 registers, no
    spills); d = 256 gets there with 16-query waves on 16x16x32 MFMA."""
    for k, r in kernels.items():
        assert r["vgpr"] + r["agpr"] <= 256 and r["vgpr_spill"] == 0 and r["scratch"] == 0, (k, r)


def test_head_dim_256_lds_is_the_two_rings(kernels):
    """d = 256: four-slot K and V rings of 32-key tiles (128 KiB) and nothing
    else (the output is staged in the rings after the loop), so one
    workgroup of 8 waves runs per CU.  The quantized caches hold 8-bit K
    tiles and an 8-bit V staging ring beside the 16-bit V ring: the same
    128 KiB."""
    for k, r in kernels.items():
        if k[0] == 256:
            assert r["lds"] == 4 * 2 * 32 * 256 * 2 == 128 * 1024, (k, r)
