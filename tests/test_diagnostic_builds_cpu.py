"""The LDS race check build is not vacuous: compiled for gfx950 with
SGEMM_LDS_POISON=1, every kernel that reads LDS writes the quiet-NaN pattern
into it, and the normal build writes it nowhere (its kernels are untouched).
Host-only: hipcc emits the device assembly without a GPU."""
import os
import re
import subprocess

import pytest

from fp32_gemm_sgemm_amd import build

NAN_BITS = "0x7fc00000"


def start_device_asm(out, defines=()):
    """Start hipcc emitting the device assembly of the library to `out`."""
    cmd = [build.HIPCC, f"--offload-arch={build.ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{build.INCLUDE}", f"-I{build.CSRC}", "--cuda-device-only", "-S",
           *defines, "-o", out, *build.SOURCES]
    return subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)


def kernels(asm):
    """Kernel name -> assembly body."""
    out = {}
    for m in re.finditer(r"\n(_Z\w+):", asm):
        end = asm.find(".Lfunc_end", m.end())
        out[m.group(1)] = asm[m.end():end if end > 0 else len(asm)]
    return out


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("asm")
    outs = [str(tmp / "normal.s"), str(tmp / "poison.s")]
    jobs = [start_device_asm(outs[0]), start_device_asm(outs[1], ["-DSGEMM_LDS_POISON=1"])]
    for j in jobs:
        assert j.wait() == 0, "hipcc failed"
    return tuple(kernels(open(o).read()) for o in outs)


def test_every_lds_kernel_is_poisoned(builds):
    normal, poisoned = builds
    assert set(normal) == set(poisoned)
    lds_kernels = [k for k, body in poisoned.items() if re.search(r"\bds_read", body)]
    assert len(lds_kernels) >= 20
    for k in lds_kernels:
        assert NAN_BITS in poisoned[k], f"{k}: no NaN written to LDS in the race check build"
        assert re.search(r"\bds_write", poisoned[k]), k


def test_normal_build_carries_no_poison(builds):
    normal, _ = builds
    for k, body in normal.items():
        assert NAN_BITS not in body, k
