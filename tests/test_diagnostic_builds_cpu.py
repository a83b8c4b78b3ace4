"""The diagnostic builds are not vacuous and leave the normal build alone.
Compiled for gfx950 with SGEMM_LDS_POISON=1, every kernel that reads LDS writes
the quiet-NaN pattern into it; with SGEMM_TIMELINE=1, every direct-load kernel
reads the shader clock and no other kernel does.  The normal build contains
neither.  Host-only: hipcc emits the device assembly without a GPU."""
import os
import re
import subprocess

import pytest

from fp32_gemm_sgemm_amd import build

NAN_BITS = "0x7fc00000"
DL_KERNEL = "sgemm_mfma_dl_kernel"


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
    names = {"normal": (), "poison": ("-DSGEMM_LDS_POISON=1",),
             "timeline": ("-DSGEMM_TIMELINE=1",)}
    jobs = {n: (str(tmp / f"{n}.s"), start_device_asm(str(tmp / f"{n}.s"), d))
            for n, d in names.items()}
    for n, (_, j) in jobs.items():
        assert j.wait() == 0, f"hipcc failed for the {n} build"
    return {n: kernels(open(path).read()) for n, (path, _) in jobs.items()}


def test_every_lds_kernel_is_poisoned(builds):
    normal, poisoned = builds["normal"], builds["poison"]
    assert set(normal) == set(poisoned)
    lds_kernels = [k for k, body in poisoned.items() if re.search(r"\bds_read", body)]
    assert len(lds_kernels) >= 20
    for k in lds_kernels:
        assert NAN_BITS in poisoned[k], f"{k}: no NaN written to LDS in the race check build"
        assert re.search(r"\bds_write", poisoned[k]), k


def test_normal_build_carries_no_poison(builds):
    for k, body in builds["normal"].items():
        assert NAN_BITS not in body, k


def test_timeline_build_reads_the_clock_in_every_direct_load_kernel(builds):
    """Entry, loop start, two readings per slice, loop end and the end: at
    least four clock readings in each direct-load kernel, none elsewhere."""
    normal = builds["normal"]
    # the timeline build adds its two device arrays to the labels
    timeline = {k: b for k, b in builds["timeline"].items() if "g_tl_" not in k}
    assert set(normal) == set(timeline)
    dl = [k for k in timeline if DL_KERNEL in k]
    assert len(dl) >= 40
    for k, body in timeline.items():
        n = len(re.findall(r"\bs_memtime\b", body))
        if DL_KERNEL in k:
            assert n >= 4, f"{k}: {n} clock readings"
        else:
            assert n == 0, k


def test_normal_build_reads_no_clock(builds):
    for k, body in builds["normal"].items():
        assert not re.search(r"\bs_memtime\b", body), k
