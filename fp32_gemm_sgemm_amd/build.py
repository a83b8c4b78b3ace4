"""Build libsgemm.so in-tree with hipcc for gfx950.

    python -m fp32_gemm_sgemm_amd.build [--save-temps DIR]

Always recompiles.  All device code is built with packed-FP32 instruction
selection switched off (-target-feature -packed-fp32-ops); the host pass
warns that it does not know that feature, which is harmless.

Besides the product library it builds the measurement probes
(libsgemm_probes.so) and the LDS race check build of the same sources
(libsgemm_lds_poison.so, SGEMM_LDS_POISON=1: LDS words are set to NaN before
each refill), which only the tests load, and the timeline build
(libsgemm_timeline.so, SGEMM_TIMELINE=1: clock readings per workgroup and per
K slice, read through include/sgemm_timeline.h).  The four compile in
parallel.
"""
import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsgemm.so")
PROBES_LIB = os.path.join(HERE, "libsgemm_probes.so")
POISON_LIB = os.path.join(HERE, "libsgemm_lds_poison.so")
TIMELINE_LIB = os.path.join(HERE, "libsgemm_timeline.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "sgemm.hip")]
PROBE_SOURCES = [os.path.join(CSRC, "probes.hip")]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc(out, sources, save_temps=None, verbose=False, extra=()):
    """Start one compilation; returns (process, output path)."""
    cmd = [HIPCC, *FLAGS, *extra]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd += ["-save-temps=cwd", "-Rpass-analysis=kernel-resource-usage"]
    cmd += ["-o", out + ".tmp", *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, cwd=save_temps or HERE), out


def build(save_temps: str = None, verbose: bool = False, extra=()) -> str:
    """Compile libsgemm.so (the product), libsgemm_probes.so (measurement
    probes), libsgemm_lds_poison.so (the LDS race check build) and
    libsgemm_timeline.so (the timeline build); returns the product library's
    path.  With save_temps, only the product library is
    built (its intermediate files go there)."""
    jobs = [_hipcc(LIB, SOURCES, save_temps, verbose, extra)]
    if not save_temps:
        jobs.append(_hipcc(PROBES_LIB, PROBE_SOURCES, None, verbose, extra))
        jobs.append(_hipcc(POISON_LIB, SOURCES, None, verbose,
                           ("-DSGEMM_LDS_POISON=1", *extra)))
        jobs.append(_hipcc(TIMELINE_LIB, SOURCES, None, verbose,
                           ("-DSGEMM_TIMELINE=1", *extra)))
    failed = []
    for proc, out in jobs:
        if proc.wait() != 0:
            failed.append(out)
        else:
            os.replace(out + ".tmp", out)
    if failed:
        raise subprocess.CalledProcessError(1, "hipcc", f"failed to build {failed}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None,
                    help="directory for intermediate files (assembly, resource usage)")
    args = ap.parse_args(argv)
    print(build(save_temps=args.save_temps, verbose=True))
    return 0


if __name__ == "__main__":
    sys.exit(main())
