"""Build libsgemm.so in-tree with hipcc for gfx950.

    python -m fp32_gemm_sgemm_amd.build [--save-temps DIR]

Always recompiles.  All device code is built with packed-FP32 instruction
selection switched off (-target-feature -packed-fp32-ops); the host pass
warns that it does not know that feature, which is harmless.
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
    cmd = [HIPCC, *FLAGS, *extra]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd += ["-save-temps=cwd", "-Rpass-analysis=kernel-resource-usage"]
    cmd += ["-o", out + ".tmp", *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=save_temps or HERE)
    os.replace(out + ".tmp", out)
    return out


def build(save_temps: str = None, verbose: bool = False, extra=()) -> str:
    """Compile libsgemm.so (the product) and libsgemm_probes.so (measurement
    probes); returns the product library's path."""
    _hipcc(LIB, SOURCES, save_temps, verbose, extra)
    _hipcc(PROBES_LIB, PROBE_SOURCES, save_temps, verbose, extra)
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
