"""Build libvlf.so in-tree: the gfx950 kernels (hipcc) and the host index code (g++); and
libvlf_probe.so, the matrix-unit probe the benchmark reads its measured peak from.

    python -m variable_length_flash_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIBRARY = os.path.join(HERE, "libvlf.so")
PROBE_LIBRARY = os.path.join(HERE, "libvlf_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 instructions stay off: hipcc forms them from ordinary float code otherwise.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    kernel_obj = os.path.join(BUILD, "vlf_attend.o")
    host_obj = os.path.join(BUILD, "vlf_host.o")
    _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "vlf_attend.hip"), "-o", kernel_obj], verbose)
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-c",
          os.path.join(CSRC, "vlf_host.cpp"), "-o", host_obj], verbose)
    tmp = LIBRARY + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", kernel_obj, host_obj, "-o", tmp],
         verbose)
    os.replace(tmp, LIBRARY)
    tmp = PROBE_LIBRARY + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", os.path.join(CSRC, "vlf_probe.hip"), "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
