"""Build libssmscan.so in-tree with hipcc for gfx950.

    python -m selective_state_space_fwd_amd.build

Every HIP source is compiled with the packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass warns that it does
not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libssmscan.so")
# The VALU throughput probes bench.py --alu-probe runs; a library of their own.
PROBE_SOURCE = os.path.join(PKG, "probes", "alu_probe.hip")
PROBE_LIB_PATH = os.path.join(PKG, "libssmprobe.so")
SOURCES = ["scan_kernels.hip", "scan_short.hip", "scan_bwd.hip", "ssd_kernels.hip", "scan_api.cpp",
           "ssd_api.cpp", "ssd_noalloc.hip"]
# A test-only build of the Mamba-1 scan with a second launch shape of the chunked kernel (the
# same 16 steps per lane, other channels per workgroup and states per LDS stage), which the
# parity tests run against the oracle and against the default build.
SHAPE2_LIB_PATH = os.path.join(PKG, "libssmscan_shape2.so")
SHAPE2_SOURCES = ["scan_kernels.hip", "scan_short.hip", "scan_bwd.hip", "scan_api.cpp"]
SHAPE2_DEFINES = ["-DSSM_BF16_K=4", "-DSSM_BF16_G=4", "-DSSM_F32_K=2", "-DSSM_F32_G=1"]
ARCH = "gfx950"


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def compile_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fvisibility=hidden", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _link(sources, target, verbose, extra=()):
    fd, tmp = tempfile.mkstemp(prefix=os.path.basename(target) + ".", suffix=".tmp", dir=PKG)
    os.close(fd)
    cmd = [hipcc(), *compile_flags(), *extra, "-shared", "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=PKG, capture_output=True, text=True)
    if r.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    os.replace(tmp, target)
    return target


def build(verbose: bool = False) -> str:
    """Build libssmscan.so (the scan library), libssmprobe.so (the VALU probes) and
    libssmscan_shape2.so (the test-only second launch shape)."""
    _link([PROBE_SOURCE], PROBE_LIB_PATH, verbose)
    _link([os.path.join(CSRC, s) for s in SHAPE2_SOURCES], SHAPE2_LIB_PATH, verbose,
          SHAPE2_DEFINES)
    return _link([os.path.join(CSRC, s) for s in SOURCES], LIB_PATH, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
