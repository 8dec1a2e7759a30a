"""Build libcgd.so (HIP, gfx950) in place with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcgd.so")
ARCH = os.environ.get("CGD_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 instructions (v_pk_*_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# A second launch geometry for the same kernels (waves per block, vectors per
# lane, slots per wave, chunk widths, no prefetch blocks): a library built
# with it must produce the same bytes as the default one, which a GPU test
# checks. It is built beside libcgd.so by the package's build step.
GEOMETRY_LIB = os.path.join(PKG, "libcgd_geometry.so")
GEOMETRY_FLAGS = [
    "-DCGD_COMBINE_WAVES=2", "-DCGD_COMBINE_U=2", "-DCGD_COMBINE_LDS_CAP=16384", "-DCGD_COMBINE_LDS_WIDE=40960",
    "-DCGD_PREFETCH_BLOCKS=0", "-DCGD_ROW_SLOTS=1", "-DCGD_LAYOUT_TILE=128", "-DCGD_DIRECT_TOPK=0",
    "-DCGD_CAST_CPL=8", "-DCGD_SCATTER_CAST_U=1",
    "-DCGD_NORMAL_COMBINE_U=1", "-DCGD_NORMAL_COMBINE_WAVES=2", "-DCGD_NORMAL_GATHER=4", "-DCGD_NORMAL_SCATTER_U=2",
    "-DCGD_NORMAL_COMBINE_LDS_WIDE=24576", "-DCGD_ROW_COPY_PF_WAVES=8", "-DCGD_ROW_COPY_PF_LDS=0",
    "-DCGD_ROW_COPY_PF_LDS_WIDE=40960", "-DCGD_SCATTER_CAST_LDS=0",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra: list[str] | None = None, out: str | None = None) -> str:
    """Compile every source into one shared library: the package's libcgd.so,
    or `out` (e.g. a build with other tuning macros or host sanitizers,
    given as `extra` flags)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = out or LIB
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *(extra or []), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build_geometry_variant(verbose: bool = False) -> str:
    return build(verbose=verbose, extra=GEOMETRY_FLAGS, out=GEOMETRY_LIB)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_geometry_variant(verbose=True))
