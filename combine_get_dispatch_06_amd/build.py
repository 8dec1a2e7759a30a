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


if __name__ == "__main__":
    print(build(verbose=True))
