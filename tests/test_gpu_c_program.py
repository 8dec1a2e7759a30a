"""The boundary from C: tests/c/cgd_c_roundtrip.c includes only cgd.h (and the
HIP runtime header it needs), links libcgd, and checks layout, dispatch and
combine against the oracle on seeded inputs (one-launch, several-tile and
top-16 batches), and the one-call rank-granular layout + dispatch in bf16 and
with the FP8 cast (one tile and several), with no Python or torch in the
process. The CPU suite
compiles and links it; the GPU suite runs it."""
import os
import subprocess

import pytest

import combine_get_dispatch_06_amd as cgd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "cgd_c_roundtrip.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(out_dir) -> str:
    import oracle
    import synth
    libs = {}
    for name, mod in (("cgd", cgd), ("oracle", oracle), ("synth", synth)):
        if mod is cgd:
            cgd.load()
            path = cgd.library_path()
        else:
            mod._load()
            path = mod._LIB
        libs[name] = os.path.dirname(path)
    exe = os.path.join(str(out_dir), "cgd_c_roundtrip")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include", SRC, "-o", exe]
    for d in dict.fromkeys(libs.values()):
        cmd += [f"-L{d}", f"-Wl,-rpath,{d}"]
    cmd += ["-lcgd", "-loracle", "-lsynth", f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib", "-lamdhip64", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"gcc failed:\n{' '.join(cmd)}\n{res.stderr}"
    return exe


def test_c_program_compiles_and_links(tmp_path):
    """cgd.h is plain C: the program builds with gcc -Wall -Werror against
    the header and links against libcgd's exported symbols."""
    if cgd.library_path() != os.path.join(ROOT, "combine_get_dispatch_06_amd", "libcgd.so"):
        pytest.skip("another libcgd build is selected")
    assert os.access(_build(tmp_path), os.X_OK)


@pytest.mark.gpu
def test_c_program_matches_the_oracle(tmp_path):
    exe = _build(tmp_path)
    print("[c program] running", exe, flush=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=100)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().splitlines()[-1] == "ok"
