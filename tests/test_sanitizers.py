"""The host C code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (oracle/oracle.c), the seeded generator (synth/synth.c) and the
host side of libcgd (its C-ABI argument checks and sizing; the device code is
built as usual) are rebuilt with both sanitizers, every report fatal, and the
CPU suite runs against those builds in a child process with the shared ASan
runtime preloaded. The child must pass and print no sanitizer report. CPU
only: the child runs no GPU code."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = [
    pytest.mark.slow,
    pytest.mark.skipif(os.environ.get("CGD_SANITIZED") == "1", reason="this is the sanitized child run"),
]


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    p = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _build_c(src, out, extra=()):
    subprocess.run([CLANG, "-std=c11", "-fPIC", "-shared", "-shared-libasan", "-ffp-contract=off", *SAN, *extra,
                    "-o", out, src, "-lm"], check=True, capture_output=True, text=True)


def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this toolchain")
    from combine_get_dispatch_06_amd import build as hip_build

    oracle_so = str(tmp_path / "liboracle_san.so")
    synth_so = str(tmp_path / "libsynth_san.so")
    cgd_so = str(tmp_path / "libcgd_san.so")
    _build_c(os.path.join(ROOT, "oracle", "oracle.c"), oracle_so)
    _build_c(os.path.join(ROOT, "synth", "synth.c"), synth_so)  # without OpenMP: one thread, same values
    host_san = []
    for flag in SAN[:3]:  # host compilation only: each sanitizer flag right after -Xarch_host
        host_san += ["-Xarch_host", flag]
    hip_build.build(out=cgd_so, extra=host_san)

    env = dict(os.environ, CGD_LIBRARY=cgd_so, CGD_ORACLE_LIBRARY=oracle_so, CGD_SYNTH_LIBRARY=synth_so,
               CGD_SANITIZED="1", LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child really loads the sanitized builds
    probe = ("import oracle, synth, combine_get_dispatch_06_amd as c; oracle._load(); synth._load(); c.load(); "
             "print(open('/proc/self/maps').read())")
    maps = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True,
                          timeout=300)
    assert maps.returncode == 0, maps.stderr[-3000:]
    for so in (oracle_so, synth_so, cgd_so, rt):
        assert so in maps.stdout, so

    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "not gpu and not slow", "-x", "-q",
                        "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True, timeout=1200)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in r.stdout + r.stderr, report
    assert " passed" in r.stdout, report
