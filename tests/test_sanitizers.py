"""The host C/C++ code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: the
library's pattern builder, CSR validation and top-k selection (plain g++ build of the host-only
sources, no HIP), and the C oracle (gcc). Each driver checks invariants on seeded inputs and prints
OK; any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_gemm_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, exe, env=None):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    e = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    e.update(env or {})
    out = subprocess.run([exe], capture_output=True, text=True, env=e, timeout=300)
    assert out.returncode == 0 and out.stdout.strip() == "OK", (out.stdout[-2000:], out.stderr[-4000:])


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_pattern_builder_under_sanitizers(tmp_path):
    exe = str(tmp_path / "pattern_check")
    srcs = [os.path.join(ROOT, "tests", "sanitize", "pattern_check.cpp")] + [
        os.path.join(CSRC, f) for f in ("bsr_pattern.cpp", "bsr_select.cpp", "bsr_error.cpp")]
    _run(["g++", "-std=c++17"] + SAN + [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"] + srcs + ["-o", exe], exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    srcs = [os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"), os.path.join(ROOT, "oracle", "oracle.c")]
    _run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off"] + SAN + srcs + ["-lm", "-o", exe], exe,
         env={"OMP_NUM_THREADS": "4"})
