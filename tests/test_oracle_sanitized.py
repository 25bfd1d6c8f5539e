"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
oracle.c and a small C driver that calls every entry point on ragged valid
and invalid inputs are compiled with gcc's sanitizers and run; any
out-of-bounds access, use after free or undefined operation aborts the run."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c")]


def _sanitizers_available(cc):
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        open(src, "w").write("int main(void) { return 0; }\n")
        r = subprocess.run([cc, "-fsanitize=address,undefined", src, "-o", os.path.join(d, "t")],
                           capture_output=True)
        return r.returncode == 0


def test_oracle_is_clean_under_asan_and_ubsan():
    cc = shutil.which("gcc")
    if cc is None or not _sanitizers_available(cc):
        pytest.skip("gcc with AddressSanitizer / UBSan is not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitized")
        build = subprocess.run(
            [cc, "-std=c11", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *SOURCES, "-o", exe,
             "-lm"], capture_output=True, text=True)
        assert build.returncode == 0, build.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert run.returncode == 0, run.stderr[-4000:]
        assert "AddressSanitizer" not in run.stderr and "runtime error" not in run.stderr, \
            run.stderr[-4000:]
