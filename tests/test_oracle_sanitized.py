"""The oracle's pins, run once more against a build of the oracle instrumented with
gcc's AddressSanitizer and UndefinedBehaviorSanitizer (host code only; the oracle is
plain C).  An out-of-bounds access, use of freed memory, signed overflow, invalid
shift or misaligned access anywhere the pins reach aborts the child run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    import oracle.build as ob
    lib = ob.build(force=True, out=str(tmp_path / "liboracle_san.so"),
                   extra_flags=["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                                "-fno-omit-frame-pointer", "-g"])
    env = dict(os.environ, BITOPT_ORACLE_LIB=lib, LD_PRELOAD=f"{asan} {ubsan}", OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_codebook.py", "test_oracle_codec.py", "test_oracle_optim.py", "test_search_tables.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
