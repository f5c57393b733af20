"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: its pins,
its mutation tests' clean baseline and the golden record, run in a child
process against liboracle_san.so (gcc, -fsanitize=address,undefined, every
finding fatal)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_oracle_pins_clean_under_asan_and_ubsan():
    import oracle
    san = oracle.build(force=True, sanitize=True)
    libasan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    env = dict(os.environ, MOE_ORACLE_LIB=san, LD_PRELOAD=libasan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_golden.py")],
                       env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
