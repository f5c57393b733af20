"""The C ABI's host side (argument validation, launch planning, status codes)
under AddressSanitizer and UndefinedBehaviorSanitizer: the library's host
code built with both (libmoe_decode_hostsan.so, device code as usual) and the
ABI tests run against it in a child process, every finding fatal.  No kernel
is launched: every call in those tests is rejected on the host."""
import glob
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_clean_under_host_asan_and_ubsan():
    spec = importlib.util.spec_from_file_location("_moe_build", os.path.join(ROOT, "quantized_moe_decode_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    lib = b.build(sanitize=True)
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    assert rts, "clang's ASan runtime not found"
    env = dict(os.environ, MOE_DECODE_LIB=lib, LD_PRELOAD=rts[-1],
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
