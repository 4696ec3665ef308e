"""The CPU suites under AddressSanitizer and UndefinedBehaviorSanitizer:
the oracle's pins against liboracle_san.so (gcc, -fsanitize=address,undefined,
gcc's ASan runtime preloaded) and the host-side ABI checks against
libflint_san.so, whose host code only is built with -Xarch_host
-fsanitize=address,undefined (clang's ASan runtime preloaded; the gfx950 code
is built as in the product).  Any report aborts the run (no recovery), so a
green suite means no report.  Each suite runs in a child process."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(so, sources):
    return not os.path.exists(so) or any(os.path.getmtime(so) < os.path.getmtime(f)
                                         for f in sources)


def _run_suite(test_file, preload):
    env = dict(os.environ, FLINT_SANITIZED="1", LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", test_file, "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    return tail


def test_oracle_pins_under_asan_and_ubsan():
    import oracle
    oracle.build(force=False, sanitize=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    assert os.path.isabs(libasan), "gcc's ASan runtime not found"
    print(_run_suite("tests/test_oracle_pins.py", libasan)[-200:])


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not installed")
def test_abi_host_checks_under_asan_and_ubsan():
    from full_gqa_decode_amd import build as flb
    sources = [os.path.join(flb.CSRC, f) for f in os.listdir(flb.CSRC)]
    sources.append(os.path.join(ROOT, "include", "flint.h"))
    if _stale(flb.SO_SANITIZED, sources):
        flb.build(sanitize=True)
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(rt) and os.path.exists(rt), "clang's ASan runtime not found"
    print(_run_suite("tests/test_abi_cpu.py", rt)[-200:])
