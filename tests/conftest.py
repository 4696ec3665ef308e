import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# FLINT_SANITIZED=1: the CPU tests run against the sanitizer builds of both
# libraries (oracle.build(sanitize=True), full_gqa_decode_amd.build
# --sanitize), with the matching ASan runtime preloaded by the caller.
if os.environ.get("FLINT_SANITIZED") == "1":
    import full_gqa_decode_amd
    import oracle
    from full_gqa_decode_amd import build as _fl_build

    full_gqa_decode_amd.LIB_PATH = _fl_build.SO_SANITIZED
    oracle.SO = oracle.SO_SANITIZED
