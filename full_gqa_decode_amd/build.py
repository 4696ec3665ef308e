"""Build libflint.so (HIP for gfx950) in-tree with hipcc.

    python -m full_gqa_decode_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libflint.so")
SOURCES = ["api.hip", "append.hip", "decode.hip", "prefill.hip", "moe.hip", "moe_api.hip"]
# measurement kernels for the bench's machine ceilings, kept out of libflint
SO_CEILING = os.path.join(HERE, "libflint_ceiling.so")
SOURCES_CEILING = ["ceiling.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# The host half of the library built with AddressSanitizer and
# UndefinedBehaviorSanitizer (build(sanitize=True)): every flag reaches the
# host compilation only, so the gfx950 code is built exactly as in the
# product.  A process loads it with clang's ASan runtime preloaded.
SO_SANITIZED = os.path.join(HERE, "libflint_san.so")
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                       "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


# The library with per-wave phase stamps in the prefill and slice kernels
# (build(stamps=True), -DFLINT_STAMPS): read by `bench.py --stamps` only.
SO_STAMPS = os.path.join(HERE, "libflint_stamps.so")


def build(verbose: bool = False, sanitize: bool = False, stamps: bool = False) -> str:
    """Compile every HIP source into one shared library (always rebuilds),
    and the ceiling kernels into libflint_ceiling.so; sanitize=True builds
    libflint_san.so with sanitized host code instead, stamps=True the
    instrumented libflint_stamps.so."""
    if sanitize:
        return _hipcc(SO_SANITIZED, SOURCES, HOST_SANITIZE_FLAGS, verbose)
    if stamps:
        return _hipcc(SO_STAMPS, SOURCES, ["-DFLINT_STAMPS"], verbose)
    _hipcc(SO_CEILING, SOURCES_CEILING, [], verbose)
    return _hipcc(SO, SOURCES, [], verbose)


def _hipcc(so: str, sources: list, extra: list, verbose: bool) -> str:
    tmp = so + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-result",
           # packed fp32 VALU ops stay off: ordinary float code only
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-o", tmp]
    cmd += extra
    cmd += [os.path.join(CSRC, s) for s in sources]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, so)
    return so


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv, stamps="--stamps" in sys.argv))
