"""The library from a plain C program on the GPU.  tests/c_client_decode_step.c
(C11; the HIP runtime API for device memory and copies; no Python in its
process) runs one fused decode step through the C ABI.  Its output and the
cache rows it wrote are checked against the oracle.  The inputs -- the caches
already holding every earlier token included -- are prepared on the host by the
oracle, so the test's own process makes no GPU call for this check."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from flint_cases import DecodeCase, assert_parity, empty_caches

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_client(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    libdir = os.path.join(ROOT, "full_gqa_decode_amd")
    exe = str(tmp_path / "c_client_decode_step")
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(rocm, "include"),
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_client_decode_step.c"), "-o", exe,
                    "-L", libdir, "-lflint", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"],
                   check=True)
    return exe


@pytest.mark.parametrize("window", [0, 513])
def test_c_client_runs_the_fused_step(tmp_path, window):
    case = DecodeCase(52, [700, 33, 1500], window=window, weights_one=False)
    # the caches with every token but each request's new one, written by the oracle
    kc, vc = empty_caches(case.L, case.num_blocks)
    keep = np.ones(case.T, bool)
    keep[case.last_row] = False
    pre = np.nonzero(keep)[0]
    oracle.append(case.L, case.q_in[:1], case.k_in[pre], case.v_in[pre], case.qw, case.kw,
                  case.pos[pre], case.slots[pre], kc, vc, want_q=False)
    r = case.last_row
    inputs = dict(q_in=case.q_in[r], k_in=case.k_in[r], v_in=case.v_in[r], q_w=case.qw,
                  k_w=case.kw, slots=case.slots[r], k_cache=kc, v_cache=vc,
                  block_tables=case.bt, seq_lens=case.seq_lens, sinks=case.sinks)
    for name, arr in inputs.items():
        want = np.uint16 if name.endswith("cache") else (
            np.int32 if name in ("slots", "block_tables", "seq_lens") else np.float32)
        assert arr.dtype == want, name
        np.ascontiguousarray(arr).tofile(tmp_path / f"{name}.bin")
    exe = _build_client(tmp_path)
    eps = f"{np.float32(1e-6):.9g}"
    scale = f"{np.float32(1.0 / np.sqrt(128)):.9g}"
    args = [exe, str(tmp_path), str(case.B), str(case.num_blocks), str(case.bt_stride),
            str(max(case.ctxs)), str(window), str(case.FL.use_rope), eps, scale]
    print("C client:", " ".join(args[1:]), flush=True)
    res = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "status 0" in res.stdout
    out = np.fromfile(tmp_path / "out.bin", np.float32).reshape(case.B, case.hq, 128)
    ref, _, kc_ref, vc_ref = case.expected()
    assert_parity(out, ref)
    # the new tokens' cache rows: V bit-exact, K within one bf16 ulp (ties of
    # the fp64 value); every other slot untouched
    kc_out = np.fromfile(tmp_path / "k_cache_out.bin", np.uint16).reshape(kc.shape)
    vc_out = np.fromfile(tmp_path / "v_cache_out.bin", np.uint16).reshape(vc.shape)
    assert np.array_equal(vc_out, vc_ref)
    assert np.abs(kc_out.astype(np.int32) - kc_ref.astype(np.int32)).max() <= 1
