"""GPU parity for sliding windows narrower than a page or a page pair
(window w: position t sees keys t-w+1..t), against the fp64 oracle.  The
513-key window of the model spans many pages; these widths put the window's
start and end inside one page, one page pair, or one split."""
import numpy as np
import pytest

from flint_cases import TOL, DecodeCase, max_err

pytestmark = pytest.mark.gpu

WINDOWS = [1, 2, 15, 16, 17, 31, 32, 33, 100]
CTXS = [1, 2, 16, 17, 40, 300]


@pytest.mark.parametrize("window", WINDOWS)
def test_decode_small_windows(window):
    case = DecodeCase(40, CTXS, window=window, weights_one=False)
    ref, _, _, _ = case.expected()
    for pps in (0, 1, 3):
        out, _, _, _ = case.run_gpu(pages_per_split=pps)
        err = max_err(out.cpu().numpy(), ref)
        assert err <= TOL, (window, pps, err)


@pytest.mark.parametrize("window", [1, 16, 17, 33])
def test_fused_step_small_windows(window):
    case = DecodeCase(41, CTXS, window=window, weights_one=False)
    ref, _, _, _ = case.expected()
    for pps in (0, 2):
        out, _, _, _ = case.run_gpu_fused(pages_per_split=pps)
        err = max_err(out.cpu().numpy(), ref)
        assert err <= TOL, (window, pps, err)


@pytest.mark.parametrize("window", [1, 2, 16, 17, 31, 33, 100])
def test_prefill_small_windows(window):
    from test_gpu_prefill import PrefillCase
    case = PrefillCase(42, [(300, 300), (500, 77), (1001, 250)], window=window)
    got, _, _, _ = case.run_gpu()
    bad = int((~np.isfinite(got)).sum())
    assert bad == 0, f"{bad} non-finite outputs"
    assert max_err(got, case.expected()) <= TOL


@pytest.mark.parametrize("window", [1, 17, 33])
def test_fp8_decode_small_windows(window):
    case = DecodeCase(43, CTXS, window=window, weights_one=False, fp8=(1.0 / 16, 0.5))
    ref, _, _, _ = case.expected()
    for pps in (0, 1):
        out, _, _, _ = case.run_gpu(pages_per_split=pps)
        err = max_err(out.cpu().numpy(), ref)
        assert err <= TOL, (window, pps, err)
