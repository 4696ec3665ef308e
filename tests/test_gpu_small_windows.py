"""GPU parity against the fp64 oracle for shapes the model's own layers do
not reach: sliding windows narrower than a page or a page pair (window w:
position t sees keys t-w+1..t, so the window's start and end fall inside one
page, one page pair or one split), and KV head counts other than four (the
C ABI admits 1..8, each with 8 query heads)."""
import numpy as np
import pytest

from flint_cases import PREFILL_GUARD, TOL, assert_parity, check_err, DecodeCase, max_err

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
        check_err(err, ref, (window, pps))


@pytest.mark.parametrize("window", [1, 16, 17, 33])
def test_fused_step_small_windows(window):
    case = DecodeCase(41, CTXS, window=window, weights_one=False)
    ref, _, _, _ = case.expected()
    for pps in (0, 2):
        out, _, _, _ = case.run_gpu_fused(pages_per_split=pps)
        err = max_err(out.cpu().numpy(), ref)
        check_err(err, ref, (window, pps))


@pytest.mark.parametrize("window", [1, 2, 16, 17, 31, 33, 100])
def test_prefill_small_windows(window):
    from test_gpu_prefill import PrefillCase
    case = PrefillCase(42, [(300, 300), (500, 77), (1001, 250)], window=window)
    got, _, _, _ = case.run_gpu()
    bad = int((~np.isfinite(got)).sum())
    assert bad == 0, f"{bad} non-finite outputs"
    assert_parity(got, case.expected(), guard=PREFILL_GUARD)


@pytest.mark.parametrize("window", [1, 17, 33])
def test_fp8_decode_small_windows(window):
    case = DecodeCase(43, CTXS, window=window, weights_one=False, fp8=(1.0 / 16, 0.5))
    ref, _, _, _ = case.expected()
    for pps in (0, 1):
        out, _, _, _ = case.run_gpu(pages_per_split=pps)
        err = max_err(out.cpu().numpy(), ref)
        check_err(err, ref, (window, pps))


# ---- KV head counts other than the model's 4 (the ABI admits 1..8) --------

@pytest.mark.parametrize("hkv", [1, 2, 8])
def test_decode_and_fused_step_other_kv_head_counts(hkv):
    for window in (0, 33):
        case = DecodeCase(44, [1, 17, 300, 2000], window=window, weights_one=False, hkv=hkv)
        ref, _, _, _ = case.expected()
        for pps in (0, 1, 4):
            out, _, _, _ = case.run_gpu(pages_per_split=pps)
            assert_parity(out.cpu().numpy(), ref, (hkv, window, pps))
        out, _, _, _ = case.run_gpu_fused()
        assert_parity(out.cpu().numpy(), ref, (hkv, window, "fused"))


@pytest.mark.parametrize("hkv", [1, 8])
def test_prefill_other_kv_head_counts(hkv):
    from test_gpu_prefill import PrefillCase
    for window in (0, 33):
        case = PrefillCase(45, [(300, 300), (700, 90)], window=window, hkv=hkv)
        got, _, _, _ = case.run_gpu()
        assert_parity(got, case.expected(), (hkv, window), guard=PREFILL_GUARD)


@pytest.mark.parametrize("hkv,reqs", [
    (8, [(800, 800), (300, 60)]),                       # 25 row blocks x 8 x 2 = 400 items
    (1, [(700 - 37 * i, 700 - 53 * i) for i in range(12)]),  # 22 x 1 x 12 = 264 items
])
def test_prefill_other_kv_head_counts_more_items_than_workgroups(hkv, reqs):
    # more (row block, KV head, request) items than the 256 workgroups of the
    # persistent prefill grid, so workgroups run several items each
    from test_gpu_prefill import PrefillCase
    for window in (0, 513):
        case = PrefillCase(47, reqs, window=window, hkv=hkv)
        got, _, _, _ = case.run_gpu()
        assert_parity(got, case.expected(), (hkv, window), guard=PREFILL_GUARD)


@pytest.mark.parametrize("hkv", [1, 8])
def test_fp8_decode_other_kv_head_counts(hkv):
    case = DecodeCase(46, [1, 40, 900], window=0, weights_one=False, fp8=(1.0 / 16, 0.5),
                      hkv=hkv)
    ref, _, _, _ = case.expected()
    out, _, _, _ = case.run_gpu()
    assert_parity(out.cpu().numpy(), ref)


# ---- layer parameters other than the model's --------------------------------

@pytest.mark.parametrize("window,rope,theta,scale,eps", [
    (0, 1, 1e6, 0.05, 1e-5),         # full attention with RoPE, another base
    (33, 1, 500000.0, 0.2, 1e-6),    # a short window, a large scale
    (513, 0, 10000.0, 0.0625, 1e-6),  # a sliding window without RoPE
])
def test_other_rope_bases_scales_and_eps(window, rope, theta, scale, eps):
    kw = dict(rope=rope, theta=theta, scale=scale, eps=eps)
    case = DecodeCase(47, [1, 17, 700, 3000], window=window, weights_one=False, **kw)
    ref, _, _, _ = case.expected()
    out, _, _, _ = case.run_gpu()
    assert_parity(out.cpu().numpy(), ref)
    out, _, _, _ = case.run_gpu_fused()
    assert_parity(out.cpu().numpy(), ref)
    from test_gpu_prefill import PrefillCase
    pc = PrefillCase(48, [(500, 500), (900, 130)], window=window, **kw)
    got, _, _, _ = pc.run_gpu()
    assert_parity(got, pc.expected(), guard=PREFILL_GUARD)
