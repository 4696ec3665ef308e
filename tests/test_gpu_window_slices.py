"""The slice kernel: a short key range (the 513-key window, or any range of at
most 40 pages) at small batch runs as one launch of 8 workgroups per (request,
KV head), each owning 16 of the 128 output dims, with no merge.  Parity
against the oracle at batch sizes on both sides of the one-round limit
(requests x KV heads x 8 <= 256 workgroups), against the key-split plan with
its merge, at the 40-page limit of full layers, and through the fused step."""
import numpy as np
import pytest

from flint_cases import DecodeCase, assert_parity, down16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B", [1, 2, 7, 8, 9])
def test_window_batches_around_the_slice_grid_limit(B):
    import full_gqa_decode_amd as fl
    ctxs = [513 + 97 * b for b in range(B)]
    ctxs[0] = 5000
    case = DecodeCase(70 + B, ctxs, window=513, ring=True, weights_one=False)
    _, splits = fl.flint_attn_decode_plan(case.FL, B, max(ctxs))
    assert (splits == 1) == (B * 4 * 8 <= 256)
    ref, _, _, _ = case.expected()
    out, qd, kd, vd = case.run_gpu()
    assert_parity(out.cpu().numpy(), ref)
    outf, qo, kdf, vdf = case.run_gpu_fused()
    assert np.array_equal(outf.cpu().numpy(), out.cpu().numpy())
    assert np.array_equal(down16(kdf), down16(kd)) and np.array_equal(down16(vdf), down16(vd))
    assert np.array_equal(qo.cpu().numpy(), qd.cpu().numpy()[case.last_row])


def test_slice_kernel_agrees_with_the_key_split_plan():
    # 5-page splits: the 33-page window in 7 splits and a merge launch
    import full_gqa_decode_amd as fl
    case = DecodeCase(80, [100_000 - 3, 7000], window=513, ring=True, weights_one=False)
    assert fl.flint_attn_decode_plan(case.FL, 2, 100_000 - 3)[1] == 1
    assert fl.flint_attn_decode_plan(case.FL, 2, 100_000 - 3, 5)[1] == 7
    ref, _, _, _ = case.expected()
    a, _, _, _ = case.run_gpu()
    b, _, _, _ = case.run_gpu(pages_per_split=5)
    assert_parity(a.cpu().numpy(), ref)
    assert_parity(b.cpu().numpy(), ref)
    assert np.abs(a.cpu().numpy() - b.cpu().numpy()).max() <= 1e-5


@pytest.mark.parametrize("ctxs", [[640, 1, 639, 17], [641, 300]])
def test_full_layer_at_the_short_range_limit(ctxs):
    # 640 keys = 40 pages: the slice kernel; 641 keys: the split plan
    import full_gqa_decode_amd as fl
    case = DecodeCase(81, ctxs, window=0, weights_one=False)
    short = max(ctxs) <= 640
    assert (fl.flint_attn_decode_plan(case.FL, len(ctxs), max(ctxs))[1] == 1) == short
    ref, _, _, _ = case.expected()
    out, _, _, _ = case.run_gpu()
    assert_parity(out.cpu().numpy(), ref)
    outf, _, _, _ = case.run_gpu_fused()
    assert np.array_equal(outf.cpu().numpy(), out.cpu().numpy())
