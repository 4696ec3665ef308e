"""GPU parity of the decode path (K1 append -> K2 split-K -> K3 merge)
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
from flint_cases import (TOL, assert_parity, check_err, CacheDecodeCase, DecodeCase, bf16_ulp_diff, down16, max_err)

pytestmark = pytest.mark.gpu


def _check_cache(case, kd, vd, kc, vc):
    # V: byte for byte, including every slot nobody wrote
    assert np.array_equal(down16(vd), vc)
    # K: untouched slots identical, written ones equal up to fp64 ties
    kg = down16(kd)
    untouched = kc == 0x7FC1
    assert np.array_equal(kg[untouched], kc[untouched])
    check_k_values(kg[~untouched], kc[~untouched])


def check_k_values(kg, ko):
    """GPU K (fp64 norm/rotation, one rounding) vs oracle K (fp64, one
    rounding): identical except where the two fp64 evaluation orders straddle
    a rounding tie (~1e-15 relative), which may move a value by one ulp."""
    ulp = bf16_ulp_diff(kg, ko)
    assert int(ulp.max()) <= 1, (kg[ulp > 1][:8], ko[ulp > 1][:8])
    assert int(np.count_nonzero(ulp)) <= max(2, kg.size // 1_000_000), int(np.count_nonzero(ulp))


@pytest.mark.parametrize("ctx", [1, 15, 16, 17, 300, 4096])
def test_full_layer_end_to_end(ctx):
    case = DecodeCase(0, [ctx], window=0)
    ref, q, kc, vc = case.expected()
    out, qd, kd, vd = case.run_gpu()
    assert_parity(out.cpu().numpy(), ref)
    _check_cache(case, kd, vd, kc, vc)
    qg = qd.cpu().numpy()[case.last_row]
    assert np.max(np.abs(qg - q)) < 1e-6


@pytest.mark.parametrize("ctx", [1, 512, 513, 514, 2000, 32768])
def test_sliding_layer_end_to_end_ring(ctx):
    case = DecodeCase(1, [ctx], window=513, ring=True)
    ref, q, kc, vc = case.expected()
    out, qd, kd, vd = case.run_gpu()
    assert_parity(out.cpu().numpy(), ref)
    _check_cache(case, kd, vd, kc, vc)


def test_ragged_batch_end_to_end_nonunit_weights():
    ctxs = [1, 15, 16, 17, 513, 514, 1000, 2049]
    for window, ring in ((0, False), (513, True)):
        case = DecodeCase(2, ctxs, window=window, ring=ring, weights_one=False)
        ref, q, kc, vc = case.expected()
        out, qd, kd, vd = case.run_gpu()
        assert_parity(out.cpu().numpy(), ref)
        _check_cache(case, kd, vd, kc, vc)


@pytest.mark.parametrize("pps", [0, 1, 2, 7, 16, 64, 1000])
def test_split_counts_agree(pps):
    case = CacheDecodeCase(3, [4096, 1, 700, 33], window=0)
    ref = case.expected()
    got = case.run_gpu(pages_per_split=pps)
    assert_parity(got, ref)


def test_full_layer_bs1_ctx4096():
    # one full NoPE layer, one decode step, batch 1, context 4096, seed 0
    case = DecodeCase(0, [4096], window=0)
    ref, _, _, _ = case.expected()
    out, _, _, _ = case.run_gpu()
    assert_parity(out.cpu().numpy(), ref)


def test_sliding_layer_bs1_ctx32768():
    # one sliding RoPE layer, context 32768, window 513, full page table
    case = DecodeCase(0, [32768], window=513, ring=False)
    ref, _, _, _ = case.expected()
    out, _, _, _ = case.run_gpu()
    assert_parity(out.cpu().numpy(), ref)


def test_sink_minus_inf_and_large_scores():
    case = CacheDecodeCase(4, [3000, 5], window=0, q_scale=4.0)
    ninf = np.full(32, -np.inf, np.float32)
    import oracle
    ref = oracle.attn_decode(case.L, case.q.astype(np.float64), case.kc, case.vc, case.bt,
                             case.seq_lens, ninf)
    got = case.run_gpu(sinks=ninf)
    assert_parity(got, ref)


def test_invalid_requests_give_nan_not_faults():
    case = CacheDecodeCase(5, [200, 300, 400], window=0)
    ref = case.expected()
    bt = case.bt.copy()
    bt[1, 3] = case.num_blocks + 5      # page id out of range
    sl = case.seq_lens.copy()
    sl[2] = 0                             # empty request
    for pps in (0, 2):
        got = case.run_gpu(pages_per_split=pps, seq_lens=sl, bt=bt)
        assert_parity(got[0], ref[0])
        assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))


def test_deterministic():
    case = CacheDecodeCase(6, [10000], window=0)
    a = case.run_gpu()
    b = case.run_gpu()
    assert np.array_equal(a, b)


def test_ragged_64_requests_scaled_lengths():
    # 64 requests, lengths uniform in [1024, 8192] (config 3's mix, scaled down),
    # one full and one sliding layer, random physical page order
    import synth
    lens = synth.uniform_ints(0, (3, 0, synth.LENS), 64, 1024, 8192)
    for window in (0, 513):
        case = CacheDecodeCase(7, lens, window=window)
        assert_parity(case.run_gpu(), case.expected())


@pytest.mark.parametrize("window,ring,ctxs,pps", [
    (0, False, [4096], 0),
    (0, False, [1, 17, 1000, 5000], 0),
    (0, False, [3000, 16], 2),
    (0, False, [700], 1000),
    (513, True, [32768], 0),
    (513, True, [1, 513, 514, 2000], 0),
    (513, False, [2000, 33], 3),
])
def test_fused_step_bitwise_equals_append_then_decode(window, ring, ctxs, pps):
    case = DecodeCase(9, ctxs, window=window, ring=ring, weights_one=False)
    out_ref, qd, kd_ref, vd_ref = case.run_gpu(pages_per_split=pps)
    out, qo, kd, vd = case.run_gpu_fused(pages_per_split=pps)
    assert np.array_equal(out.cpu().numpy(), out_ref.cpu().numpy())
    assert np.array_equal(down16(kd), down16(kd_ref))
    assert np.array_equal(down16(vd), down16(vd_ref))
    assert np.array_equal(qo.cpu().numpy(), qd.cpu().numpy()[case.last_row])
    ref, _, _, _ = case.expected()
    assert_parity(out.cpu().numpy(), ref)


def test_fused_step_rejects_a_slot_the_page_table_disagrees_with():
    case = DecodeCase(10, [300, 400, 500], window=0)
    ref, _, _, _ = case.expected()
    out, _, kd, vd = case.run_gpu_fused(slot_delta=[0, 1, 0])
    got = out.cpu().numpy()
    assert np.all(np.isnan(got[1]))
    assert_parity(got[[0, 2]], ref[[0, 2]])
    # nothing was written for request 1: its new token's row is still the sentinel
    s = int(case.slots[case.last_row[1]])
    kg = down16(kd)
    for g in range(4):
        assert np.all(oracle.k_row(case.L, kg, s // 16, g, s % 16) == 0x7FC1)


@pytest.mark.parametrize("window", [0, 513])
def test_every_request_shorter_than_the_host_bound(window):
    # the kernels start loading for a request of length max_seq_len before
    # seq_lens arrive; here every guess is wrong and must be redone
    case = CacheDecodeCase(11, [3000, 17, 640, 1], window=window)
    ref = case.expected()
    for pps in (0, 1, 3):
        got = case.run_gpu(pages_per_split=pps, max_seq_len=case.bt_stride * 16)
        assert_parity(got, ref)
