"""GPU parity of the fp8 E4M3 KV cache (K and V stored as codes of x / scale,
one scale pair per layer) against the fp64 oracle, through the C ABI: the
append's codes, decode end to end, the fused step, and K2/K3 on their own.

Unwritten cache slots hold the NaN code 0x7F, so a ragged tail or a window
edge that let one reach the accumulator would show up as NaN."""
import math

import numpy as np
import pytest

import oracle
from flint_cases import (TOL, assert_parity, check_err, guard_bar, SENTINEL8, CacheDecodeCase, DecodeCase, down, max_err, up)

pytestmark = pytest.mark.gpu

# K rows are RMS-normalised (|k| up to ~4), so k_scale 1/16 uses the upper
# binades of E4M3; raw V ~ N(0,1) over 0.5 sits around 2
FP8 = (1.0 / 16, 0.5)


def fp8_step(codes):
    """Spacing of the E4M3 grid at each code's magnitude."""
    v = np.abs(oracle.fp8_value(codes))
    return np.exp2(np.floor(np.log2(np.maximum(v, 2.0**-6))) - 3)


def check_fp8_cache(kd, vd, kc, vc):
    # V: the same single rounding of the same fp64 quotient on both sides:
    # byte for byte, every slot nobody wrote included
    assert np.array_equal(down(vd), vc)
    # K: from the two sides' fp64 norm/rotation; equal up to a rounding
    # boundary between them (one grid step, and rarely)
    kg = down(kd)
    untouched = kc == SENTINEL8
    assert np.array_equal(kg[untouched], kc[untouched])
    a, b = kg[~untouched], kc[~untouched]
    diff = np.abs(oracle.fp8_value(a) - oracle.fp8_value(b))
    assert np.all(diff <= np.maximum(fp8_step(a), fp8_step(b)))
    assert np.count_nonzero(diff) <= max(2, a.size // 1_000_000), np.count_nonzero(diff)


CASES = [
    (0, False, [1], 0),
    (0, False, [17], 0),
    (0, False, [4096], 0),
    (0, False, [1, 15, 16, 17, 513, 1000, 2049], 0),
    (0, False, [3000, 16], 1),
    (0, False, [700, 5000], 7),
    (513, True, [1, 512, 513, 514, 2000], 0),
    (513, True, [32768], 0),
    (513, False, [2000, 33], 3),
    # grids of more than 256 workgroups: the fused fp8 kernels at their
    # two-workgroups-per-CU register bound (windowed multi-split; one long
    # pipelined split per request)
    (513, True, [600, 700, 800, 513, 514, 1000, 1200, 2000, 3000, 900], 0),
    (0, False, [700 + 3 * i for i in range(65)], 60),
]


@pytest.mark.parametrize("window,ring,ctxs,pps", CASES)
def test_fp8_append_then_decode_matches_oracle(window, ring, ctxs, pps):
    case = DecodeCase(31, ctxs, window=window, ring=ring, weights_one=False, fp8=FP8)
    ref, q, kc, vc = case.expected()
    out, qd, kd, vd = case.run_gpu(pages_per_split=pps)
    got = out.cpu().numpy()
    err = max_err(got, ref)
    print(f"fp8 window {window} ctxs {ctxs} pps {pps}: max err {err:.3e}", flush=True)
    check_err(err, ref)
    check_fp8_cache(kd, vd, kc, vc)
    assert np.max(np.abs(qd.cpu().numpy()[case.last_row] - q)) < 1e-6


@pytest.mark.parametrize("window,ring,ctxs,pps", CASES)
def test_fp8_fused_step_bitwise_equals_append_then_decode(window, ring, ctxs, pps):
    case = DecodeCase(32, ctxs, window=window, ring=ring, weights_one=False, fp8=FP8)
    out_ref, qd, kd_ref, vd_ref = case.run_gpu(pages_per_split=pps)
    out, qo, kd, vd = case.run_gpu_fused(pages_per_split=pps)
    assert np.array_equal(out.cpu().numpy(), out_ref.cpu().numpy())
    assert np.array_equal(down(kd), down(kd_ref))
    assert np.array_equal(down(vd), down(vd_ref))
    assert np.array_equal(qo.cpu().numpy(), qd.cpu().numpy()[case.last_row])
    ref, _, _, _ = case.expected()
    assert_parity(out.cpu().numpy(), ref)


def test_fp8_saturates_instead_of_nan():
    # raw V far beyond 448 * v_scale: the cache holds +-448 codes, the
    # output stays finite
    case = DecodeCase(33, [40], window=0, fp8=(1.0, 1.0 / 64))
    case.v_in *= 1e4
    ref, _, kc, vc = case.expected()
    out, _, kd, vd = case.run_gpu()
    assert np.isfinite(out.cpu().numpy()).all()
    vg = down(vd)
    assert np.array_equal(vg, vc)
    written = vc != SENTINEL8
    assert np.count_nonzero((vg[written] & 0x7F) == 0x7E) > 0
    # outputs are O(448 / 64); relative bar (the guard scales with |ref|)
    err = max_err(out.cpu().numpy(), ref)
    assert err <= TOL * 8
    assert err <= guard_bar(ref)


@pytest.mark.parametrize("window,ctxs,pps", [(0, [700, 1, 333], 3), (0, [4096], 7),
                                             (0, [100, 2500], 0), (513, [2000, 100], 4)])
def test_fp8_drawn_cache_decode_partials_merge(window, ctxs, pps):
    import torch
    import full_gqa_decode_amd as fl
    case = CacheDecodeCase(34, ctxs, window=window, ring=bool(window), fp8=(2.0, 0.25))
    ref = case.expected()
    got = case.run_gpu(pages_per_split=pps)
    assert_parity(got, ref)
    if pps == 0:
        return
    q, kc, vc, bt, sl = up(case.q), up(case.kc), up(case.vc), up(case.bt), up(case.seq_lens)
    po, pl = fl.flint_attn_decode_partials(case.FL, q, kc, vc, bt, sl, max(ctxs), pps)
    out = fl.flint_attn_merge(case.FL, po, pl, up(case.sinks))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), got)
    # every split's partial against the oracle's over the same key range
    _, S = fl.flint_attn_decode_plan(case.FL, case.B, max(ctxs), pps)
    lse = pl.cpu().numpy().astype(np.float64) * math.log(2.0)
    o = po.cpu().numpy()
    qq = case.q.astype(np.float64)
    for b, c in enumerate(ctxs):
        t = c - 1
        lo = max(0, t - window + 1) if window else 0
        for s in range(S):
            j0 = max(lo, (lo // 16 + s * pps) * 16)
            j1 = min(t, (lo // 16 + (s + 1) * pps) * 16 - 1) + 1
            for h in (0, 13, 31):
                if j0 >= j1:
                    assert np.isneginf(lse[b, s, h])
                    continue
                o_ref, l_ref = oracle.attn_partial(case.L, qq[b, h], h, case.kc, case.vc,
                                                   case.bt, b, j0, j1)
                assert abs(lse[b, s, h] - l_ref) <= 1e-4
                assert_parity(o[b, s, h], o_ref)
