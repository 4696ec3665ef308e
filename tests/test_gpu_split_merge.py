"""K2 and K3 on their own, through the C ABI: flint_attn_decode_partials
against the oracle's partial over each split's key range (O6), and
flint_attn_merge fed the oracle's partials against the oracle's merge; the
two together equal flint_attn_decode_ex bit for bit."""
import math

import numpy as np
import pytest

import oracle
from flint_cases import TOL, CacheDecodeCase, assert_parity, dev, up

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-4   # natural-log units; scores are O(1) here, fp32 rounding ~1e-6


def split_ranges(case, window, pps, S):
    """Key range [j0, j1) of every (request, split), as the header defines it."""
    out = []
    for b, c in enumerate(case.ctxs):
        t = c - 1
        lo = max(0, t - window + 1) if window else 0
        rows = []
        for s in range(S):
            first = (lo // 16 + s * pps) * 16
            last = (lo // 16 + (s + 1) * pps) * 16 - 1
            rows.append((max(lo, first), min(t, last) + 1))
        out.append(rows)
    return out


def oracle_partials(case, window, pps, S):
    q = case.q.astype(np.float64)
    o = np.zeros((case.B, S, 32, 128))
    lse = np.full((case.B, S, 32), -np.inf)
    for b, rows in enumerate(split_ranges(case, window, pps, S)):
        for s, (j0, j1) in enumerate(rows):
            if j0 >= j1:
                continue
            for h in range(32):
                o[b, s, h], lse[b, s, h] = oracle.attn_partial(case.L, q[b, h], h, case.kc,
                                                               case.vc, case.bt, b, j0, j1)
    return o, lse


CASES = [
    (0, [700, 1, 333], 3),          # full layer; request 1 fills one split only
    (0, [4096], 7),
    (513, [2000, 100], 4),          # sliding: 33-page window in 9 splits
]


@pytest.mark.parametrize("window,ctxs,pps", CASES)
def test_partials_match_oracle_ranges(window, ctxs, pps):
    import torch
    import full_gqa_decode_amd as fl
    case = CacheDecodeCase(21, ctxs, window=window, ring=bool(window))
    _, S = fl.flint_attn_decode_plan(case.FL, case.B, max(ctxs), pps)
    po, pl = fl.flint_attn_decode_partials(case.FL, up(case.q), up(case.kc), up(case.vc),
                                           up(case.bt), up(case.seq_lens), max(ctxs), pps)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_partials(case, window, pps, S)
    lse_gpu = pl.cpu().numpy().astype(np.float64) * math.log(2.0)
    empty = np.isinf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty)
    assert np.abs(lse_gpu[~empty] - lse_ref[~empty]).max() <= LSE_TOL
    o_gpu = po.cpu().numpy().astype(np.float64)
    assert_parity(o_gpu[~empty], o_ref[~empty])


@pytest.mark.parametrize("window,ctxs,pps", CASES)
def test_merge_of_oracle_partials_matches_oracle(window, ctxs, pps):
    import torch
    import full_gqa_decode_amd as fl
    case = CacheDecodeCase(22, ctxs, window=window, ring=bool(window))
    _, S = fl.flint_attn_decode_plan(case.FL, case.B, max(ctxs), pps)
    o_ref, lse_ref = oracle_partials(case, window, pps, S)
    po = o_ref.astype(np.float32)
    po[np.isinf(lse_ref)] = np.nan            # an empty split's output must not be read
    pl = (lse_ref / math.log(2.0)).astype(np.float32)
    out = fl.flint_attn_merge(case.FL, up(po), up(pl), up(case.sinks))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = np.empty_like(got)
    for b in range(case.B):
        for h in range(32):
            live = ~np.isinf(lse_ref[b, :, h])
            want[b, h] = oracle.merge(o_ref[b, live, h], lse_ref[b, live, h],
                                      float(case.sinks[h]))
    assert_parity(got, want)
    # and the whole chain against the direct definition
    assert_parity(got, case.expected())


@pytest.mark.parametrize("ctx,pps", [(300, 5), (300, 1), (2000, 1)])
def test_nan_partial_makes_its_output_nan(ctx, pps):
    # 4, 19 and 125 splits: the three merge kernels (up to 8, up to 64, more)
    import torch
    import full_gqa_decode_amd as fl
    case = CacheDecodeCase(23, [ctx], window=0)
    po, pl = fl.flint_attn_decode_partials(case.FL, up(case.q), up(case.kc), up(case.vc),
                                           up(case.bt), up(case.seq_lens), ctx, pps)
    pl[0, 1, 7] = float("nan")
    out = fl.flint_attn_merge(case.FL, po, pl, up(case.sinks))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isnan(got[0, 7]).all()
    assert np.isfinite(np.delete(got[0], 7, axis=0)).all()


@pytest.mark.parametrize("window,ctxs,pps", CASES)
def test_partials_then_merge_equal_decode_bitwise(window, ctxs, pps):
    import torch
    import full_gqa_decode_amd as fl
    case = CacheDecodeCase(24, ctxs, window=window, ring=bool(window))
    q, kc, vc, bt, sl = up(case.q), up(case.kc), up(case.vc), up(case.bt), up(case.seq_lens)
    po, pl = fl.flint_attn_decode_partials(case.FL, q, kc, vc, bt, sl, max(ctxs), pps)
    out = fl.flint_attn_merge(case.FL, po, pl, up(case.sinks))
    ref = torch.empty_like(out)
    fl.flint_attn_decode(case.FL, q, kc, vc, bt, sl, max(ctxs), up(case.sinks), ref,
                         pages_per_split=pps)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("ctx,pps", [(300, 1), (4096, 4)])
def test_merge_of_unaligned_buffers(ctx, pps):
    # part_o and out only 4-byte aligned: the launcher falls back from the
    # 16-byte-load kernel; same result within rounding, and against the oracle
    import torch
    import full_gqa_decode_amd as fl
    case = CacheDecodeCase(25, [ctx], window=0)
    po, pl = fl.flint_attn_decode_partials(case.FL, up(case.q), up(case.kc), up(case.vc),
                                           up(case.bt), up(case.seq_lens), ctx, pps)
    ref = fl.flint_attn_merge(case.FL, po, pl, up(case.sinks))
    big = torch.empty(po.numel() + 1, dtype=torch.float32, device=po.device)
    po1 = big[1:].view(po.shape)
    po1.copy_(po)
    ob = torch.empty(ref.numel() + 1, dtype=torch.float32, device=po.device)
    out1 = ob[1:].view(ref.shape)
    fl.flint_attn_merge(case.FL, po1, pl, up(case.sinks), out=out1)
    torch.cuda.synchronize()
    assert po1.data_ptr() % 16 != 0 and out1.data_ptr() % 16 != 0
    got, want = out1.cpu().numpy(), ref.cpu().numpy()
    assert np.abs(got - want).max() <= 1e-5
    assert_parity(got, case.expected())
