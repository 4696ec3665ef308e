"""GPU parity of the split kernel's page-ring variants against the fp64
oracle, through the C ABI.  A launch of at most one workgroup per CU whose
waves walk at least 4 pages each keeps two pages of loads in flight per wave
(the ring); other launches keep one.  These cases put the ring through its
main loop and its peeled tail -- pages per wave of 4 to 16, odd and even
counts, the last split short -- for full and windowed layers, one and
several splits, bf16 and fp8 caches, the fused step and append + decode."""
import numpy as np
import pytest

from flint_cases import DecodeCase, assert_parity, down

pytestmark = pytest.mark.gpu

FP8 = (1.0 / 16, 0.5)

# (window, ring, ctxs, pages_per_split): every grid below is one round
CASES = [
    (0, False, [3000], 47),          # 188 pages: 4 splits of 47 (6 pages per wave, last split 47)
    (0, False, [3000], 33),          # 6 splits, the last of 23 pages
    (0, False, [2000], 125),         # one split of 125 pages: the sink folded in the split kernel
    (0, False, [4100, 2900, 33], 64),  # three requests, one of them shorter than a split
    (0, False, [2049], 128),         # one page past a whole split count
    (513, True, [20000], 32),        # the window: 2 splits of 32 / 1 page
    (513, False, [700, 514], 32),    # window edges inside the ring pages (2 splits each)
]


@pytest.mark.parametrize("fp8", [None, FP8], ids=["bf16", "fp8"])
@pytest.mark.parametrize("window,ring,ctxs,pps", CASES)
def test_ring_paths_match_oracle(window, ring, ctxs, pps, fp8):
    case = DecodeCase(71, ctxs, window=window, ring=ring, weights_one=False, fp8=fp8)
    ref, q, kc, vc = case.expected()
    out, qd, kd, vd = case.run_gpu(pages_per_split=pps)
    assert_parity(out.cpu().numpy(), ref)
    out_f, qo, kf, vf = case.run_gpu_fused(pages_per_split=pps)
    # the fused step equals append followed by decode, bit for bit
    assert np.array_equal(out_f.cpu().numpy(), out.cpu().numpy())
    assert np.array_equal(down(kf), down(kd))
    assert np.array_equal(down(vf), down(vd))
