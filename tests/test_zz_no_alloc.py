"""flint_attn_decode_step_noalloc: the fused decode step with its split
partials in the library's static device scratch.  Its outputs must equal
flint_attn_decode_step's (same kernels, a caller workspace) bit for bit, and
the oracle's within the parity bar, on two calls in a row -- the second with
a smaller batch, so that stale partials of the first call in the shared
scratch cannot leak into the second."""
import numpy as np
import pytest

from flint_cases import DecodeCase, assert_parity, down

pytestmark = pytest.mark.gpu


def _both(case, pps):
    ref_out, ref_q, ref_k, ref_v = case.run_gpu_fused(pages_per_split=pps)
    out, qo, kd, vd = case.run_gpu_fused(pages_per_split=pps, noalloc=True)
    assert np.array_equal(out.cpu().numpy(), ref_out.cpu().numpy())
    assert np.array_equal(qo.cpu().numpy(), ref_q.cpu().numpy())
    assert np.array_equal(down(kd), down(ref_k)) and np.array_equal(down(vd), down(ref_v))
    ref, _, _, _ = case.expected()
    return assert_parity(out.cpu().numpy(), ref)


def test_noalloc_step_matches_workspace_step_twice_second_smaller():
    import full_gqa_decode_amd as fl
    big = DecodeCase(90, [6000, 1200, 37, 4100], window=0, weights_one=False)
    _, splits = fl.flint_attn_decode_plan(big.FL, big.B, max(big.ctxs))
    assert splits > 1   # the partials really go through the scratch
    e1 = _both(big, 0)
    small = DecodeCase(91, [700], window=513, ring=True, weights_one=False)
    assert fl.flint_attn_decode_plan(small.FL, 1, 700, 2)[1] > 1
    e2 = _both(small, 2)
    print(f"noalloc step: max err {e1:.2e} (4 requests), {e2:.2e} (1 request)", flush=True)


def test_noalloc_step_refuses_a_batch_beyond_its_scratch():
    import torch
    import full_gqa_decode_amd as fl
    L = fl.full_layer()
    B, ctx = 64, 131072
    need = fl.flint_attn_decode_workspace_size(L, B, ctx)
    assert need > fl.NOALLOC_SCRATCH_BYTES
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt, device="cuda")
    with pytest.raises(fl.FlintError) as e:
        fl.flint_attn_decode_step_noalloc(L, z(B, 32, 128), z(B, 4, 128), z(B, 4, 128), z(128),
                                          z(128), z(B, dt=torch.int32),
                                          z(4, 4, 16, 128, dt=torch.int16),
                                          z(4, 4, 128, 16, dt=torch.int16),
                                          z(B, ctx // 16, dt=torch.int32),
                                          z(B, dt=torch.int32), ctx, z(32), z(B, 32, 128))
    assert e.value.status == 3
