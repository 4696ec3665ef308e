"""Parity at the full workload sizes, in the launch configuration the bench
times: one flint_attn_decode_step call per layer (norm/RoPE/append of the new
token fused into split-K decode, then the merge) with the default plan.

Workloads: batch 1 at a 100,000-token context on a full layer (6,250 shuffled
pages) and on a sliding layer (33-page ring); batch 1 at the model's maximum
context of 262,144 tokens ("Recursive Flint" model JSON, "maxContext") on a
full layer (16,384 pages: the plan then takes 128 splits, two rounds of
workgroups and the wide merge) and on a sliding layer whose RoPE angle is
taken at position 262,143; and 64 requests with context lengths uniform in
[1024, 131072] on a full layer (about 7.9 GB of KV, every request's output
and cache write checked) and on a sliding layer (every request checked).
Over an fp8 cache: the 100,000-token and the 262,144-token full layers, and
the 64 requests on a full and on a sliding layer.

The resident cache pages are N(0,1) bf16 drawn on the GPU by a seeded torch
generator and copied to the host for the oracle; the new tokens' q/k/v come
from synth on the host.  Nothing computed by the GPU feeds the oracle."""
import numpy as np
import pytest

import oracle
import synth
from flint_cases import TOL, check_err, dev, down, layers, up

pytestmark = pytest.mark.gpu

PAGE = 16


class BigStep:
    def __init__(self, tag, ctxs, window, full_table, fp8=None):
        import torch
        self.ctxs = np.asarray(ctxs, np.int32)
        B = len(ctxs)
        self.B = B
        self.L, self.FL = layers(window, fp8)
        logical = -(-int(self.ctxs.max()) // PAGE)
        self.bt_stride = logical
        if full_table:
            self.bt, nb = synth.shuffled_block_table(0, tag + (synth.PERM,), B,
                                                     [-(-int(c) // PAGE) for c in ctxs], logical)
        else:
            self.bt, nb = synth.ring_block_table(0, tag + (synth.PERM,), B, logical, 33, logical)
        self.nb = nb
        if fp8 is None:
            self.kd = synth.normal_bf16_bits_torch(0, tag + (synth.KC,), oracle.k_cache_shape(nb),
                                                   dev())
            self.vd = synth.normal_bf16_bits_torch(0, tag + (synth.VC,), oracle.v_cache_shape(nb),
                                                   dev())
        else:
            self.kd = synth.fp8_codes_torch(0, tag + (synth.KC,), oracle.k_cache_shape(nb), dev())
            self.vd = synth.fp8_codes_torch(0, tag + (synth.VC,), oracle.v_cache_shape(nb), dev(),
                                            0x5F)
        torch.cuda.synchronize()
        # pristine host copies for the oracle (taken before the step appends)
        self.kc = down(self.kd)
        self.vc = down(self.vd)
        self.q_in = synth.normal(0, tag + (synth.Q,), (B, 32, 128))
        self.k_in = synth.normal(0, tag + (synth.K,), (B, 4, 128))
        self.v_in = synth.normal(0, tag + (synth.V,), (B, 4, 128))
        self.sinks = synth.normal(0, tag + (synth.SINK,), 32)
        self.qw = np.ones(128, np.float32)
        self.kw = np.ones(128, np.float32)
        t = self.ctxs - 1
        self.pos = t.astype(np.int32)
        self.slots = np.array([oracle.slot(self.bt, b, int(t[b])) for b in range(B)], np.int32)

    def run_gpu(self, pages_per_split=0):
        import torch
        import full_gqa_decode_amd as fl
        out = torch.empty((self.B, 32, 128), dtype=torch.float32, device=dev())
        fl.flint_attn_decode_step(self.FL, up(self.q_in), up(self.k_in), up(self.v_in),
                                  up(self.qw), up(self.kw), up(self.slots), self.kd, self.vd,
                                  up(self.bt), up(self.ctxs), int(self.ctxs.max()),
                                  up(self.sinks), out, pages_per_split=pages_per_split)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle_step(self, sel):
        """Append every request's new token to the host caches (in place),
        then attention for the requests in `sel`."""
        q = oracle.append(self.L, self.q_in, self.k_in, self.v_in, self.qw, self.kw, self.pos,
                          self.slots, self.kc, self.vc)
        return oracle.attn_decode(self.L, q[sel], self.kc, self.vc, self.bt[sel], self.ctxs[sel],
                                  self.sinks)

    def check_written_rows(self):
        """The new tokens' cache rows: V bit-exact, K within one bf16 ulp (one
        fp8 grid step) of the oracle's correctly rounded value (ties of the
        fp64 value aside)."""
        k_gpu = down(self.kd) if self.nb * 4 * 16 * 128 < (1 << 28) else None
        for b in range(self.B):
            page, row = divmod(int(self.slots[b]), PAGE)
            if self.L.kv_fp8:
                # the fp8 tile order: rows gathered through the oracle's offsets
                vg = self.vd.view(self.nb, -1)[page].cpu().numpy()
                kg = self.kd.view(self.nb, -1)[page].cpu().numpy()
                for g in range(4):
                    v_ref = oracle.v_row(self.L, self.vc, page, g, row)
                    v_got = oracle.v_row(self.L, vg, 0, g, row)
                    assert np.array_equal(v_got, v_ref), f"V row of request {b}"
                    a = oracle.fp8_value(oracle.k_row(self.L, kg, 0, g, row))
                    r = oracle.fp8_value(oracle.k_row(self.L, self.kc, page, g, row))
                    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 2.0**-6))) - 3)
                    assert np.all(np.abs(a - r) <= step), f"K row of request {b}"
                continue
            v_ref = self.vc.reshape(self.nb, 4, 128, PAGE)[page, :, :, row]
            v_got = down(self.vd.view(self.nb, 4, 128, PAGE)[page, :, :, row])
            assert np.array_equal(v_got, v_ref), f"V row of request {b}"
            kg = k_gpu.reshape(self.nb, -1)[page] if k_gpu is not None else \
                down(self.kd.view(self.nb, -1)[page])
            for g in range(4):
                k_ref = oracle.k_row(self.L, self.kc, page, g, row)
                k_got = oracle.k_row(self.L, kg, 0, g, row)
                diff = np.abs(k_got.astype(np.int32) - k_ref.astype(np.int32))
                assert diff.max() <= 1, f"K row of request {b}"
        return k_gpu


def test_bs1_100k_full_layer_step():
    import full_gqa_decode_amd as fl
    case = BigStep((11, 1), [100_000], window=0, full_table=True)
    assert fl.flint_attn_decode_plan(case.FL, 1, 100_000) == (98, 64)
    got = case.run_gpu()
    ref = case.oracle_step(np.arange(1))
    err = float(np.abs(got - ref).max())
    print(f"bs1 100K full layer: max err {err:.3e}", flush=True)
    check_err(err, ref)
    k_gpu = case.check_written_rows()
    # nothing but the new token's row changed anywhere in the 204.8 MB cache
    assert k_gpu is not None
    slot = int(case.slots[0])
    kr = k_gpu.reshape(-1).copy()
    for g in range(4):
        off = oracle.k_offsets(case.L, slot // PAGE, g, slot % PAGE)
        kr[off] = case.kc.reshape(-1)[off]
    assert np.array_equal(kr, case.kc.reshape(-1))
    assert np.array_equal(case.vd.cpu().numpy().view(np.uint16), case.vc)


@pytest.mark.parametrize("pps", [0, 5])
def test_bs1_100k_sliding_layer_step(pps):
    # the default plan (one launch of 16-dim slice workgroups) and the
    # key-split plan (7 splits of 5 pages and a merge launch)
    import full_gqa_decode_amd as fl
    case = BigStep((11, 2), [100_000], window=513, full_table=False)
    assert fl.flint_attn_decode_plan(case.FL, 1, 100_000, pps) == ((33, 1) if pps == 0 else (5, 7))
    got = case.run_gpu(pps)
    ref = case.oracle_step(np.arange(1))
    err = float(np.abs(got - ref).max())
    print(f"bs1 100K sliding layer: max err {err:.3e}", flush=True)
    check_err(err, ref)
    case.check_written_rows()


MAX_CONTEXT = 262_144


def test_bs1_max_context_full_layer_step():
    # the plan at the maximum context: 128-page splits x 128 splits x 4 KV
    # heads = 512 workgroups (two rounds), folded by the >64-split merge
    import full_gqa_decode_amd as fl
    assert fl.flint_attn_decode_plan(fl.full_layer(), 1, MAX_CONTEXT) == (128, 128)
    case = BigStep((11, 9), [MAX_CONTEXT], window=0, full_table=True)
    got = case.run_gpu()
    ref = case.oracle_step(np.arange(1))
    err = float(np.abs(got - ref).max())
    print(f"bs1 262,144-token full layer: max err {err:.3e}", flush=True)
    check_err(err, ref)
    case.check_written_rows()


def test_bs1_max_context_sliding_layer_step():
    # the new token at position 262,143: RoPE angles pos * theta^(-2i/128)
    # up to 2.6e5 rad, reduced on the GPU in fp64
    import full_gqa_decode_amd as fl
    case = BigStep((11, 10), [MAX_CONTEXT], window=513, full_table=False)
    got = case.run_gpu()
    ref = case.oracle_step(np.arange(1))
    err = float(np.abs(got - ref).max())
    print(f"bs1 262,144-token sliding layer: max err {err:.3e}", flush=True)
    check_err(err, ref)
    case.check_written_rows()
    # the stand-alone append at that position: q rotated like the oracle's
    import torch
    qo = torch.empty((1, 32, 128), dtype=torch.float32, device=dev())
    kd = torch.empty_like(case.kd)
    vd = torch.empty_like(case.vd)
    fl.flint_qk_norm_rope_append(case.FL, up(case.q_in), up(case.k_in), up(case.v_in),
                                 up(case.qw), up(case.kw), up(case.pos),
                                 up(np.array([-1], np.int32)), qo, kd, vd)
    torch.cuda.synchronize()
    q_ref = oracle.append(case.L, case.q_in, case.k_in, case.v_in, case.qw, case.kw, case.pos,
                          np.array([-1], np.int32), case.kc.copy(), case.vc.copy())
    assert np.abs(qo.cpu().numpy() - q_ref).max() < 1e-6


def ragged_lengths():
    return synth.uniform_ints(0, (11, 3), 64, 1024, 131072)


def test_ragged_64_requests_full_layer_full_size():
    lens = ragged_lengths()
    case = BigStep((11, 4), lens, window=0, full_table=True)
    got = case.run_gpu()
    assert np.isfinite(got).all()
    ref = case.oracle_step(np.arange(64))
    err = float(np.abs(got - ref).max())
    print(f"64 ragged requests, full layer, {int(lens.sum())} keys: all 64 checked, "
          f"max err {err:.3e}", flush=True)
    check_err(err, ref)
    case.check_written_rows()


def test_ragged_64_requests_sliding_layer_full_size():
    lens = ragged_lengths()
    case = BigStep((11, 6), lens, window=513, full_table=False)
    got = case.run_gpu()
    ref = case.oracle_step(np.arange(64))
    err = float(np.abs(got - ref).max())
    print(f"64 ragged requests, sliding layer: max err {err:.3e}", flush=True)
    check_err(err, ref)
    case.check_written_rows()


def test_bs1_100k_full_layer_step_fp8():
    # the fp8 cache of the same workload: 102.4 MB of codes (K below 2 and V
    # below 30 before the scales)
    import full_gqa_decode_amd as fl
    case = BigStep((11, 7), [100_000], window=0, full_table=True, fp8=(1.0, 0.25))
    got = case.run_gpu()
    ref = case.oracle_step(np.arange(1))
    err = float(np.abs(got - ref).max())
    print(f"bs1 100K full layer, fp8 cache: max err {err:.3e}", flush=True)
    check_err(err, ref)
    k_gpu = case.check_written_rows()
    # nothing but the new token's K row changed in the 51.2 MB K cache
    slot = int(case.slots[0])
    kr = k_gpu.reshape(-1).copy()
    for g in range(4):
        off = oracle.k_offsets(case.L, slot // PAGE, g, slot % PAGE)
        kr[off] = case.kc.reshape(-1)[off]
    assert np.array_equal(kr, case.kc.reshape(-1))


def test_ragged_64_requests_sliding_layer_fp8():
    lens = ragged_lengths()
    case = BigStep((11, 8), lens, window=513, full_table=False, fp8=(1.0 / 16, 0.25))
    got = case.run_gpu()
    ref = case.oracle_step(np.arange(64))
    err = float(np.abs(got - ref).max())
    print(f"64 ragged requests, sliding layer, fp8 cache: max err {err:.3e}", flush=True)
    check_err(err, ref)
    case.check_written_rows()


def test_bs1_max_context_full_layer_step_fp8():
    # the fp8 cache at the maximum context: the same 128 x 128 plan, two
    # rounds of workgroups (the fp8 kernel's one-page loop) and the wide merge
    import full_gqa_decode_amd as fl
    L = fl.layer(window=0, use_rope=0, kv_dtype=fl.FLINT_KV_FP8_E4M3, k_scale=1.0, v_scale=0.25)
    assert fl.flint_attn_decode_plan(L, 1, MAX_CONTEXT) == (128, 128)
    case = BigStep((11, 12), [MAX_CONTEXT], window=0, full_table=True, fp8=(1.0, 0.25))
    got = case.run_gpu()
    ref = case.oracle_step(np.arange(1))
    err = float(np.abs(got - ref).max())
    print(f"bs1 262,144-token full layer, fp8 cache: max err {err:.3e}", flush=True)
    check_err(err, ref)
    case.check_written_rows()


def test_ragged_64_requests_full_layer_fp8():
    # 64 requests of 1024..131072 tokens over an fp8 cache (about 4 GB of
    # codes): a multi-round plan; every request's output and cache write checked
    lens = ragged_lengths()
    case = BigStep((11, 13), lens, window=0, full_table=True, fp8=(1.0 / 16, 0.25))
    got = case.run_gpu()
    assert np.isfinite(got).all()
    ref = case.oracle_step(np.arange(64))
    err = float(np.abs(got - ref).max())
    print(f"64 ragged requests, full layer, fp8 cache: all 64 checked, max err {err:.3e}",
          flush=True)
    check_err(err, ref)
    case.check_written_rows()
