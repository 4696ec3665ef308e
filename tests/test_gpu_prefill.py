"""GPU parity of the MFMA prefill path (K1 append with bf16 q -> K4) against
the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
import flint_cases as fc
from flint_cases import GUARD, PREFILL_GUARD, TOL, dev, empty_caches, layers, max_err, up


def assert_parity(got, ref, what=""):
    """The contract and the prefill guard (fp16 P in the value product)."""
    return fc.assert_parity(got, ref, what, guard=PREFILL_GUARD)


def check_err(err, ref, what=""):
    return fc.check_err(err, ref, what, guard=PREFILL_GUARD)

pytestmark = pytest.mark.gpu


class PrefillCase:
    """Requests with (seq_len, q_len): every token is appended; the last q_len
    rows of each request are the chunk's queries."""

    def __init__(self, seed, reqs, window=0, fp8=None, hkv=4, **layer_kw):
        self.L, self.FL = layers(window, fp8, hkv, **layer_kw)
        self.hkv, self.hq = hkv, 8 * hkv
        self.reqs = reqs
        B = len(reqs)
        tag = (hash((tuple(reqs), window, 11)) & 0xFFFF,)
        self.bt_stride = max(-(-s // 16) for s, _ in reqs) + 1
        self.bt, nb = synth.shuffled_block_table(seed, tag + (synth.PERM,), B,
                                                 [-(-s // 16) for s, _ in reqs], self.bt_stride)
        self.num_blocks = nb + 2
        self.sinks = synth.normal(seed, tag + (synth.SINK,), self.hq)
        self.qw = synth.norm_weight(seed, tag + (synth.QW,), 128, False)
        self.kw = synth.norm_weight(seed, tag + (synth.KW,), 128, False)
        T = sum(s for s, _ in reqs)
        self.k_in = np.empty((T, hkv, 128), np.float32)
        self.v_in = np.empty((T, hkv, 128), np.float32)
        self.q_in = np.empty((T, self.hq, 128), np.float32)
        self.pos = np.empty(T, np.int32)
        self.slots = np.empty(T, np.int32)
        chunk_rows, cu = [], [0]
        o = 0
        for b, (s, ql) in enumerate(reqs):
            self.k_in[o:o + s] = synth.normal(seed, tag + (synth.K, b), (s, hkv, 128))
            self.v_in[o:o + s] = synth.normal(seed, tag + (synth.V, b), (s, hkv, 128))
            self.q_in[o:o + s] = synth.normal(seed, tag + (synth.Q, b), (s, self.hq, 128))
            self.pos[o:o + s] = np.arange(s)
            self.slots[o:o + s] = [oracle.slot(self.bt, b, p) for p in range(s)]
            chunk_rows += list(range(o + s - ql, o + s))
            cu.append(cu[-1] + ql)
            o += s
        self.chunk_rows = np.array(chunk_rows, np.int64)
        self.cu = np.array(cu, np.int32)
        self.seq_lens = np.array([s for s, _ in reqs], np.int32)
        self.max_q = max(ql for _, ql in reqs)

    def expected(self, rows=None):
        """Oracle: append K/V for every token, q for the chunk rows, round q to
        bf16 (the prefill q format), then O7 on `rows` of the chunk."""
        kc, vc = empty_caches(self.L, self.num_blocks)
        oracle.append(self.L, self.q_in[:1], self.k_in, self.v_in, self.qw, self.kw, self.pos,
                      self.slots, kc, vc, want_q=False)
        need = self.chunk_rows if rows is None else self.chunk_rows[rows]
        skip = np.full(len(need), -1, np.int32)
        qh = oracle.append(self.L, self.q_in[need], self.k_in[need], self.v_in[need], self.qw,
                           self.kw, self.pos[need], skip, kc, vc)
        qb = oracle.bf16_rne_f64(qh)
        qf = synth.bf16_bits_to_f32(qb).astype(np.float64)
        full_q = np.zeros((len(self.chunk_rows), self.hq, 128))
        idx = np.arange(len(self.chunk_rows)) if rows is None else np.asarray(rows)
        full_q[idx] = qf
        return oracle.attn_prefill(self.L, full_q, self.cu, kc, vc, self.bt, self.seq_lens,
                                   self.sinks, rows=None if rows is None else idx)

    def run_gpu(self, bt=None, seq_lens=None, workspace=None):
        import torch
        import full_gqa_decode_amd as fl
        kd, vd = empty_caches(self.L, self.num_blocks, device=True)
        qb = torch.empty(self.q_in.shape, dtype=torch.int16, device=dev())
        fl.flint_qk_norm_rope_append(self.FL, up(self.q_in), up(self.k_in), up(self.v_in),
                                     up(self.qw), up(self.kw), up(self.pos), up(self.slots), qb,
                                     kd, vd)
        qc = qb[torch.from_numpy(self.chunk_rows).to(dev())].contiguous()
        out = torch.empty((len(self.chunk_rows), self.hq, 128), dtype=torch.float32,
                          device=dev())
        bt = self.bt if bt is None else bt
        sl = self.seq_lens if seq_lens is None else seq_lens
        fl.flint_attn_prefill(self.FL, qc, up(self.cu), self.max_q, kd, vd, up(bt), up(sl),
                              int(self.seq_lens.max()), up(self.sinks), out, workspace)
        torch.cuda.synchronize()
        return out.cpu().numpy(), kd, vd, qb


@pytest.mark.parametrize("window", [0, 513])
def test_prefill_whole_prompt(window):
    case = PrefillCase(0, [(700, 700)], window=window)
    got, _, _, _ = case.run_gpu()
    assert_parity(got, case.expected())


@pytest.mark.parametrize("window", [0, 513])
def test_prefill_chunk_ragged_batch(window):
    # chunks that start mid-page, a one-row chunk, a chunk shorter than a page
    case = PrefillCase(1, [(1000, 300), (37, 1), (530, 530), (65, 9)], window=window)
    got, _, _, _ = case.run_gpu()
    assert_parity(got, case.expected())


def test_windowed_prefill_with_chunk_starts_at_every_offset_mod_16():
    # A chunk that starts at position base sees its window start at base - 512
    # + row.  For base % 16 != 0 the first page pair a wave reads can hold
    # keys of its first row's window while its later rows see none of them
    # yet; those rows must come out finite and right.
    reqs = [(513 + r + 96, 96) for r in range(16)]
    case = PrefillCase(14, reqs, window=513)
    got, _, _, _ = case.run_gpu()
    bad = int((~np.isfinite(got)).sum())
    assert bad == 0, f"{bad} non-finite outputs"
    assert_parity(got, case.expected())


def test_last_prefill_row_matches_decode_at_same_position():
    import torch
    import full_gqa_decode_amd as fl
    case = PrefillCase(2, [(900, 64)], window=0)
    got, kd, vd, _ = case.run_gpu()
    # decode of the last row with fp32 q from the same append
    qf = torch.empty(case.q_in.shape, dtype=torch.float32, device=dev())
    kd2 = torch.empty_like(kd)
    vd2 = torch.empty_like(vd)
    fl.flint_qk_norm_rope_append(case.FL, up(case.q_in), up(case.k_in), up(case.v_in),
                                 up(case.qw), up(case.kw), up(case.pos), up(case.slots), qf, kd2,
                                 vd2)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=dev())
    fl.flint_attn_decode(case.FL, qf[-1:].contiguous(), kd, vd, up(case.bt), up(case.seq_lens),
                         900, up(case.sinks), out)
    torch.cuda.synchronize()
    assert max_err(got[-1], out.cpu().numpy()[0].astype(np.float64)) <= 2 * TOL


def prefill_sample_rows(window, T=32768):
    """Rows of the 32,768-token prompt the oracle checks: rows 0..599, one
    whole 32-row workgroup tile mid-prompt (rows 16384..16415), a stride
    coprime with 32 (509 for the full layer, 7 for the cheaper windowed
    one) so that every row offset inside a tile is checked mid-prompt, and
    the last 64 rows."""
    stride = 7 if window else 509
    assert np.gcd(stride, 32) == 1
    rows = np.unique(np.concatenate([np.arange(600), np.arange(16384, 16416),
                                     np.arange(3, T, stride), np.arange(T - 64, T)]))
    assert len(np.unique(rows[(rows >= 600) & (rows < T - 64)] % 32)) == 32
    return rows


@pytest.mark.parametrize("window", [0, 513])
def test_prefill_32768_token_prompt_sampled_rows(window):
    # causal prefill of a 32,768-token prompt; the oracle checks sampled rows
    case = PrefillCase(0, [(32768, 32768)], window=window)
    got, _, _, _ = case.run_gpu()
    rows = prefill_sample_rows(window)
    ref = case.expected(rows=rows)
    err = check_err(max_err(got[rows], ref[rows]), ref[rows])
    print(f"prefill 32768 window {window}: {len(rows)} rows checked, max err {err:.3e}",
          flush=True)
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("window", [0, 513])
def test_prefill_short_chunk_at_the_end_of_a_long_context(window):
    case = PrefillCase(4, [(12000, 80)], window=window)
    got, _, _, _ = case.run_gpu()
    assert_parity(got, case.expected())


def test_prefill_empty_chunk_in_a_batch():
    case = PrefillCase(5, [(100, 50), (64, 0), (200, 20)], window=0)
    got, _, _, _ = case.run_gpu()
    assert got.shape[0] == 70
    assert_parity(got, case.expected())


@pytest.mark.parametrize("window", [0, 513])
def test_prefill_invalid_requests_give_nan_and_spare_the_rest(window):
    # request 1: a page id past num_blocks; request 2: a chunk longer than
    # its context.  Both come out NaN; request 0 is untouched by them.
    case = PrefillCase(6, [(300, 100), (200, 50), (150, 150)], window=window)
    bt = case.bt.copy()
    bt[1, 3] = case.num_blocks + 7
    sl = case.seq_lens.copy()
    sl[2] = 149
    got, _, _, _ = case.run_gpu(bt=bt, seq_lens=sl)
    assert np.isnan(got[100:300]).all()
    ok = PrefillCase(6, [(300, 100), (200, 50), (150, 150)], window=window).expected(
        rows=np.arange(100))
    assert_parity(got[:100], ok[:100])


def _many_requests():
    """24 requests with chunks of 1..119 rows on contexts up to 300 tokens
    longer, request 0 the longest chunk (200 rows: 7 row blocks), request 5
    an empty chunk."""
    rng = np.random.default_rng(21)
    reqs = []
    for _ in range(24):
        ql = int(rng.integers(1, 120))
        reqs.append((ql + int(rng.integers(0, 300)), ql))
    reqs[0] = (600, 200)
    reqs[5] = (reqs[5][0], 0)
    return reqs


@pytest.mark.parametrize("window", [0, 513])
def test_prefill_many_requests_more_items_than_workgroups(window):
    # 7 row blocks x 4 KV heads x 24 requests = 672 work items for the 256
    # workgroups of the persistent grid, most of them past the end of a
    # short chunk.  Request 9 holds a page id past num_blocks and request 14
    # a chunk longer than its context: their rows come out NaN, and the
    # workgroups that meet them go on to the next items unharmed.
    reqs = _many_requests()
    case = PrefillCase(7, reqs, window=window)
    bt = case.bt.copy()
    bt[9, 1] = case.num_blocks + 3
    sl = case.seq_lens.copy()
    sl[14] = reqs[14][1] - 1
    got, _, _, _ = case.run_gpu(bt=bt, seq_lens=sl)
    bad = np.zeros(len(case.chunk_rows), bool)
    for b in (9, 14):
        bad[case.cu[b]:case.cu[b + 1]] = True
    assert bad.sum() > 0 and np.isnan(got[bad]).all()
    good = np.flatnonzero(~bad)
    want = case.expected(rows=good)
    assert_parity(got[good], want[good])


def _sample(n, stride=7):
    rows = np.concatenate([np.arange(min(n, 64)), np.arange(3, n, stride), np.arange(n - 64, n)])
    return np.unique(rows[(rows >= 0) & (rows < n)])


@pytest.mark.parametrize("window,hkv,reqs", [
    (513, 1, [(257 * 32, 257 * 32)]),                             # 257 items: one claimed
    (0, 4, [(65 * 32 + 5, 65 * 32)]),                             # 260 items
    (513, 2, [(3000, 1500), (40, 40), (900, 0), (2100, 2000)]),   # 504, many without rows
])
def test_prefill_claimed_items_share_one_workspace_across_calls(window, hkv, reqs):
    # Past 256 work items the persistent grid claims the later ones from a
    # counter in the workspace, which must be zero when a call starts and
    # which every call leaves zero: two calls in a row on one workspace give
    # the same, correct output and leave it zero.
    import torch
    import full_gqa_decode_amd as fl
    case = PrefillCase(15, reqs, window=window, hkv=hkv)
    need = fl.flint_attn_prefill_workspace_size(case.FL, len(reqs), case.max_q,
                                                int(case.seq_lens.max()))
    items = -(-case.max_q // 32) * hkv * len(reqs)
    assert need == 16 + 4 * items
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    first, _, _, _ = case.run_gpu(workspace=ws)
    assert not ws.any().item()
    second, _, _, _ = case.run_gpu(workspace=ws)
    assert not ws.any().item()
    assert np.array_equal(first, second)
    rows = _sample(len(case.chunk_rows))
    want = case.expected(rows=rows)
    assert_parity(first[rows], want[rows])


def test_prefill_graph_replays_match_eager():
    import torch
    import full_gqa_decode_amd as fl
    case = PrefillCase(7, [(700, 300), (90, 90)], window=513)
    eager, kd, vd, qb = case.run_gpu()
    qc = qb[torch.from_numpy(case.chunk_rows).to(dev())].contiguous()
    cu, bt, sl, sk = up(case.cu), up(case.bt), up(case.seq_lens), up(case.sinks)
    out = torch.empty((len(case.chunk_rows), 32, 128), dtype=torch.float32, device=dev())
    ws = torch.zeros(fl.flint_attn_prefill_workspace_size(case.FL, 2, case.max_q, 700),
                     dtype=torch.uint8, device=dev())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fl.flint_attn_prefill(case.FL, qc, cu, case.max_q, kd, vd, bt, sl,
                                  int(case.seq_lens.max()), sk, out, ws)
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager)
        # eager work between replays
        fl.flint_attn_prefill(case.FL, qc, cu, case.max_q, kd, vd, bt, sl,
                              int(case.seq_lens.max()), sk, torch.empty_like(out))
        torch.cuda.synchronize()


def test_prefill_graph_with_claimed_items_replays_match_eager():
    # 7 row blocks x 4 heads x 24 requests = 672 items, the later ones claimed:
    # each replay finds the counter the previous launch left at zero
    import torch
    import full_gqa_decode_amd as fl
    reqs = _many_requests()
    case = PrefillCase(16, reqs, window=513)
    eager, kd, vd, qb = case.run_gpu()
    qc = qb[torch.from_numpy(case.chunk_rows).to(dev())].contiguous()
    cu, bt, sl, sk = up(case.cu), up(case.bt), up(case.seq_lens), up(case.sinks)
    ws = torch.zeros(fl.flint_attn_prefill_workspace_size(case.FL, len(reqs), case.max_q,
                                                          int(case.seq_lens.max())),
                     dtype=torch.uint8, device=dev())
    out = torch.empty((len(case.chunk_rows), 32, 128), dtype=torch.float32, device=dev())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fl.flint_attn_prefill(case.FL, qc, cu, case.max_q, kd, vd, bt, sl,
                                  int(case.seq_lens.max()), sk, out, ws)
    torch.cuda.synchronize()
    assert not ws.any().item()  # captured, not run
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager)
        assert not ws.any().item()
        fl.flint_attn_prefill(case.FL, qc, cu, case.max_q, kd, vd, bt, sl,
                              int(case.seq_lens.max()), sk, torch.empty_like(out), ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("window,reqs", [(0, [(700, 700)]), (513, [(700, 700)]),
                                         (0, [(1000, 300), (37, 1), (65, 9)]),
                                         (513, [(1200, 520), (530, 17)])])
def test_prefill_over_an_fp8_cache(window, reqs):
    # the fp8 tile order widened while staged; unwritten slots hold the NaN code
    case = PrefillCase(12, reqs, window=window, fp8=(1.0 / 16, 0.5))
    got, _, _, _ = case.run_gpu()
    err = max_err(got, case.expected())
    print(f"fp8 prefill window {window} {reqs}: max err {err:.3e}", flush=True)
    check_err(err, case.expected())


def test_last_fp8_prefill_row_matches_fp8_decode():
    # prefill and decode read the same fp8 cache the same way
    import torch
    import full_gqa_decode_amd as fl
    case = PrefillCase(13, [(900, 40)], window=0, fp8=(1.0 / 16, 0.5))
    got, kd, vd, _ = case.run_gpu()
    qf = torch.empty(case.q_in.shape, dtype=torch.float32, device=dev())
    kd2, vd2 = empty_caches(case.L, case.num_blocks, device=True)
    fl.flint_qk_norm_rope_append(case.FL, up(case.q_in), up(case.k_in), up(case.v_in),
                                 up(case.qw), up(case.kw), up(case.pos), up(case.slots), qf, kd2,
                                 vd2)
    assert torch.equal(kd, kd2) and torch.equal(vd, vd2)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=dev())
    fl.flint_attn_decode(case.FL, qf[-1:].contiguous(), kd, vd, up(case.bt), up(case.seq_lens),
                         900, up(case.sinks), out)
    torch.cuda.synchronize()
    # prefill's q is bf16, decode's fp32: they agree to the bf16 rounding of q
    assert np.abs(got[-1] - out.cpu().numpy()[0]).max() <= TOL


@pytest.mark.parametrize("window", [0, 513])
def test_prefill_values_beyond_fp16_range_are_recomputed_in_bf16(window):
    # V values past fp16's range (65504) in a bf16 cache: the work items whose
    # page pairs hold them are flagged and recomputed by the fix-up launch
    # with bf16 V; every other item keeps the fp16 value product.  The
    # workspace's flags and counts are back at zero after each call, and a
    # second call on the same workspace gives the same result.
    import torch
    import full_gqa_decode_amd as fl
    case = PrefillCase(23, [(700, 700), (300, 100)], window=window)
    case.v_in[600:611] *= 3.0e4          # request 0, positions 600..610: |V| up to ~1.3e5
    assert np.abs(case.v_in[600:611]).max() > 65504
    want = case.expected()
    ws = torch.zeros(fl.flint_attn_prefill_workspace_size(case.FL, 2, case.max_q, 700),
                     dtype=torch.uint8, device=dev())
    first = None
    for _ in range(2):
        got, _, _, _ = case.run_gpu(workspace=ws)
        assert int(ws.count_nonzero()) == 0
        if first is None:
            first = got
        assert np.array_equal(got, first)
    assert np.isfinite(got).all()
    # rows that see none of the large values: the contract and the guard
    far = np.r_[0:576, 700:800]
    assert_parity(got[far], want[far])
    # rows that average values of ~1e5: the bar relative to each row's scale
    # (a fixed 4e-3 presumes outputs of order one)
    for r in range(576, 700):
        err = max_err(got[r], want[r])
        assert err <= GUARD * max(1.0, float(np.abs(want[r]).max())), (r, err)
    # the same chunk without the large values takes no fix-up (nothing flagged)
    plain = PrefillCase(23, [(700, 700), (300, 100)], window=window)
    got2, _, _, _ = plain.run_gpu(workspace=ws)
    assert int(ws.count_nonzero()) == 0
    assert_parity(got2, plain.expected())
