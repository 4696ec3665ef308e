"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against something it does not compute itself:
values the pages print, closed forms, invariants, an independent library
routine (torch's bf16 conversion, numpy complex rotation) or brute force in
50-digit arithmetic on tiny inputs.  The comment on each test names the
plausible oracle mistake it would catch.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ---------------------------------------------------------------------------
# O1 bf16
# ---------------------------------------------------------------------------

def test_bf16_widen_matches_bit_view():
    # all 65536 patterns: the definition-based value equals reading the bits as
    # the top half of an fp32 (catches a wrong bias / subnormal scale)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_value(bits)
    with np.errstate(invalid="ignore"):
        ref = synth.bf16_bits_to_f32(bits).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _torch_bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_bf16_rne_matches_torch():
    # independent library rounding: catches truncation instead of RNE, a wrong
    # tie rule, overflow and subnormal handling
    r = synth.rng(0, 99, 1)
    u = r.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    specials = np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 1.0078125,
                         3.3895314e38, 3.3961e38, 3.4028235e38, -3.4028235e38, 1e-40, -1e-45,
                         1.1754944e-38, 9.18e-41, np.inf, -np.inf], dtype=np.float32)
    halfway = (((np.arange(4096, dtype=np.uint32) << 16) | 0x8000)).view(np.float32)
    halfway = halfway[np.isfinite(halfway)]
    for arr in (x, specials, halfway):
        assert np.array_equal(oracle.bf16_rne(arr), _torch_bf16_bits(arr))


def test_bf16_rne_f64_matches_torch_and_midpoints():
    r = synth.rng(0, 99, 2)
    x = r.standard_normal(50_000).astype(np.float32)
    assert np.array_equal(oracle.bf16_rne_f64(x.astype(np.float64)), _torch_bf16_bits(x))
    # a value just above a bf16 midpoint rounds up even though its fp32 image
    # (the midpoint itself, a tie) would round to even = down
    mid = 1.0 + 2.0 ** -8                      # halfway between 1.0 and 1 + 2^-7
    assert oracle.bf16_rne_f64([mid])[0] == 0x3F80
    assert oracle.bf16_rne_f64([mid + 2.0 ** -40])[0] == 0x3F81
    assert oracle.bf16_rne_f64([-(mid + 2.0 ** -40)])[0] == 0xBF81


def test_bf16_nan_stays_nan():
    b = oracle.bf16_rne([np.float32("nan")])[0]
    assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


# ---------------------------------------------------------------------------
# O2 RMSNorm
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_rmsnorm_rms_closed_form(eps):
    # with w = 1 the output RMS is sqrt(ms/(ms+eps)): catches sum-vs-mean and
    # eps outside the square root
    x = synth.normal(1, (7,), 128) * 3.0
    y = oracle.rmsnorm(x, np.ones(128, np.float32), eps)
    ms = np.mean(x.astype(np.float64) ** 2)
    assert math.isclose(np.sqrt(np.mean(y ** 2)), math.sqrt(ms / (ms + eps)), rel_tol=1e-13)


def test_rmsnorm_scale_invariance_and_weight():
    # eps = 0: RMSNorm(c x) = RMSNorm(x); weight multiplies elementwise
    x = synth.normal(2, (1,), 128)
    w = synth.norm_weight(2, (2,), 128, ones=False)
    y1 = oracle.rmsnorm(x, w, 0.0)
    y2 = oracle.rmsnorm(x * np.float32(4.0), w, 0.0)
    y0 = oracle.rmsnorm(x, np.ones(128, np.float32), 0.0)
    assert np.allclose(y1, y2, rtol=1e-14, atol=0)
    assert np.allclose(y1, y0 * w.astype(np.float64), rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------
# O3 RoPE
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("pos", [0, 1, 511, 99999, 262143])
def test_rope_is_complex_rotation(pos):
    # independent formulation: z_i = x_i + i x_{i+64} times exp(i pos theta^(-2i/128));
    # catches a wrong sign, the interleaved pairing and a wrong frequency exponent
    x = synth.normal(3, (pos,), 128).astype(np.float64)
    y = oracle.rope(x, pos)
    i = np.arange(64)
    freq = np.exp(-(2.0 * i / 128.0) * np.log(10000.0))
    z = (x[:64] + 1j * x[64:]) * np.exp(1j * (pos * freq))
    assert np.allclose(y[:64], z.real, rtol=0, atol=1e-9)
    assert np.allclose(y[64:], z.imag, rtol=0, atol=1e-9)


def test_rope_relative_position():
    # <rope(q, a), rope(k, b)> depends only on a - b
    q = synth.normal(4, (1,), 128).astype(np.float64)
    k = synth.normal(4, (2,), 128).astype(np.float64)
    d0 = np.dot(oracle.rope(q, 700), oracle.rope(k, 650))
    d1 = np.dot(oracle.rope(q, 50), oracle.rope(k, 0))
    d2 = np.dot(oracle.rope(q, 100050), oracle.rope(k, 100000))
    assert math.isclose(d0, d1, rel_tol=1e-11) and math.isclose(d0, d2, rel_tol=1e-9)


# ---------------------------------------------------------------------------
# attention: helpers to build a small paged problem
# ---------------------------------------------------------------------------

def _paged(L, dense_k_bits, dense_v_bits, seed, perm=True):
    """Place dense [n, hkv, d] bf16 rows of one request into a shuffled paged
    cache; returns (kc, vc, block_tables)."""
    n = dense_k_bits.shape[0]
    pages = -(-n // L.bs)
    extra = 3
    order = synth.permutation(seed, (77,), pages + extra) if perm else np.arange(pages + extra)
    bt = np.full((1, pages + 2), -1, np.int32)
    bt[0, :pages] = order[:pages]
    kl = np.full((pages + extra, L.hkv, L.bs, L.d), 0x7FC0, np.uint16)  # NaN where unused
    vc = np.full((pages + extra, L.hkv, L.d, L.bs), 0x7FC0, np.uint16)
    for p in range(n):
        pg, r = bt[0, p // L.bs], p % L.bs
        kl[pg, :, r, :] = dense_k_bits[p]
        vc[pg, :, :, r] = dense_v_bits[p]
    return oracle.k_to_cache(L, kl), vc, bt


def _brute(L, q, kbits, vbits, t, sinks, lo=None):
    """50-digit evaluation of the definition on dense (unpaged) rows, without
    max subtraction: out_h = sum_j e^{s_j} V_j / (e^{sink_h} + sum_j e^{s_j})."""
    mpmath.mp.dps = 50
    kf = synth.bf16_bits_to_f32(kbits).astype(np.float64)
    vf = synth.bf16_bits_to_f32(vbits).astype(np.float64)
    if lo is None:
        lo = max(0, t - L.window + 1) if L.window > 0 else 0
    grp = L.hq // L.hkv
    out = np.empty((L.hq, L.d))
    sc = mpmath.mpf(1) / mpmath.sqrt(L.d)
    for h in range(L.hq):
        g = h // grp
        es = []
        for j in range(lo, t + 1):
            s = mpmath.fsum(mpmath.mpf(float(q[h, i])) * mpmath.mpf(float(kf[j, g, i]))
                            for i in range(L.d))
            es.append(mpmath.exp(sc * s))
        z = mpmath.exp(mpmath.mpf(float(sinks[h]))) + mpmath.fsum(es)
        for i in range(L.d):
            out[h, i] = float(mpmath.fsum(e * mpmath.mpf(float(vf[lo + jj, g, i]))
                                          for jj, e in enumerate(es)) / z)
    return out


def _small_layer(window=0):
    return oracle.layer(window=window, hq=4, hkv=2, d=8, bs=4)


@pytest.mark.parametrize("n,window", [(1, 0), (3, 0), (7, 0), (9, 5), (6, 3)])
def test_attention_brute_force_small_shape(n, window):
    # catches a wrong GQA head mapping, a transposed K/V index, a wrong scale,
    # a dropped sink term and window off-by-one, on a shape other than Flint's
    L = _small_layer(window)
    kb = synth.normal_bf16_bits(5, (n, 1), (n, L.hkv, L.d))
    vb = synth.normal_bf16_bits(5, (n, 2), (n, L.hkv, L.d))
    q = synth.normal(5, (n, 3), (L.hq, L.d)).astype(np.float64)
    sinks = synth.normal(5, (n, 4), L.hq)
    kc, vc, bt = _paged(L, kb, vb, seed=n)
    out = oracle.attn_decode(L, q[None], kc, vc, bt, np.array([n], np.int32), sinks)[0]
    ref = _brute(L, q, kb, vb, n - 1, sinks)
    assert np.max(np.abs(out - ref)) < 1e-15


@pytest.mark.parametrize("n,window", [(5, 0), (8, 0), (8, 513)])
def test_attention_brute_force_flint_shape(n, window):
    L = oracle.layer(window=window, use_rope=1 if window else 0)
    kb = synth.normal_bf16_bits(6, (n, 1), (n, 4, 128))
    vb = synth.normal_bf16_bits(6, (n, 2), (n, 4, 128))
    q = synth.normal(6, (n, 3), (32, 128)).astype(np.float64)
    sinks = synth.normal(6, (n, 4), 32)
    kc, vc, bt = _paged(L, kb, vb, seed=n)
    out = oracle.attn_decode(L, q[None], kc, vc, bt, np.array([n], np.int32), sinks)[0]
    ref = _brute(L, q, kb, vb, n - 1, sinks)
    assert np.max(np.abs(out - ref)) < 1e-14


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _flint_case(n, seed, window=0, same_keys=False, q_zero=False, sink=None):
    L = oracle.layer(window=window)
    kb = synth.normal_bf16_bits(seed, (1,), (n, 4, 128))
    if same_keys:
        kb[:] = kb[0]
    vb = synth.normal_bf16_bits(seed, (2,), (n, 4, 128))
    q = synth.normal(seed, (3,), (32, 128)).astype(np.float64)
    if q_zero:
        q[:] = 0.0
    sinks = synth.normal(seed, (4,), 32)
    if sink is not None:
        sinks[:] = sink
    kc, vc, bt = _paged(L, kb, vb, seed)
    out = oracle.attn_decode(L, q[None], kc, vc, bt, np.array([n], np.int32), sinks)[0]
    kf = synth.bf16_bits_to_f32(kb).astype(np.float64)
    vf = synth.bf16_bits_to_f32(vb).astype(np.float64)
    return L, q, kf, vf, sinks.astype(np.float64), out


def test_identical_keys_give_sink_weighted_mean():
    # all scores equal s: out = (1 - w) mean_j V_j with w = e^sink/(e^sink + n e^s)
    n = 37
    L, q, kf, vf, sinks, out = _flint_case(n, 11, same_keys=True)
    for h in range(32):
        g = h // 8
        s = np.dot(q[h], kf[0, g]) / math.sqrt(128)
        w = math.exp(sinks[h]) / (math.exp(sinks[h]) + n * math.exp(s))
        assert np.allclose(out[h], (1 - w) * vf[:, g].mean(axis=0), rtol=0, atol=1e-13)


def test_sink_minus_inf_is_plain_softmax():
    # library softmax (scipy) as the independent routine
    from scipy.special import softmax
    n = 50
    L, q, kf, vf, sinks, out = _flint_case(n, 12, sink=-np.inf)
    for h in range(32):
        g = h // 8
        p = softmax(kf[:, g] @ q[h] / math.sqrt(128))
        assert np.allclose(out[h], p @ vf[:, g], rtol=0, atol=1e-13)


def test_zero_query_gives_value_sum_over_n_plus_exp_sink():
    n = 21
    L, q, kf, vf, sinks, out = _flint_case(n, 13, q_zero=True)
    for h in range(32):
        assert np.allclose(out[h], vf[:, h // 8].sum(0) / (n + math.exp(sinks[h])), atol=1e-13)


def test_single_key_is_sigmoid_gate():
    # n = 1: out = V_0 * sigmoid(s_0 - sink)
    L, q, kf, vf, sinks, out = _flint_case(1, 14)
    for h in range(32):
        s = np.dot(q[h], kf[0, h // 8]) / math.sqrt(128)
        assert np.allclose(out[h], vf[0, h // 8] / (1 + math.exp(sinks[h] - s)), atol=1e-14)


def test_gqa_equal_heads_equal_outputs():
    L = oracle.layer()
    n = 40
    kb = synth.normal_bf16_bits(15, (1,), (n, 4, 128))
    vb = synth.normal_bf16_bits(15, (2,), (n, 4, 128))
    q = synth.normal(15, (3,), (32, 128)).astype(np.float64)
    q[8:16] = q[8]
    sinks = synth.normal(15, (4,), 32)
    sinks[8:16] = sinks[8]
    kc, vc, bt = _paged(L, kb, vb, 15)
    out = oracle.attn_decode(L, q[None], kc, vc, bt, np.array([n], np.int32), sinks)[0]
    for h in range(9, 16):
        assert np.array_equal(out[h], out[8])
    assert not np.allclose(out[0], out[8])


# ---------------------------------------------------------------------------
# window (P3)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 17, 512, 513])
def test_sliding_equals_full_below_window(n):
    # t = n - 1 < 513: the window covers every key
    Lf, Ls = oracle.layer(window=0), oracle.layer(window=513)
    kb = synth.normal_bf16_bits(16, (n, 1), (n, 4, 128))
    vb = synth.normal_bf16_bits(16, (n, 2), (n, 4, 128))
    q = synth.normal(16, (n, 3), (1, 32, 128)).astype(np.float64)
    sinks = synth.normal(16, (n, 4), 32)
    kc, vc, bt = _paged(Lf, kb, vb, 16)
    sl = np.array([n], np.int32)
    assert np.array_equal(oracle.attn_decode(Lf, q, kc, vc, bt, sl, sinks),
                          oracle.attn_decode(Ls, q, kc, vc, bt, sl, sinks))


@pytest.mark.parametrize("n", [514, 530, 1000])
def test_sliding_sees_exactly_last_513_keys(n):
    # t = n-1 >= 513: sliding equals full attention over keys t-512..t only
    Lf, Ls = oracle.layer(window=0), oracle.layer(window=513)
    kb = synth.normal_bf16_bits(17, (n, 1), (n, 4, 128))
    vb = synth.normal_bf16_bits(17, (n, 2), (n, 4, 128))
    q = synth.normal(17, (n, 3), (1, 32, 128)).astype(np.float64)
    sinks = synth.normal(17, (n, 4), 32)
    kc, vc, bt = _paged(Ls, kb, vb, 17)
    out_s = oracle.attn_decode(Ls, q, kc, vc, bt, np.array([n], np.int32), sinks)
    kc2, vc2, bt2 = _paged(Lf, kb[n - 513:], vb[n - 513:], 18)
    out_f = oracle.attn_decode(Lf, q, kc2, vc2, bt2, np.array([513], np.int32), sinks)
    assert np.allclose(out_s, out_f, rtol=0, atol=1e-15)
    kc3, vc3, bt3 = _paged(Lf, kb[n - 512:], vb[n - 512:], 19)
    out_short = oracle.attn_decode(Lf, q, kc3, vc3, bt3, np.array([512], np.int32), sinks)
    assert not np.allclose(out_s, out_short, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# split / merge (P5) and paging (P6)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_split_merge_equals_direct(splits):
    n = 300
    L = oracle.layer()
    kb = synth.normal_bf16_bits(20, (1,), (n, 4, 128))
    vb = synth.normal_bf16_bits(20, (2,), (n, 4, 128))
    q = synth.normal(20, (3,), (32, 128)).astype(np.float64)
    sinks = synth.normal(20, (4,), 32)
    kc, vc, bt = _paged(L, kb, vb, 20)
    ref = oracle.attn_decode(L, q[None], kc, vc, bt, np.array([n], np.int32), sinks)[0]
    edges = np.linspace(0, n, splits + 1).round().astype(int)
    edges = np.concatenate([[0, 0], edges])  # plus an empty range at the front
    for h in (0, 13, 31):
        parts = [oracle.attn_partial(L, q[h], h, kc, vc, bt, 0, edges[i], edges[i + 1])
                 for i in range(len(edges) - 1)]
        got = oracle.merge(np.stack([p[0] for p in parts]), np.array([p[1] for p in parts]),
                           sinks[h])
        assert np.allclose(got, ref[h], rtol=0, atol=1e-12)


def test_page_permutation_is_bit_identical():
    n = 200
    L = oracle.layer()
    kb = synth.normal_bf16_bits(21, (1,), (n, 4, 128))
    vb = synth.normal_bf16_bits(21, (2,), (n, 4, 128))
    q = synth.normal(21, (3,), (1, 32, 128)).astype(np.float64)
    sinks = synth.normal(21, (4,), 32)
    a = _paged(L, kb, vb, 21, perm=False)
    b = _paged(L, kb, vb, 22, perm=True)
    sl = np.array([n], np.int32)
    assert np.array_equal(oracle.attn_decode(L, q, *a, sl, sinks),
                          oracle.attn_decode(L, q, *b, sl, sinks))


def test_ring_aliasing_outside_window_is_bit_identical():
    # a 33-page ring for a sliding layer gives the same output as a full table
    n = 2000
    Ls = oracle.layer(window=513)
    kb = synth.normal_bf16_bits(23, (1,), (n, 4, 128))
    vb = synth.normal_bf16_bits(23, (2,), (n, 4, 128))
    q = synth.normal(23, (3,), (1, 32, 128)).astype(np.float64)
    sinks = synth.normal(23, (4,), 32)
    kc, vc, bt = _paged(Ls, kb, vb, 23)
    logical = -(-n // 16)
    rbt, nb = synth.ring_block_table(23, (5,), 1, logical, 33, logical + 1)
    rk = np.zeros((nb, 4, 16, 128), np.uint16)
    rv = np.zeros((nb, 4, 128, 16), np.uint16)
    for p in range(n):  # later tokens overwrite ring pages, as appends would
        pg = rbt[0, p // 16]
        rk[pg, :, p % 16] = kb[p]
        rv[pg, :, :, p % 16] = vb[p]
    rk = oracle.k_to_cache(Ls, rk)
    sl = np.array([n], np.int32)
    assert np.array_equal(oracle.attn_decode(Ls, q, kc, vc, bt, sl, sinks),
                          oracle.attn_decode(Ls, q, rk, rv, rbt, sl, sinks))


def test_window_spans_33_pages():
    # keys t-512..t always touch 33 pages of 16 once t >= 512
    for t in range(512, 512 + 64):
        assert (t // 16) - ((t - 512) // 16) + 1 == 33


# ---------------------------------------------------------------------------
# append (O4) and page walk (O8)
# ---------------------------------------------------------------------------

def test_append_places_rows_and_rounds_v_like_torch():
    L = oracle.layer(window=513, use_rope=1)
    T = 40
    nb = 8
    bt = synth.permutation(30, (1,), nb)[None, :]
    pos = np.arange(100, 100 + T, dtype=np.int32)
    slots = np.array([oracle.slot(bt, 0, p % (nb * 16)) for p in range(T)], np.int32)
    slots[5] = -1  # skipped token
    q = synth.normal(30, (2,), (T, 32, 128))
    k = synth.normal(30, (3,), (T, 4, 128))
    v = synth.normal(30, (4,), (T, 4, 128))
    ones = np.ones(128, np.float32)
    kc = np.full((nb, 4, 16, 128), 0xBEEF, np.uint16)
    vc = np.full((nb, 4, 128, 16), 0xBEEF, np.uint16)
    qo = oracle.append(L, q, k, v, ones, ones, pos, slots, kc, vc)
    kl = oracle.k_from_cache(L, kc)
    written = np.zeros((nb, 16), bool)
    for t in range(T):
        if slots[t] < 0:
            continue
        pg, r = divmod(int(slots[t]), 16)
        written[pg, r] = True
        assert np.array_equal(vc[pg, :, :, r], _torch_bf16_bits(v[t]))
        for g in range(4):
            kk = oracle.rope(oracle.rmsnorm(k[t, g], ones), pos[t])
            # the oracle rounds the fp64 value once; torch rounds its fp32 image
            ref = _torch_bf16_bits(kk.astype(np.float32)).astype(int)
            assert np.max(np.abs(kl[pg, g, r].astype(int) - ref)) <= 1
    untouched = ~written
    assert np.all(kl.transpose(0, 2, 1, 3)[untouched] == 0xBEEF)
    assert np.all(vc.transpose(0, 3, 1, 2)[untouched] == 0xBEEF)
    # q out: norm then rope; norms are preserved by the rotation
    for t in (0, 17):
        for h in (0, 31):
            qn = oracle.rmsnorm(q[t, h], ones)
            assert math.isclose(np.linalg.norm(qo[t, h]), np.linalg.norm(qn), rel_tol=1e-13)


def test_append_rejects_slot_out_of_range():
    L = oracle.layer()
    kc = np.zeros((2, 4, 16, 128), np.uint16)
    vc = np.zeros((2, 4, 128, 16), np.uint16)
    x = np.zeros((1, 4, 128), np.float32)
    with pytest.raises(ValueError):
        oracle.append(L, np.zeros((1, 32, 128), np.float32), x, x, np.ones(128), np.ones(128),
                      [0], [32], kc, vc)


def test_page_walk_reconstructs_sequence():
    # every logical token lands in a distinct slot, and reading pages in table
    # order returns the tokens in order
    n = 16 * 37 + 5
    bt, nb = synth.shuffled_block_table(31, (1,), 1, [-(-n // 16)], 40)
    slots = [oracle.slot(bt, 0, p) for p in range(n)]
    assert len(set(slots)) == n and min(slots) >= 0 and max(slots) < nb * 16
    flat = np.full(nb * 16, -1)
    flat[slots] = np.arange(n)
    seq = np.concatenate([flat[pg * 16:(pg + 1) * 16] for pg in bt[0, :-(-n // 16)]])
    assert np.array_equal(seq[:n], np.arange(n))


# ---------------------------------------------------------------------------
# prefill (O7)
# ---------------------------------------------------------------------------

def test_prefill_rows_equal_decode_at_same_position():
    L = oracle.layer(window=513)
    n = 700
    kb = synth.normal_bf16_bits(40, (1,), (n, 4, 128))
    vb = synth.normal_bf16_bits(40, (2,), (n, 4, 128))
    q = synth.normal(40, (3,), (n, 32, 128)).astype(np.float64)
    sinks = synth.normal(40, (4,), 32)
    kc, vc, bt = _paged(L, kb, vb, 40)
    start = 100  # chunk of rows 100..699 with 100 keys already cached
    out = oracle.attn_prefill(L, q[start:], np.array([0, n - start], np.int32), kc, vc, bt,
                              np.array([n], np.int32), sinks)
    for i in (0, 1, 412, 413, 599):
        t = start + i
        dec = oracle.attn_decode(L, q[t][None], kc, vc, bt, np.array([t + 1], np.int32), sinks)
        assert np.array_equal(out[i], dec[0])


def test_prefill_brute_force_small():
    L = _small_layer(window=3)
    n = 9
    kb = synth.normal_bf16_bits(41, (1,), (n, L.hkv, L.d))
    vb = synth.normal_bf16_bits(41, (2,), (n, L.hkv, L.d))
    q = synth.normal(41, (3,), (n, L.hq, L.d)).astype(np.float64)
    sinks = synth.normal(41, (4,), L.hq)
    kc, vc, bt = _paged(L, kb, vb, 41)
    out = oracle.attn_prefill(L, q, np.array([0, n], np.int32), kc, vc, bt,
                              np.array([n], np.int32), sinks)
    for i in range(n):
        assert np.max(np.abs(out[i] - _brute(L, q[i], kb, vb, i, sinks))) < 1e-15


# ---------------------------------------------------------------------------
# footprint (P8): the pages' own numbers
# ---------------------------------------------------------------------------

def test_full_layer_kv_is_28_kib_per_token():
    shape = json.load(open(os.path.join(GOLDEN, "flint_attention_shape.json")))
    assert oracle.full_kv_bytes_per_token(shape["full_layers"], shape["kv_heads"],
                                          shape["head_dim"], 2) == shape["kv_bytes_per_token"]
    assert shape["sliding_layers"] + shape["full_layers"] == shape["layers"]


def test_kv_calculator_table():
    tab = json.load(open(os.path.join(GOLDEN, "kv_cache_gib_per_request.json")))
    for row in tab["rows"]:
        for fmt, eb in (("bf16", 2), ("fp8", 1)):
            gib = oracle.kv_bytes_per_request(row["context"], elem_bytes=eb) / 2**30
            assert round(gib, 3) == pytest.approx(row[fmt], abs=1e-9), (row, fmt, gib)


# ---------------------------------------------------------------------------
# fp8 E4M3 KV cache (OCP 8-bit floating point: E4M3, bias 7, no infinities,
# S.1111.111 is NaN, largest finite 448)
# ---------------------------------------------------------------------------

def _torch_fp8_values(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _torch_fp8_codes(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_fp8_value_of_every_code_matches_torch():
    codes = np.arange(256)
    got, ref = oracle.fp8_value(codes), _torch_fp8_values(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    # and the format's landmarks, from its definition
    assert oracle.fp8_value(0x7E) == 448.0 and oracle.fp8_value(0x08) == 2.0**-6
    assert oracle.fp8_value(0x01) == 2.0**-9 and oracle.fp8_value(0x38) == 1.0
    assert oracle.fp8_value(0xC0) == -2.0


def test_fp8_rounding_matches_torch_below_overflow():
    # nearest with ties to even; inputs are fp32 so torch rounds the same real.
    # Below the overflow threshold torch and the saturating reading agree.
    mags = oracle.fp8_value(np.arange(0x7F))                 # 0 .. 448, increasing
    mids = (mags[:-1] + mags[1:]) / 2                         # every tie, exact in fp32
    nudged = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                             np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    rnd = synth.normal(40, (1,), 4000) * np.exp2(synth.rng(40, 2).random(4000) * 18 - 12)
    x = np.concatenate([mags, mids, nudged, rnd, [2.0**-11, 2.0**-10, 3 * 2.0**-10, 1e-30]])
    x = np.concatenate([x, -x]).astype(np.float32)
    x = x[np.abs(x) < 448]
    assert np.array_equal(oracle.fp8_rne(x.astype(np.float64)), _torch_fp8_codes(x))


def test_fp8_ties_go_to_even_code():
    # 1 + 1/16 lies halfway between 1 (code 0x38) and 1.125 (0x39): even wins;
    # 1 + 3/16 lies between 0x39 and 0x3A: again the even code
    assert oracle.fp8_rne([1.0625, 1.1875, -1.0625]).tolist() == [0x38, 0x3A, 0xB8]
    # subnormal tie: 2^-10 is halfway between 0 and 2^-9
    assert oracle.fp8_rne([2.0**-10, 3 * 2.0**-10]).tolist() == [0x00, 0x02]


def test_fp8_saturates_and_keeps_nan():
    big = [448.0, 449.0, 464.0, 480.0, 1e6, 1e300, np.inf]
    assert (oracle.fp8_rne(big) == 0x7E).all()
    assert (oracle.fp8_rne(np.negative(big)) == 0xFE).all()
    assert (oracle.fp8_rne([np.nan]) & 0x7F == 0x7F).all()


def _fp8_layer(**kw):
    return oracle.layer(kv_fp8=1, **kw)


def test_cache_tile_orders_follow_the_abi_header():
    # the layouts include/flint.h documents, written out here from that text:
    # bf16 K in blocks of 32 dims of 8-dim groups, V dim-major; fp8 in its
    # MFMA-native tile order.
    # Every (row, dim) of a tile lands on a distinct element of that tile.
    for fp8 in (0, 1):
        L = oracle.layer(kv_fp8=fp8, hkv=4)
        for page, g in ((0, 0), (5, 3)):
            tile = (page * 4 + g) * 2048
            ks, vs = set(), set()
            for r in range(16):
                ko, vo = oracle.k_offsets(L, page, g, r), oracle.v_offsets(L, page, g, r)
                for d in range(128):
                    if fp8:
                        k_ref = ((d >> 4) & 1) * 1024 + (d >> 5) * 256 + r * 16 + (d & 15)
                        v_ref = ((d >> 6) * 1024 + ((r >> 2) * 16 + (d & 15)) * 16
                                 + ((d >> 4) & 3) * 4 + (r & 3))
                    else:
                        k_ref = (d >> 5) * 512 + ((d >> 3) & 3) * 128 + r * 8 + (d & 7)
                        v_ref = d * 16 + r
                    assert ko[d] == tile + k_ref and vo[d] == tile + v_ref
                ks.update(ko.tolist())
                vs.update(vo.tolist())
            assert ks == vs == set(range(tile, tile + 2048))


def test_fp8_needs_the_flint_tile_shape():
    L = _fp8_layer(hq=4, hkv=2, d=8, bs=4)
    kc = np.zeros((2, 2, 4, 8), np.uint8)
    x = np.zeros((1, 2, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.append(L, np.zeros((1, 4, 8), np.float32), x, x, np.ones(8), np.ones(8), [0], [0],
                      kc, kc.copy())


def test_fp8_append_places_scaled_codes():
    # V codes are the rounding of v / v_scale (fp32 inputs: torch rounds the
    # same real when v_scale is a power of two); K codes are within one code of
    # torch's rounding of the fp32 image of the normed, rotated row / k_scale
    L = _fp8_layer(window=513, use_rope=1, k_scale=0.25, v_scale=2.0)
    T, nb = 24, 6
    bt = synth.permutation(41, (1,), nb)[None, :]
    pos = np.arange(7, 7 + T, dtype=np.int32)
    slots = np.array([oracle.slot(bt, 0, p) for p in pos], np.int32)
    slots[3] = -1
    q = synth.normal(41, (2,), (T, 32, 128))
    k = synth.normal(41, (3,), (T, 4, 128))
    v = synth.normal(41, (4,), (T, 4, 128)) * 50.0
    ones = np.ones(128, np.float32)
    kc = np.full((nb, 4, 16, 128), 0x5A, np.uint8)
    vc = np.full((nb, 4, 128, 16), 0x5A, np.uint8)
    oracle.append(L, q, k, v, ones, ones, pos, slots, kc, vc)
    kw = np.zeros(kc.size, bool)
    vw = np.zeros(vc.size, bool)
    for t in range(T):
        if slots[t] < 0:
            continue
        pg, r = divmod(int(slots[t]), 16)
        for g in range(4):
            kw[oracle.k_offsets(L, pg, g, r)] = True
            vw[oracle.v_offsets(L, pg, g, r)] = True
            assert np.array_equal(oracle.v_row(L, vc, pg, g, r),
                                  _torch_fp8_codes(v[t, g] / np.float32(2.0)))
            kk = oracle.rope(oracle.rmsnorm(k[t, g], ones), pos[t]) / 0.25
            ref = _torch_fp8_values(_torch_fp8_codes(kk.astype(np.float32)))
            got = oracle.fp8_value(oracle.k_row(L, kc, pg, g, r))
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0**-6))) - 3)
            assert np.all(np.abs(got - ref) <= ulp)
    assert kw.sum() == vw.sum() == (T - 1) * 4 * 128
    assert np.all(kc.reshape(-1)[~kw] == 0x5A) and np.all(vc.reshape(-1)[~vw] == 0x5A)
    # values beyond 448 * v_scale saturate instead of turning into NaN
    v2 = np.full((1, 4, 128), 2000.0, np.float32)
    oracle.append(L, q[:1], k[:1], v2, ones, ones, pos[:1], slots[:1], kc, vc)
    pg, r = divmod(int(slots[0]), 16)
    assert all((oracle.v_row(L, vc, pg, g, r) == 0x7E).all() for g in range(4))


def test_fp8_attention_is_bf16_attention_of_the_dequantised_cache():
    # attention over fp8 codes with scales equals attention over a bf16 cache
    # holding code value x scale (exact in bf16 for power-of-two scales),
    # which the brute-force pins above tie to the definition; one KV group of
    # the Flint tile shape (d = 128, 16-token pages), two pages
    for window in (0, 5):
        L8 = _fp8_layer(window=window, hq=8, hkv=1, k_scale=0.5, v_scale=4.0)
        L16 = oracle.layer(window=window, hq=8, hkv=1)
        n = 21
        kcode = synth.fp8_codes(42, (1, window), (n, 1, 128))          # |k| < 2
        vcode = synth.fp8_codes(42, (2, window), (n, 1, 128), 0x7E)    # all finite codes
        kb = _torch_bf16_bits(oracle.fp8_value(kcode) * 0.5)
        vb = _torch_bf16_bits(oracle.fp8_value(vcode) * 4.0)
        q = synth.normal(42, (3, window), (8, 128)).astype(np.float64) * 0.1
        sinks = synth.normal(42, (4, window), 8)
        kc16, vc16, bt = _paged(L16, kb, vb, seed=9)
        kc8 = np.zeros(kc16.shape, np.uint8)
        vc8 = np.zeros(vc16.shape, np.uint8)
        for p in range(n):
            pg, r = bt[0, p // 16], p % 16
            oracle.put_k_row(L8, kc8, pg, 0, r, kcode[p, 0])
            oracle.put_v_row(L8, vc8, pg, 0, r, vcode[p, 0])
        sl = np.array([n], np.int32)
        out8 = oracle.attn_decode(L8, q[None], kc8, vc8, bt, sl, sinks)[0]
        out16 = oracle.attn_decode(L16, q[None], kc16, vc16, bt, sl, sinks)[0]
        assert np.array_equal(out8, out16)
        ref = _brute(L16, q, kb, vb, n - 1, sinks)
        assert np.max(np.abs(out8 - ref)) < 1e-13 * max(1.0, np.abs(ref).max())


# ---------------------------------------------------------------------------
# MoE sublayer (O9 router + top-k, O10 experts): closed forms from rank-one
# weights whose products are exact, ties, invariants
# ---------------------------------------------------------------------------

def _bf16_exact(vals):
    """Values that bf16 holds exactly (3 significant bits), as (bits, values)."""
    v = np.asarray(vals, np.float64)
    b = _torch_bf16_bits(v.astype(np.float32))
    return b, synth.bf16_bits_to_f32(b).astype(np.float64)


def _rank_one_moe(M, seed):
    """Weights where every product is exact: router row e = c_e * e_0, gate /
    up row j of expert e = a_j^e * e_0 / b_j^e * e_0, down row r of expert e
    = c_r^e * v^e.  With x[0] = 1: z_e = c_e, g_j = a_j, u_j = b_j and
    E_e(x)_r = c_r^e * sum_j v_j^e silu(a_j^e) b_j^e."""
    rng = synth.rng(seed, 1)
    H, I, E, S = M.hidden, M.inter, M.experts, M.shared
    quant = lambda a: np.round(a * 8) / 8                    # multiples of 1/8, small: exact
    c_route = rng.permutation(E) / 8.0 - E / 16.0            # distinct router logits
    a = quant(rng.uniform(-2, 2, (E + S, I)))
    bu = quant(rng.uniform(-2, 2, (E + S, I)))
    c = quant(rng.uniform(-1, 1, (E + S, H)))
    v = quant(rng.uniform(-1, 1, (E + S, I)))
    wr = np.zeros((E, H), np.uint16)
    wr[:, 0] = _bf16_exact(c_route)[0]
    wgu = np.zeros((E + S, 2, I, H), np.uint16)
    wgu[:, 0, :, 0] = _bf16_exact(a)[0]
    wgu[:, 1, :, 0] = _bf16_exact(bu)[0]
    # c_r * v_j: a product of two multiples of 1/8 below 2, exact in bf16
    c32, v32 = c.astype(np.float32), v.astype(np.float32)
    wd = _torch_bf16_bits(np.einsum("er,ej->erj", c32, v32))
    x = synth.normal(seed, (2,), (1, H))   # coordinates 1.. meet zero weights
    x[0, 0] = 1.0
    silu = lambda g: g / (1.0 + np.exp(-g))
    expert = np.array([c[e] * float(np.sum(v[e] * silu(a[e]) * bu[e])) for e in range(E + S)])
    return wr, wgu, wd, x, c_route, expert


@pytest.mark.parametrize("shape", [dict(hidden=64, experts=16, top_k=3, inter=8, shared=1),
                                   dict(hidden=2048, experts=16, top_k=6, inter=512, shared=1),
                                   dict(hidden=64, experts=16, top_k=6, inter=8, shared=2)])
def test_moe_closed_form(shape):
    # catches a dropped term (shared expert, a routed slot), swapped gate/up,
    # a transposed down projection, unnormalised or wrongly paired weights
    M = oracle.moe(**shape)
    wr, wgu, wd, x, z, expert = _rank_one_moe(M, 50 + shape["top_k"])
    ids, w, y = oracle.moe_forward(M, x, wr, wgu, wd)
    top = np.argsort(-z, kind="stable")[:M.top_k]
    assert ids[0].tolist() == top.tolist()
    s = 1.0 / (1.0 + np.exp(-z[top]))
    assert np.allclose(w[0], s / s.sum(), rtol=0, atol=1e-15)
    ref = (s / s.sum()) @ expert[top] + expert[M.experts:].sum(axis=0)
    assert np.max(np.abs(y[0] - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())


def test_moe_route_ties_go_to_the_lower_index():
    M = oracle.moe(hidden=64, experts=16, top_k=6, inter=8, shared=1)
    wr = np.zeros((16, 64), np.uint16)
    wr[:, 0] = _bf16_exact(np.full(16, 0.5))[0]
    wr[[3, 11], 0] = _bf16_exact([0.75, 0.75])[0]
    x = np.zeros(64, np.float32)
    x[0] = 1.0
    ids, w = oracle.moe_route(M, x, wr)
    assert ids.tolist() == [3, 11, 0, 1, 2, 4]
    assert abs(w.sum() - 1.0) < 1e-15 and w[0] == w[1] and w[2] == w[5]


def test_moe_route_ranks_the_exact_logits_not_their_fp32_rounding():
    # experts 3 and 11 have logits 0.5 and 0.5 + 2^-30, equal once rounded to
    # fp32: the definition (the exact logit) picks 11 first, a rounded
    # comparison would pick 3 by the lower-index rule
    M = oracle.moe(hidden=64, experts=16, top_k=2, inter=8, shared=1)
    wr = np.zeros((16, 64), np.uint16)
    wr[:, 0] = _bf16_exact(np.full(16, 0.25))[0]
    wr[[3, 11], 0] = _bf16_exact([0.5, 0.5])[0]
    wr[11, 1] = _bf16_exact([2.0 ** -10])[0][0]
    x = np.zeros(64, np.float32)
    x[0] = 1.0
    x[1] = np.float32(2.0 ** -20)
    assert np.float32(0.5 + 2.0 ** -30) == np.float32(0.5)
    ids, _ = oracle.moe_route(M, x, wr)
    assert ids.tolist() == [11, 3]


def test_moe_route_matches_a_sort_of_the_logits():
    # random router: the selection is the stable descending order of the
    # exact (fp64) logits, computed here by numpy's matmul and argsort
    M = oracle.moe()
    wr = synth.normal_bf16_bits(51, (1,), (256, 2048))
    for t in range(4):
        x = synth.normal(51, (2, t), 2048) * np.float32(0.03)
        ids, w = oracle.moe_route(M, x, wr)
        z = synth.bf16_bits_to_f32(wr).astype(np.float64) @ x.astype(np.float64)
        top = np.argsort(-z, kind="stable")[:6]
        assert ids.tolist() == top.tolist()
        s = 1.0 / (1.0 + np.exp(-z[top]))
        assert np.allclose(w, s / s.sum(), rtol=1e-12, atol=0)
        assert len(set(ids.tolist())) == 6


def test_moe_is_linear_in_the_down_projection_and_the_shared_expert_adds():
    M = oracle.moe(hidden=64, experts=16, top_k=3, inter=16, shared=1)
    wr = synth.normal_bf16_bits(52, (1,), (16, 64))
    wgu = synth.normal_bf16_bits(52, (2,), oracle.gate_up_shape(M))
    wd = synth.normal_bf16_bits(52, (3,), oracle.down_shape(M))
    x = synth.normal(52, (4,), (3, 64)) * np.float32(0.2)
    _, _, y = oracle.moe_forward(M, x, wr, wgu, wd)
    # doubling every bf16 down weight (exact: exponent + 1) doubles y
    wd2 = (wd.astype(np.uint32) + (1 << 7)).astype(np.uint16)
    _, _, y2 = oracle.moe_forward(M, x, wr, wgu, wd2)
    assert np.max(np.abs(y2 - 2 * y)) <= 1e-12 * np.abs(y).max()
    # zero routed down projections: only the shared expert remains
    wd0 = wd.copy()
    wd0[:16] = 0
    _, _, y0 = oracle.moe_forward(M, x, wr, wgu, wd0)
    wd_s = np.zeros_like(wd)
    wd_s[16] = wd[16]
    _, _, ys = oracle.moe_forward(M, x, wr, wgu, wd_s)
    assert np.array_equal(y0, ys)
    assert np.abs(ys).max() > 0
