"""Shared builders for the GPU parity tests: seeded inputs (synth), the
oracle's expected values, and uploads for the HIP path.  Nothing here feeds a
GPU result back into the oracle."""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL = 4e-3          # max |GPU - oracle| on fp32 attention outputs (the contract)
# Regression guard beside the contract: the errors observed are ~1e-6 of the
# outputs' scale, while losing the bf16 remainder of q or of P (the hi/lo
# splits that carry the fp32 precision through the matrix cores) costs
# ~1e-3 -- which would still pass TOL.  Scaled by max(1, max|reference|) so
# that fp8 caches with large V keep the same relative bar.
GUARD = 1e-4
# Prefill's value product takes P in fp16: relative rounding at most 2^-11,
# so an output can move by up to 2^-11 of the largest |V| it averages.  Over
# the prefill tests the errors stay below 2e-4 of max(1, max|reference|);
# bf16 P (2^-8) would cost about 8 times more.  The prefill guard sits
# between the two.
PREFILL_GUARD = 5e-4
SENTINEL = 0x7FC1   # NaN bit pattern in every bf16 cache slot nobody wrote
SENTINEL8 = 0x7F    # the NaN code in every fp8 cache slot nobody wrote


def dev():
    import torch
    return torch.device("cuda:0")


def up(a):
    """numpy -> cuda tensor (uint16 arrays travel as int16 bits)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def down16(t):
    return t.cpu().numpy().view(np.uint16)


def layers(window, fp8=None, hkv=4, rope=None, theta=10000.0, scale=None, eps=1e-6):
    """(oracle layer, library layer) with hkv KV heads (8 query heads each);
    fp8 = (k_scale, v_scale) selects an fp8 E4M3 cache with those scales
    (fp32 values, passed to both sides).  RoPE is on for sliding layers
    unless `rope` says otherwise; theta, scale (default 1/sqrt(128)) and eps
    go to both sides, rounded to fp32 where the library takes fp32."""
    import full_gqa_decode_amd as fl
    rope = (1 if window else 0) if rope is None else int(rope)
    # the library receives eps and the softmax scale as fp32; the oracle uses
    # those same values
    eps = float(np.float32(eps))
    scale = float(np.float32(1.0 / np.sqrt(128) if scale is None else scale))
    common = dict(window=window, use_rope=rope)
    ks, vs, kvf = 1.0, 1.0, 0
    if fp8 is not None:
        ks, vs = (float(np.float32(x)) for x in fp8)
        kvf = 1
    Lo = oracle.layer(**common, eps=eps, hq=8 * hkv, hkv=hkv, theta=theta, scale=scale,
                      kv_fp8=kvf, k_scale=ks, v_scale=vs)
    Lf = fl.layer(**common, rms_eps=eps, num_q_heads=8 * hkv, num_kv_heads=hkv,
                  rope_theta=theta, softmax_scale=scale,
                  kv_dtype=fl.FLINT_KV_FP8_E4M3 if kvf else fl.FLINT_KV_BF16,
                  k_scale=ks, v_scale=vs)
    return Lo, Lf


def empty_caches(L, num_blocks, device=False):
    """K and V caches of num_blocks pages filled with the format's NaN
    sentinel, on the host (numpy) or the GPU (torch)."""
    fill = SENTINEL8 if L.kv_fp8 else SENTINEL
    shapes = (oracle.k_cache_shape(num_blocks, hkv=L.hkv), oracle.v_cache_shape(num_blocks, hkv=L.hkv))
    if not device:
        return tuple(np.full(sh, fill, oracle.cache_dtype(L)) for sh in shapes)
    import torch
    dt = torch.uint8 if L.kv_fp8 else torch.int16
    return tuple(torch.full(sh, fill, dtype=dt, device=dev()) for sh in shapes)


def down(t):
    """cache tensor -> numpy codes (uint16 bf16 bits or uint8 fp8 codes)."""
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


class DecodeCase:
    """B requests of context lengths `ctxs` with a shuffled (or ring) paged
    cache.  Raw q/k/v ~ N(0,1); every token a request still needs is appended
    (both sides); the new token of request b is at position ctxs[b]-1."""

    def __init__(self, seed, ctxs, window=0, ring=False, weights_one=True, extra_pages=3,
                 fp8=None, hkv=4, **layer_kw):
        self.seed, self.ctxs, self.window = seed, list(ctxs), window
        self.L, self.FL = layers(window, fp8, hkv, **layer_kw)
        self.hkv, self.hq = hkv, 8 * hkv
        B = len(ctxs)
        self.B = B
        tag = (hash((tuple(ctxs), window, ring)) & 0xFFFF,)
        maxctx = max(ctxs)
        logical = -(-maxctx // 16)
        self.bt_stride = logical + 1
        if ring:
            self.bt, nb = synth.ring_block_table(seed, tag + (synth.PERM,), B, logical, 33,
                                                 self.bt_stride)
        else:
            self.bt, nb = synth.shuffled_block_table(seed, tag + (synth.PERM,), B,
                                                     [-(-c // 16) for c in ctxs], self.bt_stride)
        self.num_blocks = nb + extra_pages
        self.qw = synth.norm_weight(seed, tag + (synth.QW,), 128, weights_one)
        self.kw = synth.norm_weight(seed, tag + (synth.KW,), 128, weights_one)
        self.sinks = synth.normal(seed, tag + (synth.SINK,), self.hq)
        # tokens to append: all of them, or (ring) only the pages the window can see
        toks, q_rows = [], []
        for b, c in enumerate(ctxs):
            first = 0
            if ring:
                first = max(0, ((c - 1) // 16 - 32) * 16)
            toks.append((b, first, c))
        self.toks = toks
        T = sum(c - f for _, f, c in toks)
        self.T = T
        self.q_in = np.zeros((T, self.hq, 128), np.float32)
        self.k_in = np.empty((T, hkv, 128), np.float32)
        self.v_in = np.empty((T, hkv, 128), np.float32)
        self.pos = np.empty(T, np.int32)
        self.slots = np.empty(T, np.int32)
        self.last_row = np.empty(B, np.int64)
        o = 0
        for b, f, c in toks:
            n = c - f
            self.k_in[o:o + n] = synth.normal(seed, tag + (synth.K, b), (n, hkv, 128))
            self.v_in[o:o + n] = synth.normal(seed, tag + (synth.V, b), (n, hkv, 128))
            self.q_in[o + n - 1] = synth.normal(seed, tag + (synth.Q, b), (self.hq, 128))
            self.pos[o:o + n] = np.arange(f, c)
            for p in range(f, c):
                self.slots[o + p - f] = oracle.slot(self.bt, b, p)
            self.last_row[b] = o + n - 1
            o += n
        self.seq_lens = np.array(ctxs, np.int32)

    def oracle_cache(self):
        """O4 for every token's K/V; q only for each request's new token.
        Returns (q_hat of the new tokens [B,32,128] fp64, K cache, V cache)."""
        kc, vc = empty_caches(self.L, self.num_blocks)
        oracle.append(self.L, self.q_in[:1], self.k_in, self.v_in, self.qw, self.kw, self.pos,
                      self.slots, kc, vc, want_q=False)
        r = self.last_row
        q = oracle.append(self.L, self.q_in[r], self.k_in[r], self.v_in[r], self.qw, self.kw,
                          self.pos[r], np.full(len(r), -1, np.int32), kc, vc)
        return q, kc, vc

    def expected(self):
        q, kc, vc = self.oracle_cache()
        out = oracle.attn_decode(self.L, q, kc, vc, self.bt, self.seq_lens, self.sinks)
        return out, q, kc, vc

    def run_gpu(self, pages_per_split=0, workspace=None):
        """append every token, then decode; returns (out, q_out, kc, vc) tensors."""
        import torch
        import full_gqa_decode_amd as fl
        kd, vd = empty_caches(self.L, self.num_blocks, device=True)
        qd = up(self.q_in)
        fl.flint_qk_norm_rope_append(self.FL, qd, up(self.k_in), up(self.v_in), up(self.qw),
                                     up(self.kw), up(self.pos), up(self.slots), qd, kd, vd)
        qdec = qd[torch.from_numpy(self.last_row).to(dev())].contiguous()
        out = torch.empty((self.B, self.hq, 128), dtype=torch.float32, device=dev())
        fl.flint_attn_decode(self.FL, qdec, kd, vd, up(self.bt), up(self.seq_lens),
                             max(self.ctxs), up(self.sinks), out, workspace=workspace,
                             pages_per_split=pages_per_split)
        torch.cuda.synchronize()
        return out, qd, kd, vd


    def run_gpu_fused(self, pages_per_split=0, slot_delta=None, noalloc=False):
        """append every token except each request's new one, then the fused
        step (append of the new token + decode in one launch); noalloc: through
        flint_attn_decode_step_noalloc (the library's static scratch)."""
        import torch
        import full_gqa_decode_amd as fl
        kd, vd = empty_caches(self.L, self.num_blocks, device=True)
        keep = np.ones(self.T, bool)
        keep[self.last_row] = False
        pre = np.nonzero(keep)[0]
        if len(pre):
            qs = torch.empty((len(pre), self.hq, 128), dtype=torch.float32, device=dev())
            fl.flint_qk_norm_rope_append(self.FL, up(self.q_in[pre]), up(self.k_in[pre]),
                                         up(self.v_in[pre]), up(self.qw), up(self.kw),
                                         up(self.pos[pre]), up(self.slots[pre]), qs, kd, vd)
        r = self.last_row
        slots = self.slots[r].copy()
        if slot_delta is not None:
            slots = slots + np.asarray(slot_delta, np.int32)
        out = torch.empty((self.B, self.hq, 128), dtype=torch.float32, device=dev())
        qo = torch.empty((self.B, self.hq, 128), dtype=torch.float32, device=dev())
        step = fl.flint_attn_decode_step_noalloc if noalloc else fl.flint_attn_decode_step
        step(self.FL, up(self.q_in[r]), up(self.k_in[r]), up(self.v_in[r]), up(self.qw),
             up(self.kw), up(slots), kd, vd, up(self.bt), up(self.seq_lens), max(self.ctxs),
             up(self.sinks), out, q_out=qo, pages_per_split=pages_per_split)
        torch.cuda.synchronize()
        return out, qo, kd, vd


class CacheDecodeCase:
    """Decode only: the cache and the fp32 q are drawn directly (no append),
    so K2/K3 are tested on their own.  fp8 = (k_scale, v_scale): an fp8 cache
    of random codes (K magnitudes below 2, V below 30, before scaling)."""

    def __init__(self, seed, ctxs, window=0, ring=False, q_scale=1.0, fp8=None, hkv=4):
        self.L, self.FL = layers(window, fp8, hkv)
        self.hkv, self.hq = hkv, 8 * hkv
        self.ctxs = list(ctxs)
        B = len(ctxs)
        self.B = B
        tag = (hash((tuple(ctxs), window, ring, 7)) & 0xFFFF,)
        logical = -(-max(ctxs) // 16)
        self.bt_stride = logical + 2
        if ring:
            self.bt, nb = synth.ring_block_table(seed, tag + (synth.PERM,), B, logical, 33,
                                                 self.bt_stride)
        else:
            self.bt, nb = synth.shuffled_block_table(seed, tag + (synth.PERM,), B,
                                                     [-(-c // 16) for c in ctxs], self.bt_stride)
        self.num_blocks = nb
        if fp8 is None:
            self.kc = synth.normal_bf16_bits(seed, tag + (synth.KC,),
                                             oracle.k_cache_shape(nb, hkv=hkv))
            self.vc = synth.normal_bf16_bits(seed, tag + (synth.VC,),
                                             oracle.v_cache_shape(nb, hkv=hkv))
        else:
            self.kc = synth.fp8_codes(seed, tag + (synth.KC,), oracle.k_cache_shape(nb, hkv=hkv),
                                      0x3F)
            self.vc = synth.fp8_codes(seed, tag + (synth.VC,), oracle.v_cache_shape(nb, hkv=hkv),
                                      0x5F)
        self.q = synth.normal(seed, tag + (synth.Q,), (B, self.hq, 128)) * np.float32(q_scale)
        self.sinks = synth.normal(seed, tag + (synth.SINK,), self.hq)
        self.seq_lens = np.array(ctxs, np.int32)

    def expected(self):
        return oracle.attn_decode(self.L, self.q.astype(np.float64), self.kc, self.vc, self.bt,
                                  self.seq_lens, self.sinks)

    def run_gpu(self, pages_per_split=0, sinks=None, seq_lens=None, bt=None, max_seq_len=None):
        import torch
        import full_gqa_decode_amd as fl
        out = torch.empty((self.B, self.hq, 128), dtype=torch.float32, device=dev())
        fl.flint_attn_decode(self.FL, up(self.q), up(self.kc), up(self.vc),
                             up(self.bt if bt is None else bt),
                             up(self.seq_lens if seq_lens is None else seq_lens),
                             max(self.ctxs) if max_seq_len is None else max_seq_len,
                             up(self.sinks if sinks is None else sinks), out,
                             pages_per_split=pages_per_split)
        torch.cuda.synchronize()
        return out.cpu().numpy()


def max_err(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)))


def guard_bar(ref, guard=GUARD):
    """The regression bar for outputs whose reference is `ref`."""
    r = np.asarray(ref, np.float64)
    finite = r[np.isfinite(r)]
    return guard * max(1.0, float(np.abs(finite).max()) if finite.size else 1.0)


def check_err(err, ref, what="", guard=GUARD):
    """err (max |GPU - oracle|) within the 4e-3 contract and the guard."""
    assert err <= TOL, f"{what} max err {err:.3e} above the {TOL} contract"
    bar = guard_bar(ref, guard)
    assert err <= bar, f"{what} max err {err:.3e} above the regression guard {bar:.1e}"
    return err


def assert_parity(got, ref, what="", guard=GUARD):
    """max |got - ref| within the contract and the regression guard."""
    return check_err(max_err(got, ref), ref, what, guard)


def bf16_ulp_diff(a, b):
    """|a - b| in bf16 ulps for two uint16 arrays of finite values."""
    def key(x):
        x = x.astype(np.int64)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(key(a) - key(b))
