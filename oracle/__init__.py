"""fp64 CPU oracle for Flint's decode-attention hot path (ctypes wrapper).

TEST INFRASTRUCTURE: only the tests, `__graft_entry__.smoke()` and the bench's
cpu_baseline leg may import this package.  It shares no code with the HIP
library in `full_gqa_decode_amd/`, and the HIP library never imports it.

The arithmetic lives in `oracle.c` (plain C, double precision); this module
only builds it with gcc and marshals numpy arrays.  The definitions it follows
are cited in `oracle.h`.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "liboracle.so")
# the same sources built with AddressSanitizer and UndefinedBehaviorSanitizer
# (build(sanitize=True)); a process loads it with gcc's libasan preloaded
SO_SANITIZED = os.path.join(HERE, "liboracle_san.so")
SRC = os.path.join(HERE, "oracle.c")
SRCS = [SRC, os.path.join(HERE, "moe.c")]
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP for the
    independent per-(query, head) work items); sanitize=True builds
    liboracle_san.so with ASan and UBSan instead."""
    so = SO_SANITIZED if sanitize else SO
    if not force and os.path.exists(so) and all(os.path.getmtime(so) >= os.path.getmtime(f)
                                                 for f in SRCS):
        return so
    tmp = so + ".tmp"
    extra = SANITIZE_FLAGS if sanitize else []
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                           "-Wall", "-Werror", *extra, "-o", tmp, *SRCS, "-lm"], cwd=HERE)
    os.replace(tmp, so)
    return so


class Layer(C.Structure):
    _fields_ = [("hq", C.c_int), ("hkv", C.c_int), ("d", C.c_int), ("bs", C.c_int),
                ("window", C.c_int), ("use_rope", C.c_int), ("theta", C.c_double),
                ("eps", C.c_double), ("scale", C.c_double), ("kv_fp8", C.c_int),
                ("k_scale", C.c_double), ("v_scale", C.c_double)]


def layer(window: int = 0, use_rope: int = 0, hq: int = 32, hkv: int = 4, d: int = 128,
          bs: int = 16, theta: float = 10000.0, eps: float = 1e-6, scale: float | None = None,
          kv_fp8: int = 0, k_scale: float = 1.0, v_scale: float = 1.0):
    """kv_fp8 = 1: the caches hold fp8 E4M3 codes (uint8) of K / k_scale and
    V / v_scale; otherwise bf16 codes (uint16)."""
    return Layer(hq, hkv, d, bs, window, use_rope, theta, eps,
                 (1.0 / np.sqrt(d)) if scale is None else scale, kv_fp8, k_scale, v_scale)


def cache_dtype(L: Layer):
    return np.uint8 if L.kv_fp8 else np.uint16


def _cache(L: Layer, a):
    assert a.dtype == cache_dtype(L) and a.flags.c_contiguous, "cache dtype/layout"
    return a


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            build()
        L = C.CDLL(SO)
        P = C.c_void_p
        L.orc_bf16_rne.restype = C.c_uint16
        L.orc_bf16_rne.argtypes = [C.c_float]
        L.orc_bf16_value.restype = C.c_double
        L.orc_bf16_value.argtypes = [C.c_uint16]
        L.orc_bf16_rne_array.argtypes = [P, P, C.c_int64]
        for name in ("orc_k_offset", "orc_v_offset"):
            f = getattr(L, name)
            f.restype = C.c_int64
            f.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_int, C.c_int]
        L.orc_fp8_rne.restype = C.c_uint8
        L.orc_fp8_rne.argtypes = [C.c_double]
        L.orc_fp8_value.restype = C.c_double
        L.orc_fp8_value.argtypes = [C.c_uint8]
        L.orc_rmsnorm.argtypes = [P, P, C.c_int, C.c_double, P]
        L.orc_rope.argtypes = [P, C.c_int, C.c_double, C.c_double]
        L.orc_slot.restype = C.c_int64
        L.orc_slot.argtypes = [P, C.c_int, C.c_int, C.c_int, C.c_int]
        L.orc_append.argtypes = [C.POINTER(Layer), C.c_int, P, P, P, P, P, P, P, P, P, P, C.c_int]
        L.orc_attn_decode.argtypes = [C.POINTER(Layer), C.c_int, P, P, P, C.c_int, P, C.c_int,
                                      P, P, P, C.c_int]
        L.orc_attn_partial.argtypes = [C.POINTER(Layer), P, C.c_int, P, P, P, C.c_int, C.c_int,
                                       C.c_int, C.c_int, P, P]
        L.orc_merge.argtypes = [C.c_int, C.c_int, P, P, C.c_double, P]
        L.orc_attn_prefill.argtypes = [C.POINTER(Layer), C.c_int, P, P, P, P, C.c_int, P, C.c_int,
                                       P, P, P, P, C.c_int, C.c_int]
        L.orc_full_kv_bytes_per_token.restype = C.c_int64
        L.orc_full_kv_bytes_per_token.argtypes = [C.c_int] * 4
        L.orc_kv_bytes_per_request.restype = C.c_int64
        L.orc_kv_bytes_per_request.argtypes = [C.c_int64, C.c_int, C.c_int, C.c_int, C.c_int,
                                               C.c_int, C.c_int]
        L.orc_default_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# --- O1 -------------------------------------------------------------------
def bf16_rne(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32).ravel()
    f = lib().orc_bf16_rne
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def bf16_rne_f64(x) -> np.ndarray:
    """Round fp64 values to bf16 bits (once, no fp32 step); keeps the shape."""
    x = _c(x, np.float64)
    y = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_rne_array(_p(x), _p(y), x.size)
    return y


def bf16_value(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16).ravel()
    f = lib().orc_bf16_value
    return np.array([f(int(b)) for b in bits], dtype=np.float64)


# --- O2 / O3 ----------------------------------------------------------------
def rmsnorm(x, w, eps=1e-6) -> np.ndarray:
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    y = np.empty(x.shape[-1], dtype=np.float64)
    lib().orc_rmsnorm(_p(x), _p(w), x.shape[-1], eps, _p(y))
    return y


def rope(x, pos, theta=10000.0) -> np.ndarray:
    y = _c(x, np.float64).copy()
    lib().orc_rope(_p(y), y.shape[-1], float(pos), float(theta))
    return y


# --- O4 ----------------------------------------------------------------------
def append(L: Layer, q_in, k_in, v_in, qw, kw, positions, slots, k_cache, v_cache,
           want_q=True):
    """Apply O4 for T tokens; the caches (uint16 bf16 codes, or uint8 fp8 codes
    for an fp8 layer) are updated in place.
    Returns q_out [T, hq, d] fp64 (or None)."""
    q_in = _c(q_in, np.float32)
    k_in = _c(k_in, np.float32)
    v_in = _c(v_in, np.float32)
    T = k_in.shape[0]
    positions = _c(positions, np.int32)
    slots = _c(slots, np.int32)
    _cache(L, k_cache)
    _cache(L, v_cache)
    num_blocks = k_cache.size // (L.hkv * L.bs * L.d)
    q_out = np.empty((T, L.hq, L.d), dtype=np.float64) if want_q else None
    rc = lib().orc_append(C.byref(L), T, _p(q_in), _p(k_in), _p(v_in), _p(_c(qw, np.float32)),
                          _p(_c(kw, np.float32)), _p(positions), _p(slots), _p(q_out),
                          _p(k_cache), _p(v_cache), num_blocks)
    if rc == -2:
        raise ValueError("oracle append: an fp8 cache needs d = 128 and bs = 16")
    if rc != 0:
        raise ValueError("oracle append: slot out of range")
    return q_out


# --- O5 ----------------------------------------------------------------------
def attn_decode(L: Layer, q, k_cache, v_cache, block_tables, seq_lens, sinks, nthreads=0):
    q = _c(q, np.float64)
    B = q.shape[0]
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    sk = _c(sinks, np.float32)
    num_blocks = k_cache.size // (L.hkv * L.bs * L.d)
    out = np.empty((B, L.hq, L.d), dtype=np.float64)
    rc = lib().orc_attn_decode(C.byref(L), B, _p(q), _p(_cache(L, k_cache)),
                               _p(_cache(L, v_cache)), num_blocks,
                               _p(bt), bt.shape[1], _p(sl), _p(sk), _p(out), int(nthreads))
    if rc == -2:
        raise ValueError("oracle decode: an fp8 cache needs d = 128 and bs = 16")
    if rc != 0:
        raise ValueError("oracle decode: bad page id or seq_len")
    return out


# --- O6 ----------------------------------------------------------------------
def attn_partial(L: Layer, q_h, h, k_cache, v_cache, block_tables, b, j0, j1):
    q_h = _c(q_h, np.float64)
    bt = _c(block_tables, np.int32)
    ot = np.empty(L.d, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    lib().orc_attn_partial(C.byref(L), _p(q_h), int(h), _p(_cache(L, k_cache)),
                           _p(_cache(L, v_cache)), _p(bt),
                           bt.shape[1], int(b), int(j0), int(j1), _p(ot), _p(lse))
    return ot, float(lse[0])


def merge(o_tildes, lses, sink):
    ot = _c(o_tildes, np.float64)
    ls = _c(lses, np.float64)
    out = np.empty(ot.shape[-1], dtype=np.float64)
    lib().orc_merge(ot.shape[0], ot.shape[-1], _p(ot), _p(ls), float(sink), _p(out))
    return out


# --- O7 ----------------------------------------------------------------------
def attn_prefill(L: Layer, q, cu_q_lens, k_cache, v_cache, block_tables, seq_lens, sinks,
                 rows=None, nthreads=0):
    """q [total_q, hq, d] (fp64 values); returns out [total_q, hq, d] (rows not
    requested are NaN)."""
    q = _c(q, np.float64)
    cu = _c(cu_q_lens, np.int32)
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    sk = _c(sinks, np.float32)
    B = cu.shape[0] - 1
    num_blocks = k_cache.size // (L.hkv * L.bs * L.d)
    out = np.full(q.shape, np.nan, dtype=np.float64)
    r = None if rows is None else _c(rows, np.int32)
    rc = lib().orc_attn_prefill(C.byref(L), B, _p(q), _p(cu), _p(_cache(L, k_cache)),
                                _p(_cache(L, v_cache)),
                                num_blocks, _p(bt), bt.shape[1], _p(sl), _p(sk), _p(out), _p(r),
                                0 if r is None else r.shape[0], int(nthreads))
    if rc == -2:
        raise ValueError("oracle prefill: an fp8 cache needs d = 128 and bs = 16")
    if rc != 0:
        raise ValueError("oracle prefill: bad row, page id or seq_len")
    return out


# --- cache layout ----------------------------------------------------------------
def k_offsets(L: Layer, page, g, row) -> np.ndarray:
    """Element offsets, in dim order, of one K row in its cache array."""
    f = lib().orc_k_offset
    return np.array([f(C.byref(L), int(page), int(g), int(row), i) for i in range(L.d)], np.int64)


def v_offsets(L: Layer, page, g, row) -> np.ndarray:
    """Element offsets, in dim order, of one token's V values in its cache array."""
    f = lib().orc_v_offset
    return np.array([f(C.byref(L), int(page), int(g), int(row), i) for i in range(L.d)], np.int64)


def _tile_patterns(L: Layer):
    """Offsets of (row, dim) inside one (page, KV head) tile, for K and V."""
    fk, fv = lib().orc_k_offset, lib().orc_v_offset
    k = np.array([[fk(C.byref(L), 0, 0, r, d) for d in range(L.d)] for r in range(L.bs)], np.int64)
    v = np.array([[fv(C.byref(L), 0, 0, r, d) for d in range(L.d)] for r in range(L.bs)], np.int64)
    return k, v


def k_to_cache(L: Layer, rows) -> np.ndarray:
    """K rows in logical order [pages, hkv, bs, d] -> the cache array (same
    shape and dtype) in the layout the library and the oracle read."""
    rows = np.ascontiguousarray(rows)
    kp, _ = _tile_patterns(L)
    n = rows.shape[0] * rows.shape[1]
    out = np.empty((n, L.bs * L.d), rows.dtype)
    out[:, kp.reshape(-1)] = rows.reshape(n, L.bs * L.d)
    return out.reshape(rows.shape)


def k_from_cache(L: Layer, cache) -> np.ndarray:
    """The cache array -> K rows in logical order [pages, hkv, bs, d]."""
    cache = np.asarray(cache)
    kp, _ = _tile_patterns(L)
    n = cache.size // (L.bs * L.d)
    flat = cache.reshape(n, L.bs * L.d)
    nb = cache.size // (L.hkv * L.bs * L.d)
    return flat[:, kp.reshape(-1)].reshape(nb, L.hkv, L.bs, L.d)


def k_row(L: Layer, cache, page, g, row) -> np.ndarray:
    return np.asarray(cache).reshape(-1)[k_offsets(L, page, g, row)]


def v_row(L: Layer, cache, page, g, row) -> np.ndarray:
    return np.asarray(cache).reshape(-1)[v_offsets(L, page, g, row)]


def put_k_row(L: Layer, cache, page, g, row, values) -> None:
    cache.reshape(-1)[k_offsets(L, page, g, row)] = values


def put_v_row(L: Layer, cache, page, g, row, values) -> None:
    cache.reshape(-1)[v_offsets(L, page, g, row)] = values


# --- fp8 E4M3 ------------------------------------------------------------------
def fp8_rne(x) -> np.ndarray:
    """fp8 E4M3 codes of reals (nearest, ties to even, saturating at 448)."""
    x = np.asarray(x, dtype=np.float64)
    f = lib().orc_fp8_rne
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def fp8_value(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    f = lib().orc_fp8_value
    return np.array([f(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


# --- O9 / O10: MoE sublayer -------------------------------------------------------
class Moe(C.Structure):
    _fields_ = [("hidden", C.c_int), ("experts", C.c_int), ("top_k", C.c_int),
                ("inter", C.c_int), ("shared", C.c_int)]


def moe(hidden: int = 2048, experts: int = 256, top_k: int = 6, inter: int = 512,
        shared: int = 1) -> Moe:
    return Moe(hidden, experts, top_k, inter, shared)


def gate_up_shape(M: Moe):
    return (M.experts + M.shared, 2, M.inter, M.hidden)


def down_shape(M: Moe):
    return (M.experts + M.shared, M.hidden, M.inter)


def moe_route(M: Moe, x, w_router):
    """One token: (ids [top_k] int32, weights [top_k] fp64)."""
    x = _c(x, np.float32)
    ids = np.empty(M.top_k, np.int32)
    w = np.empty(M.top_k, np.float64)
    if lib().orc_moe_route(C.byref(M), _p(x), _p(_c(w_router, np.uint16)), _p(ids), _p(w)) != 0:
        raise ValueError("oracle moe_route: bad top_k")
    return ids, w


def moe_forward(M: Moe, x, w_router, w_gate_up, w_down, nthreads=0):
    """x [T, hidden] fp32 -> (ids [T, top_k], weights [T, top_k], y [T, hidden] fp64)."""
    x = _c(x, np.float32)
    T = x.shape[0]
    ids = np.empty((T, M.top_k), np.int32)
    w = np.empty((T, M.top_k), np.float64)
    y = np.empty((T, M.hidden), np.float64)
    rc = lib().orc_moe_forward(C.byref(M), T, _p(x), _p(_c(w_router, np.uint16)),
                               _p(_c(w_gate_up, np.uint16)), _p(_c(w_down, np.uint16)), _p(ids),
                               _p(w), _p(y), int(nthreads))
    if rc != 0:
        raise ValueError("oracle moe_forward: bad top_k")
    return ids, w, y


# --- O8 / footprint -----------------------------------------------------------
def slot(block_tables, b, pos, bs=16) -> int:
    bt = _c(block_tables, np.int32)
    return int(lib().orc_slot(_p(bt), bt.shape[1], bs, int(b), int(pos)))


def full_kv_bytes_per_token(full_layers=14, hkv=4, d=128, elem_bytes=2) -> int:
    return int(lib().orc_full_kv_bytes_per_token(full_layers, hkv, d, elem_bytes))


def kv_bytes_per_request(ctx, full_layers=14, sliding_layers=35, window=513, hkv=4, d=128,
                         elem_bytes=2) -> int:
    return int(lib().orc_kv_bytes_per_request(int(ctx), full_layers, sliding_layers, window,
                                              hkv, d, elem_bytes))


def default_threads() -> int:
    return int(lib().orc_default_threads())


# --- helpers for tests: the oracle's own view of a paged cache ----------------
def k_cache_shape(num_blocks, hkv=4, bs=16, d=128):
    """K pages: [page][kv_head][row][dim]."""
    return (num_blocks, hkv, bs, d)


def v_cache_shape(num_blocks, hkv=4, bs=16, d=128):
    """V pages: [page][kv_head][dim][row] (dim-major)."""
    return (num_blocks, hkv, d, bs)


def depage(k_cache, v_cache, block_tables, b, n_tokens, bs=16):
    """Gather tokens 0..n_tokens-1 of request b into dense [n_tokens, hkv, d]
    K and V arrays (uses the oracle's own slot function)."""
    hkv, d = k_cache.shape[1], k_cache.shape[3]
    k = np.empty((n_tokens, hkv, d), dtype=k_cache.dtype)
    v = np.empty((n_tokens, hkv, d), dtype=v_cache.dtype)
    for p in range(n_tokens):
        s = slot(block_tables, b, p, bs)
        k[p] = k_cache[s // bs, :, s % bs, :]
        v[p] = v_cache[s // bs, :, :, s % bs]
    return k, v
