"""Python binding of libflint, the MI355X decode-attention library for Flint.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libflint.so.  PyTorch supplies device memory (tensor data
pointers) and the stream (the current HIP stream).  If the library has not
been built this module raises on first use; there is no fallback.

Functions carry the C names of include/flint.h:
    flint_qk_norm_rope_append, flint_attn_decode, flint_attn_prefill,
    flint_attn_decode_step (append + decode fused into one launch),
    flint_attn_decode_partials, flint_attn_merge, flint_moe_forward,
plus the size / plan queries.  bf16 tensors (K/V caches, prefill q) may be
torch.bfloat16, torch.int16 or torch.uint16, and fp8 caches torch.uint8 or
torch.float8_e4m3fn: only their bits are used.
"""
from __future__ import annotations

import ctypes as C
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflint.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "flint.h")

FLINT_OK = 0
STATUS_NAMES = {0: "FLINT_OK", 1: "FLINT_ERR_INVALID_ARGUMENT", 2: "FLINT_ERR_UNSUPPORTED",
                3: "FLINT_ERR_WORKSPACE_TOO_SMALL", 4: "FLINT_ERR_HIP"}


class FlintError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class FlintAttnLayer(C.Structure):
    _fields_ = [("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("block_size", C.c_int32), ("window", C.c_int32),
                ("use_rope", C.c_int32), ("rope_theta", C.c_float), ("rms_eps", C.c_float),
                ("softmax_scale", C.c_float), ("kv_dtype", C.c_int32), ("k_scale", C.c_float),
                ("v_scale", C.c_float)]


FLINT_KV_BF16 = 0
FLINT_KV_FP8_E4M3 = 1


def layer(window: int = 0, use_rope: int = 0, num_q_heads: int = 32, num_kv_heads: int = 4,
          head_dim: int = 128, block_size: int = 16, rope_theta: float = 10000.0,
          rms_eps: float = 1e-6, softmax_scale: float | None = None,
          kv_dtype: int = FLINT_KV_BF16, k_scale: float = 1.0,
          v_scale: float = 1.0) -> FlintAttnLayer:
    """kv_dtype FLINT_KV_FP8_E4M3: the caches hold fp8 codes of K / k_scale and
    V / v_scale (uint8 or torch.float8_e4m3fn tensors)."""
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale
    return FlintAttnLayer(num_q_heads, num_kv_heads, head_dim, block_size, window, use_rope,
                          rope_theta, rms_eps, scale, kv_dtype, k_scale, v_scale)


def full_layer(**kw) -> FlintAttnLayer:
    """One of Flint's 14 full-context layers: no positional encoding."""
    return layer(window=0, use_rope=0, **kw)


def sliding_layer(**kw) -> FlintAttnLayer:
    """One of Flint's 35 sliding layers: 513-key window with RoPE."""
    return layer(window=513, use_rope=1, **kw)


class FlintMoeLayer(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("num_experts", C.c_int32), ("top_k", C.c_int32),
                ("inter", C.c_int32), ("num_shared", C.c_int32)]


def moe_layer(hidden: int = 2048, num_experts: int = 256, top_k: int = 6, inter: int = 512,
              num_shared: int = 1) -> FlintMoeLayer:
    """Flint's MoE sublayer: 256 routed experts, top 6, one shared expert,
    hidden 2048; the expert FFN width 512 is a reading (the pages give none)."""
    return FlintMoeLayer(hidden, num_experts, top_k, inter, num_shared)


_lib = None
_P = C.c_void_p
_I = C.c_int32
_SZ = C.c_size_t
_LP = C.POINTER(FlintAttnLayer)
_MP = C.POINTER(FlintMoeLayer)

# (name, restype, argtypes) of every symbol include/flint.h declares
SIGNATURES = [
    ("flint_qk_norm_rope_append", C.c_int,
     [_LP, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P]),
    ("flint_attn_decode_workspace_size", _SZ, [_LP, _I, _I]),
    ("flint_attn_decode", C.c_int, [_LP, _I, _P, _P, _P, _I, _P, _I, _P, _I, _P, _P, _P, _SZ, _P]),
    ("flint_attn_decode_workspace_size_ex", _SZ, [_LP, _I, _I, _I]),
    ("flint_attn_decode_ex", C.c_int,
     [_LP, _I, _P, _P, _P, _I, _P, _I, _P, _I, _P, _P, _P, _SZ, _I, _P]),
    ("flint_attn_decode_step", C.c_int,
     [_LP, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _P, _P, _P, _SZ, _I, _P]),
    ("flint_attn_decode_step_noalloc", C.c_int,
     [_LP, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P]),
    ("flint_attn_decode_plan", C.c_int, [_LP, _I, _I, _I, C.POINTER(_I), C.POINTER(_I)]),
    ("flint_attn_decode_partials", C.c_int,
     [_LP, _I, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _P, _P, _P]),
    ("flint_attn_merge", C.c_int, [_LP, _I, _I, _P, _P, _P, _P, _P]),
    ("flint_attn_prefill_workspace_size", _SZ, [_LP, _I, _I, _I]),
    ("flint_attn_prefill", C.c_int,
     [_LP, _I, _P, _P, _I, _I, _P, _P, _I, _P, _I, _P, _I, _P, _P, _P, _SZ, _P]),
    ("flint_moe_workspace_size", _SZ, [_MP, _I]),
    ("flint_moe_forward", C.c_int, [_MP, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("flint_status_string", C.c_char_p, [C.c_int]),
    ("flint_last_error", C.c_char_p, []),
    ("flint_abi_version", _I, []),
]


def lib() -> C.CDLL:
    """Load libflint.so (built by `python -m full_gqa_decode_amd.build`)."""
    global _lib
    if _lib is None:
        # torch ships its own copy of the HIP runtime under the same soname as
        # ROCm's.  Loaded first, it is the copy libflint.so binds to, so one
        # runtime owns the device memory, the streams and our launches;
        # loading libflint.so first would bring in a second runtime, which
        # torch's memory and streams do not belong to.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with `python -m full_gqa_decode_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != FLINT_OK:
        raise FlintError(status, lib().flint_last_error().decode())


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t, dtypes, name, cuda=True):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if cuda and not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _sizes(L, B=None, **tensors):
    """Element counts the kernels assume, checked before any pointer crosses
    the C ABI (which sees no sizes).  Each keyword is a tensor (or None) and
    the count it must hold; block tables need at least B rows."""
    for name, (t, n) in tensors.items():
        if t is None:
            continue
        if name == "block_tables":
            if t.dim() != 2 or (B is not None and t.shape[0] < B):
                raise ValueError(f"block_tables must be 2-D with at least {B} rows, "
                                 f"got shape {tuple(t.shape)}")
            continue
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, expected {n}")


def _cache_elems(L, k_cache):
    return k_cache.shape[0] * L.num_kv_heads * L.block_size * L.head_dim


def _f32():
    return (_torch().float32,)


def _i32():
    return (_torch().int32,)


def _b16():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _kv(L):
    """Accepted cache tensor dtypes for the layer's KV element format."""
    torch = _torch()
    if L.kv_dtype == FLINT_KV_FP8_E4M3:
        return (torch.uint8, torch.float8_e4m3fn)
    return _b16()


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def flint_qk_norm_rope_append(L: FlintAttnLayer, q_in, k_in, v_in, q_norm_w, k_norm_w,
                              positions, slot_mapping, q_out, k_cache, v_cache, stream=None):
    """Fused per-head RMSNorm + RoPE + paged append of num_tokens tokens.
    q_out is float32 (decode) or a bf16-bits tensor (prefill); it may be q_in."""
    torch = _torch()
    T = k_in.shape[0]
    num_blocks = k_cache.shape[0]
    Hq, Hkv, D = L.num_q_heads, L.num_kv_heads, L.head_dim
    _sizes(L, q_in=(q_in, T * Hq * D), k_in=(k_in, T * Hkv * D), v_in=(v_in, T * Hkv * D),
           q_norm_w=(q_norm_w, D), k_norm_w=(k_norm_w, D), positions=(positions, T),
           slot_mapping=(slot_mapping, T), q_out=(q_out, T * Hq * D),
           k_cache=(k_cache, _cache_elems(L, k_cache)), v_cache=(v_cache, _cache_elems(L, k_cache)))
    q_f32 = q_out if q_out is not None and q_out.dtype == torch.float32 else None
    q_b16 = q_out if q_out is not None and q_out.dtype != torch.float32 else None
    _check(lib().flint_qk_norm_rope_append(
        C.byref(L), T, _ptr(q_in, _f32(), "q_in"), _ptr(k_in, _f32(), "k_in"),
        _ptr(v_in, _f32(), "v_in"), _ptr(q_norm_w, _f32(), "q_norm_w"),
        _ptr(k_norm_w, _f32(), "k_norm_w"), _ptr(positions, _i32(), "positions"),
        _ptr(slot_mapping, _i32(), "slot_mapping"), _ptr(q_f32, _f32(), "q_out"),
        _ptr(q_b16, _b16(), "q_out"), _ptr(k_cache, _kv(L), "k_cache"),
        _ptr(v_cache, _kv(L), "v_cache"), num_blocks, _stream(stream)))


def flint_attn_decode_workspace_size(L: FlintAttnLayer, num_seqs: int, max_seq_len: int,
                                     pages_per_split: int = 0) -> int:
    return int(lib().flint_attn_decode_workspace_size_ex(C.byref(L), num_seqs, max_seq_len,
                                                          pages_per_split))


def flint_attn_decode_plan(L: FlintAttnLayer, num_seqs: int, max_seq_len: int,
                           pages_per_split: int = 0):
    """(pages_per_split, num_splits) the library will use."""
    pps, ns = _I(), _I()
    _check(lib().flint_attn_decode_plan(C.byref(L), num_seqs, max_seq_len, pages_per_split,
                                        C.byref(pps), C.byref(ns)))
    return pps.value, ns.value


def flint_attn_decode_partials(L: FlintAttnLayer, q, k_cache, v_cache, block_tables, seq_lens,
                               max_seq_len: int, pages_per_split: int, part_o=None,
                               part_lse=None, stream=None):
    """K2 alone: every split's partial (normalised output, base-2 lse) for
    splits of `pages_per_split` pages; returns (part_o [B,S,Hq,128],
    part_lse [B,S,Hq]), allocated here when not given."""
    torch = _torch()
    B = q.shape[0]
    _, S = flint_attn_decode_plan(L, B, max_seq_len, pages_per_split)
    Hq, D = L.num_q_heads, L.head_dim
    _sizes(L, B, q=(q, B * Hq * D), k_cache=(k_cache, _cache_elems(L, k_cache)),
           v_cache=(v_cache, _cache_elems(L, k_cache)), block_tables=(block_tables, 0),
           seq_lens=(seq_lens, B), part_o=(part_o, B * S * Hq * D), part_lse=(part_lse, B * S * Hq))
    if part_o is None:
        part_o = torch.empty((B, S, L.num_q_heads, 128), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((B, S, L.num_q_heads), dtype=torch.float32, device=q.device)
    _check(lib().flint_attn_decode_partials(
        C.byref(L), B, _ptr(q, _f32(), "q"), _ptr(k_cache, _kv(L), "k_cache"),
        _ptr(v_cache, _kv(L), "v_cache"), k_cache.shape[0],
        _ptr(block_tables, _i32(), "block_tables"), block_tables.shape[1],
        _ptr(seq_lens, _i32(), "seq_lens"), max_seq_len, pages_per_split, S,
        _ptr(part_o, _f32(), "part_o"), _ptr(part_lse, _f32(), "part_lse"), _stream(stream)))
    return part_o, part_lse


def flint_attn_merge(L: FlintAttnLayer, part_o, part_lse, sinks, out=None, stream=None):
    """K3 alone: fold the partials [B,S,Hq,...] and the sinks into out [B,Hq,128]."""
    torch = _torch()
    B, S = part_lse.shape[0], part_lse.shape[1]
    Hq, D = L.num_q_heads, L.head_dim
    _sizes(L, part_o=(part_o, B * S * Hq * D), part_lse=(part_lse, B * S * Hq),
           sinks=(sinks, Hq), out=(out, B * Hq * D))
    if out is None:
        out = torch.empty((B, L.num_q_heads, 128), dtype=torch.float32, device=part_o.device)
    _check(lib().flint_attn_merge(C.byref(L), B, S, _ptr(part_o, _f32(), "part_o"),
                                  _ptr(part_lse, _f32(), "part_lse"), _ptr(sinks, _f32(), "sinks"),
                                  _ptr(out, _f32(), "out"), _stream(stream)))
    return out


def flint_attn_decode(L: FlintAttnLayer, q, k_cache, v_cache, block_tables, seq_lens,
                      max_seq_len: int, sinks, out, workspace=None, pages_per_split: int = 0,
                      stream=None):
    """Decode attention for q.shape[0] requests; writes out [B, Hq, 128] fp32.
    `workspace` (uint8 tensor) is allocated (zero-filled) here when not given;
    pass one (zero-filled once, e.g. torch.zeros) to keep the call free of
    allocations, e.g. under HIP-graph capture."""
    torch = _torch()
    B = q.shape[0]
    need = flint_attn_decode_workspace_size(L, B, max_seq_len, pages_per_split)
    Hq, D = L.num_q_heads, L.head_dim
    _sizes(L, B, q=(q, B * Hq * D), k_cache=(k_cache, _cache_elems(L, k_cache)),
           v_cache=(v_cache, _cache_elems(L, k_cache)), block_tables=(block_tables, 0),
           seq_lens=(seq_lens, B), sinks=(sinks, Hq), out=(out, B * Hq * D))
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().flint_attn_decode_ex(
        C.byref(L), B, _ptr(q, _f32(), "q"), _ptr(k_cache, _kv(L), "k_cache"),
        _ptr(v_cache, _kv(L), "v_cache"), k_cache.shape[0],
        _ptr(block_tables, _i32(), "block_tables"), block_tables.shape[1],
        _ptr(seq_lens, _i32(), "seq_lens"), max_seq_len, _ptr(sinks, _f32(), "sinks"),
        _ptr(out, _f32(), "out"),
        None if workspace is None else workspace.data_ptr(), ws_bytes, pages_per_split,
        _stream(stream)))
    return out


def flint_attn_decode_step(L: FlintAttnLayer, q_in, k_in, v_in, q_norm_w, k_norm_w,
                           slot_mapping, k_cache, v_cache, block_tables, seq_lens,
                           max_seq_len: int, sinks, out, q_out=None, workspace=None,
                           pages_per_split: int = 0, stream=None):
    """One fused decode step of one layer: norm/RoPE/append of each request's
    new token (raw q_in/k_in/v_in) and decode attention, in one launch."""
    torch = _torch()
    B = q_in.shape[0]
    need = flint_attn_decode_workspace_size(L, B, max_seq_len, pages_per_split)
    Hq, Hkv, D = L.num_q_heads, L.num_kv_heads, L.head_dim
    _sizes(L, B, q_in=(q_in, B * Hq * D), k_in=(k_in, B * Hkv * D), v_in=(v_in, B * Hkv * D),
           q_norm_w=(q_norm_w, D), k_norm_w=(k_norm_w, D), slot_mapping=(slot_mapping, B),
           q_out=(q_out, B * Hq * D), k_cache=(k_cache, _cache_elems(L, k_cache)),
           v_cache=(v_cache, _cache_elems(L, k_cache)), block_tables=(block_tables, 0),
           seq_lens=(seq_lens, B), sinks=(sinks, Hq), out=(out, B * Hq * D))
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q_in.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().flint_attn_decode_step(
        C.byref(L), B, _ptr(q_in, _f32(), "q_in"), _ptr(k_in, _f32(), "k_in"),
        _ptr(v_in, _f32(), "v_in"), _ptr(q_norm_w, _f32(), "q_norm_w"),
        _ptr(k_norm_w, _f32(), "k_norm_w"), _ptr(slot_mapping, _i32(), "slot_mapping"),
        _ptr(q_out, _f32(), "q_out"), _ptr(k_cache, _kv(L), "k_cache"),
        _ptr(v_cache, _kv(L), "v_cache"), k_cache.shape[0],
        _ptr(block_tables, _i32(), "block_tables"), block_tables.shape[1],
        _ptr(seq_lens, _i32(), "seq_lens"), max_seq_len, _ptr(sinks, _f32(), "sinks"),
        _ptr(out, _f32(), "out"), None if workspace is None else workspace.data_ptr(), ws_bytes,
        pages_per_split, _stream(stream)))
    return out


def flint_attn_decode_step_noalloc(L: FlintAttnLayer, q_in, k_in, v_in, q_norm_w, k_norm_w,
                                   slot_mapping, k_cache, v_cache, block_tables, seq_lens,
                                   max_seq_len: int, sinks, out, q_out=None,
                                   pages_per_split: int = 0, stream=None):
    """flint_attn_decode_step with the split partials in the library's static
    device scratch instead of a workspace: nothing is allocated."""
    B = q_in.shape[0]
    Hq, Hkv, D = L.num_q_heads, L.num_kv_heads, L.head_dim
    _sizes(L, B, q_in=(q_in, B * Hq * D), k_in=(k_in, B * Hkv * D), v_in=(v_in, B * Hkv * D),
           q_norm_w=(q_norm_w, D), k_norm_w=(k_norm_w, D), slot_mapping=(slot_mapping, B),
           q_out=(q_out, B * Hq * D), k_cache=(k_cache, _cache_elems(L, k_cache)),
           v_cache=(v_cache, _cache_elems(L, k_cache)), block_tables=(block_tables, 0),
           seq_lens=(seq_lens, B), sinks=(sinks, Hq), out=(out, B * Hq * D))
    _check(lib().flint_attn_decode_step_noalloc(
        C.byref(L), B, _ptr(q_in, _f32(), "q_in"), _ptr(k_in, _f32(), "k_in"),
        _ptr(v_in, _f32(), "v_in"), _ptr(q_norm_w, _f32(), "q_norm_w"),
        _ptr(k_norm_w, _f32(), "k_norm_w"), _ptr(slot_mapping, _i32(), "slot_mapping"),
        _ptr(q_out, _f32(), "q_out"), _ptr(k_cache, _kv(L), "k_cache"),
        _ptr(v_cache, _kv(L), "v_cache"), k_cache.shape[0],
        _ptr(block_tables, _i32(), "block_tables"), block_tables.shape[1],
        _ptr(seq_lens, _i32(), "seq_lens"), max_seq_len, _ptr(sinks, _f32(), "sinks"),
        _ptr(out, _f32(), "out"), pages_per_split, _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def flint_attn_prefill_workspace_size(L: FlintAttnLayer, num_seqs: int, max_q_len: int,
                                      max_seq_len: int) -> int:
    return int(lib().flint_attn_prefill_workspace_size(C.byref(L), num_seqs, max_q_len,
                                                        max_seq_len))


def flint_attn_prefill(L: FlintAttnLayer, q, cu_q_lens, max_q_len: int, k_cache, v_cache,
                       block_tables, seq_lens, max_seq_len: int, sinks, out, workspace=None,
                       stream=None):
    """Causal prefill for the rows in cu_q_lens; q bf16 bits [total_q, Hq, 128],
    out fp32 [total_q, Hq, 128].  workspace: a device tensor of at least
    flint_attn_prefill_workspace_size bytes holding zeros (each call leaves it
    so), or None for a fresh zero-filled one."""
    torch = _torch()
    B = cu_q_lens.shape[0] - 1
    Hq, D = L.num_q_heads, L.head_dim
    _sizes(L, B, q=(q, q.shape[0] * Hq * D), out=(out, q.shape[0] * Hq * D),
           k_cache=(k_cache, _cache_elems(L, k_cache)), v_cache=(v_cache, _cache_elems(L, k_cache)),
           block_tables=(block_tables, 0), seq_lens=(seq_lens, B), sinks=(sinks, Hq))
    need = flint_attn_prefill_workspace_size(L, B, max_q_len, max_seq_len)
    if workspace is None and need > 0:  # zero-filled; every call leaves it zero
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().flint_attn_prefill(
        C.byref(L), B, _ptr(q, _b16(), "q"), _ptr(cu_q_lens, _i32(), "cu_q_lens"), q.shape[0],
        max_q_len,
        _ptr(k_cache, _kv(L), "k_cache"), _ptr(v_cache, _kv(L), "v_cache"), k_cache.shape[0],
        _ptr(block_tables, _i32(), "block_tables"), block_tables.shape[1],
        _ptr(seq_lens, _i32(), "seq_lens"), max_seq_len, _ptr(sinks, _f32(), "sinks"),
        _ptr(out, _f32(), "out"), None if workspace is None else workspace.data_ptr(), ws_bytes,
        _stream(stream)))
    return out


def flint_moe_workspace_size(M: FlintMoeLayer, num_tokens: int) -> int:
    return int(lib().flint_moe_workspace_size(C.byref(M), num_tokens))


def flint_moe_forward(M: FlintMoeLayer, x, w_router, w_gate_up, w_down, out=None, topk_ids=None,
                      topk_weights=None, workspace=None, stream=None):
    """MoE sublayer for x [T, hidden] fp32 (T <= 8); weights are bf16-bits
    tensors in the layout of include/flint.h.  Returns (out [T, hidden] fp32,
    topk_ids [T, top_k] int32, topk_weights [T, top_k] fp32)."""
    torch = _torch()
    T = x.shape[0]
    dev = x.device
    H, E, I, S, K = M.hidden, M.num_experts, M.inter, M.num_shared, M.top_k
    _sizes(M, x=(x, T * H), w_router=(w_router, E * H), w_gate_up=(w_gate_up, (E + S) * 2 * I * H),
           w_down=(w_down, (E + S) * H * I), out=(out, T * H), topk_ids=(topk_ids, T * K),
           topk_weights=(topk_weights, T * K))
    if out is None:
        out = torch.empty((T, M.hidden), dtype=torch.float32, device=dev)
    if topk_ids is None:
        topk_ids = torch.empty((T, M.top_k), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, M.top_k), dtype=torch.float32, device=dev)
    need = flint_moe_workspace_size(M, T)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().flint_moe_forward(
        C.byref(M), T, _ptr(x, _f32(), "x"), _ptr(w_router, _b16(), "w_router"),
        _ptr(w_gate_up, _b16(), "w_gate_up"), _ptr(w_down, _b16(), "w_down"),
        _ptr(topk_ids, _i32(), "topk_ids"), _ptr(topk_weights, _f32(), "topk_weights"),
        _ptr(out, _f32(), "out"), None if workspace is None else workspace.data_ptr(), ws_bytes,
        _stream(stream)))
    return out, topk_ids, topk_weights


def abi_version() -> int:
    return int(lib().flint_abi_version())
