"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad host-visible arguments before any HIP call."""
import ctypes as C
import os
import re

import pytest

import full_gqa_decode_amd as fl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(flint_\w+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    lib = fl.lib()
    declared = _declared_symbols()
    assert {"flint_qk_norm_rope_append", "flint_attn_decode", "flint_attn_prefill"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == {s[0] for s in fl.SIGNATURES}


def test_abi_version_and_status_strings():
    lib = fl.lib()
    assert lib.flint_abi_version() == 4
    # 12 four-byte fields, in the header's order
    assert C.sizeof(fl.FlintAttnLayer) == 48
    assert [f[0] for f in fl.FlintAttnLayer._fields_][-3:] == ["kv_dtype", "k_scale", "v_scale"]
    for s, name in fl.STATUS_NAMES.items():
        assert lib.flint_status_string(s).decode() == name


# fake device pointers: validation must fail before they are ever used
P = 0x100000
Q = 0x200000
WS = 0x300000


def _decode(L, **kw):
    a = dict(num_seqs=1, q=P, k=Q, v=Q + 0x1000, nb=4, bt=P + 0x10000, bt_stride=4, sl=P + 0x20000,
             max_seq_len=64, sinks=P + 0x30000, out=P + 0x40000, ws=WS, ws_bytes=1 << 20, pps=0)
    a.update(kw)
    return fl.lib().flint_attn_decode_ex(C.byref(L), a["num_seqs"], a["q"], a["k"], a["v"], a["nb"],
                                          a["bt"], a["bt_stride"], a["sl"], a["max_seq_len"],
                                          a["sinks"], a["out"], a["ws"], a["ws_bytes"], a["pps"],
                                          None)


INVALID, UNSUPPORTED, WS_SMALL = 1, 2, 3


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID),
    (dict(out=None), INVALID),
    (dict(sinks=None), INVALID),
    (dict(nb=0), INVALID),
    (dict(bt_stride=0), INVALID),
    (dict(max_seq_len=0), INVALID),
    (dict(max_seq_len=65), INVALID),       # > bt_stride * 16
    (dict(num_seqs=-1), INVALID),
    (dict(pps=-1), INVALID),
    (dict(q=P + 4), INVALID),              # misaligned
    (dict(out=P), INVALID),                # aliases q
    (dict(ws=WS + 8, ws_bytes=1 << 20, max_seq_len=64, pps=1), INVALID),  # workspace alignment
])
def test_decode_rejects_bad_arguments(kw, status):
    L = fl.full_layer()
    assert _decode(L, **kw) == status
    assert fl.lib().flint_last_error().decode() != ""


def test_decode_workspace_too_small():
    L = fl.full_layer()
    need = fl.flint_attn_decode_workspace_size(L, 1, 64, pages_per_split=1)
    assert need > 0
    assert _decode(L, ws_bytes=need - 1, pps=1) == WS_SMALL
    assert _decode(L, ws=None, pps=1) == WS_SMALL


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, UNSUPPORTED),
    ("block_size", 32, UNSUPPORTED),
    ("num_kv_heads", 0, UNSUPPORTED),
    ("num_q_heads", 16, UNSUPPORTED),
    ("window", -1, INVALID),
    ("use_rope", 2, INVALID),
    ("softmax_scale", float("inf"), INVALID),
    ("kv_dtype", 2, INVALID),
    ("kv_dtype", -1, INVALID),
])
def test_layer_validation(field, value, status):
    L = fl.full_layer()
    setattr(L, field, value)
    assert _decode(L) == status


@pytest.mark.parametrize("k_scale,v_scale", [(0.0, 1.0), (1.0, -2.0), (float("inf"), 1.0),
                                             (1.0, float("nan"))])
def test_fp8_layer_needs_positive_finite_scales(k_scale, v_scale):
    L = fl.full_layer(kv_dtype=fl.FLINT_KV_FP8_E4M3, k_scale=k_scale, v_scale=v_scale)
    assert _decode(L) == INVALID
    # a bf16 layer ignores the scales
    L = fl.full_layer(k_scale=k_scale, v_scale=v_scale)
    assert _decode(L, q=None) == INVALID and "NULL" in fl.lib().flint_last_error().decode()


def test_prefill_checks_fp8_scales():
    lib = fl.lib()
    L = fl.full_layer(kv_dtype=fl.FLINT_KV_FP8_E4M3, k_scale=0.0, v_scale=2.0)
    args = [C.byref(L), 1, P, P + 0x10000, 32, 32, Q, Q + 0x10000, 4, P + 0x20000, 4,
            P + 0x30000, 64, P + 0x40000, P + 0x50000, None, 0, None]
    assert lib.flint_attn_prefill(*args) == INVALID


def test_fused_step_rejects_q_out_aliasing_q_in():
    # every split workgroup of the fused step reads the raw q_in while one of
    # them writes q_out: a shared buffer must be refused before any launch
    lib = fl.lib()
    L = fl.full_layer()
    qi, qo = P + 0x80000, P + 0x90000
    args = [C.byref(L), 1, qi, P + 0x10000, P + 0x20000, P + 0x30000, P + 0x40000, P + 0x50000,
            qo, Q, Q + 0x10000, 4, P + 0x60000, 4, P + 0x70000, 64, P + 0xA0000, P + 0xB0000,
            WS, 1 << 20, 0, None]
    for alias in (qi, qi + 256):
        bad = list(args)
        bad[8] = alias
        assert lib.flint_attn_decode_step(*bad) == INVALID
        assert "q_out" in lib.flint_last_error().decode()


def test_noalloc_step_limit_is_checked_before_any_launch():
    # a plan whose partials exceed the static scratch is refused on the host
    lib = fl.lib()
    L = fl.full_layer()
    B, ctx = 64, 131072
    assert fl.flint_attn_decode_workspace_size(L, B, ctx) > fl.NOALLOC_SCRATCH_BYTES
    args = [C.byref(L), B, P, P + 0x10000, P + 0x20000, P + 0x30000, P + 0x40000, P + 0x50000,
            None, Q, Q + 0x10000, 4, P + 0x60000, ctx // 16, P + 0x70000, ctx, P + 0xA0000,
            P + 0xB0000, 0, None]
    assert lib.flint_attn_decode_step_noalloc(*args) == WS_SMALL
    assert "static scratch" in lib.flint_last_error().decode()
    bad = list(args)
    bad[1] = -1
    assert lib.flint_attn_decode_step_noalloc(*bad) == INVALID
    bad = list(args)
    bad[1] = 0
    assert lib.flint_attn_decode_step_noalloc(*bad) == 0


def test_zero_requests_is_a_no_op():
    assert _decode(fl.full_layer(), num_seqs=0, q=None, out=None) == 0


def test_append_rejects_bad_arguments():
    lib = fl.lib()
    L = fl.sliding_layer()
    args = [C.byref(L), 1, P, P + 0x10000, P + 0x20000, P + 0x30000, P + 0x40000, P + 0x50000,
            P + 0x60000, P + 0x70000, None, Q, Q + 0x10000, 4, None]
    bad = list(args)
    bad[10] = P + 0x80000  # both q outputs set
    assert lib.flint_qk_norm_rope_append(*bad) == INVALID
    bad = list(args)
    bad[9] = None  # no q output
    assert lib.flint_qk_norm_rope_append(*bad) == INVALID
    bad = list(args)
    bad[13] = 0  # no pages
    assert lib.flint_qk_norm_rope_append(*bad) == INVALID
    bad = list(args)
    bad[11] = Q + 2  # misaligned cache
    assert lib.flint_qk_norm_rope_append(*bad) == INVALID
    bad = list(args)
    bad[1] = -1
    assert lib.flint_qk_norm_rope_append(*bad) == INVALID
    bad = list(args)
    bad[1] = 0  # nothing to do
    assert lib.flint_qk_norm_rope_append(*bad) == 0


def test_prefill_rejects_bad_arguments():
    lib = fl.lib()
    L = fl.full_layer()
    base = [C.byref(L), 1, P, P + 0x10000, 32, 32, Q, Q + 0x10000, 4, P + 0x20000, 4,
            P + 0x30000, 64, P + 0x40000, P + 0x50000, None, 0, None]
    for idx, val in ((5, 65), (12, 65), (12, 0), (2, None), (14, None), (8, 0), (2, P + 2),
                     (4, -1)):
        bad = list(base)
        bad[idx] = val
        assert lib.flint_attn_prefill(*bad) == INVALID, (idx, val)
    # no rows: nothing to do, whatever the pointers
    empty = list(base)
    empty[4] = 0
    empty[2] = None
    assert lib.flint_attn_prefill(*empty) == 0


def test_prefill_workspace_is_a_counter_and_one_flag_per_item():
    # work items: ceil(max_q_len / 32) row blocks x KV heads x requests; the
    # workspace holds the claim counter (8 bytes), the count of items flagged
    # for the bf16 fix-up launch (4 + 4 bytes) and one 4-byte flag per item
    L = fl.full_layer()
    size = fl.flint_attn_prefill_workspace_size
    assert size(L, 1, 64 * 32, 4096) == 16 + 4 * 256       # 64 x 4 x 1 items
    assert size(L, 1, 64 * 32 + 1, 4096) == 16 + 4 * 260   # 65 row blocks
    assert size(L, 64, 32, 4096) == 16 + 4 * 256 and size(L, 65, 32, 4096) == 16 + 4 * 260
    assert size(L, 1, 32768, 32768) == 16 + 4 * 4096 and size(L, 0, 32768, 32768) == 0
    assert size(L, 1, 0, 4096) == 0
    L1 = fl.full_layer(num_q_heads=8, num_kv_heads=1)
    assert size(L1, 1, 256 * 32, 8192) == 16 + 4 * 256
    lib = fl.lib()
    # 128 row blocks x 4 heads = 512 items: 2064 bytes, checked before
    # anything is launched
    base = [C.byref(L), 1, P, P + 0x10000, 4096, 4096, Q, Q + 0x10000, 256, P + 0x20000, 256,
            P + 0x30000, 4096, P + 0x40000, P + 0x50000, None, 0, None]
    assert lib.flint_attn_prefill(*base) == WS_SMALL
    assert "need 2064" in lib.flint_last_error().decode()
    small = list(base)
    small[15], small[16] = P + 0x60000, 2060
    assert lib.flint_attn_prefill(*small) == WS_SMALL
    misaligned = list(base)
    misaligned[15], misaligned[16] = P + 0x60004, 2064
    assert lib.flint_attn_prefill(*misaligned) == INVALID


def test_decode_plan_covers_every_page():
    L = fl.full_layer()
    for B, ctx, pps in ((1, 100000, 0), (1, 4096, 0), (64, 131072, 0), (3, 17, 0), (1, 100000, 7)):
        p, s = fl.flint_attn_decode_plan(L, B, ctx, pps)
        pages = -(-ctx // 16)
        assert p >= 1 and s >= 1 and (s - 1) * p < pages <= s * p
    Ls = fl.sliding_layer()
    p, s = fl.flint_attn_decode_plan(Ls, 1, 100000, 0)
    assert s * p >= 33 and (s - 1) * p < 33


def _partials(L, **kw):
    a = dict(num_seqs=1, q=P, k=Q, v=Q + 0x1000, nb=4, bt=P + 0x10000, bt_stride=4,
             sl=P + 0x20000, max_seq_len=64, pps=1, ns=4, po=P + 0x40000, pl=P + 0x50000)
    a.update(kw)
    return fl.lib().flint_attn_decode_partials(C.byref(L), a["num_seqs"], a["q"], a["k"], a["v"],
                                                a["nb"], a["bt"], a["bt_stride"], a["sl"],
                                                a["max_seq_len"], a["pps"], a["ns"], a["po"],
                                                a["pl"], None)


@pytest.mark.parametrize("kw", [
    dict(pps=0),               # the split size must be explicit
    dict(ns=3),                # 64 keys in 1-page splits is 4 splits
    dict(q=None),
    dict(po=None),
    dict(pl=None),
    dict(po=P + 0x40004),      # misaligned partial outputs
    dict(max_seq_len=65),      # > bt_stride * 16
    dict(nb=0),
])
def test_partials_reject_bad_arguments(kw):
    assert _partials(fl.full_layer(), **kw) == INVALID
    assert fl.lib().flint_last_error().decode() != ""


def test_partials_split_count_follows_the_plan():
    L = fl.sliding_layer()
    # a 513-key window spans at most 33 pages: 3-page splits give 11
    assert fl.flint_attn_decode_plan(L, 1, 100_000, 3) == (3, 11)
    assert _partials(L, max_seq_len=64, bt_stride=4, pps=3, ns=2, num_seqs=0) == 0


@pytest.mark.parametrize("kw", [
    dict(ns=0), dict(po=None), dict(pl=None), dict(sinks=None), dict(out=None),
])
def test_merge_rejects_bad_arguments(kw):
    a = dict(num_seqs=1, ns=4, po=P, pl=P + 0x10000, sinks=P + 0x20000, out=P + 0x30000)
    a.update(kw)
    assert fl.lib().flint_attn_merge(C.byref(fl.full_layer()), a["num_seqs"], a["ns"], a["po"],
                                     a["pl"], a["sinks"], a["out"], None) == INVALID


# ---------------------------------------------------------------------------
# MoE sublayer
# ---------------------------------------------------------------------------

def _moe(M, **kw):
    a = dict(T=1, x=P, wr=Q, wgu=Q + 0x100000, wd=Q + 0x200000, ids=P + 0x10000,
             wts=P + 0x20000, out=P + 0x30000, ws=WS, ws_bytes=1 << 20)
    a.update(kw)
    return fl.lib().flint_moe_forward(C.byref(M), a["T"], a["x"], a["wr"], a["wgu"], a["wd"],
                                      a["ids"], a["wts"], a["out"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("field,value", [("hidden", 1000), ("hidden", 8192), ("inter", 256),
                                         ("num_experts", 257), ("num_experts", 0), ("top_k", 9),
                                         ("top_k", 0), ("num_shared", 3)])
def test_moe_rejects_unsupported_shapes(field, value):
    M = fl.moe_layer()
    setattr(M, field, value)
    assert _moe(M) == UNSUPPORTED
    assert fl.flint_moe_workspace_size(M, 1) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(T=9), UNSUPPORTED),
    (dict(x=None), INVALID),
    (dict(wd=None), INVALID),
    (dict(ids=None), INVALID),
    (dict(x=P + 4), INVALID),
    (dict(wgu=Q + 8), INVALID),
    (dict(out=P), INVALID),              # aliases x
    (dict(ws_bytes=16), WS_SMALL),
    (dict(ws=None), WS_SMALL),
    (dict(ws=WS + 64), INVALID),
])
def test_moe_rejects_bad_arguments(kw, status):
    assert _moe(fl.moe_layer(), **kw) == status
    assert fl.lib().flint_last_error().decode() != ""


def test_moe_zero_tokens_is_a_no_op_and_workspace_grows_with_tokens():
    M = fl.moe_layer()
    assert _moe(M, T=0, x=None, out=None) == 0
    w1, w8 = fl.flint_moe_workspace_size(M, 1), fl.flint_moe_workspace_size(M, 8)
    # logits and the SwiGLU activations, fp32, each part 256-byte aligned
    assert w1 == 1024 + 7 * 512 * 4
    assert w8 == 8 * 256 * 4 + 8 * 7 * 512 * 4


def _z(*shape, dtype="float32"):
    import torch
    return torch.zeros(shape, dtype=getattr(torch, dtype))


def test_python_binding_checks_tensor_sizes_before_the_abi():
    # The C ABI sees only pointers; the binding checks every tensor's element
    # count against the layer and the batch first (host tensors reach no
    # kernel: a size error is raised before the device checks).
    L = fl.layer(window=0)
    B, nb = 2, 3
    kc, vc = _z(nb, 4, 16, 128, dtype="int16"), _z(nb, 4, 128, 16, dtype="int16")
    bt, sl = _z(B, 8, dtype="int32"), _z(B, dtype="int32")
    q, out, sinks = _z(B, 32, 128), _z(B, 32, 128), _z(32)
    bad = [
        dict(q=_z(B, 32, 127)),
        dict(out=_z(B, 31, 128)),
        dict(sinks=_z(31)),
        dict(seq_lens=_z(B + 1, dtype="int32")),
        dict(v_cache=_z(nb - 1, 4, 128, 16, dtype="int16")),
        dict(block_tables=_z(B - 1, 8, dtype="int32")),
    ]
    for kw in bad:
        args = dict(q=q, k_cache=kc, v_cache=vc, block_tables=bt, seq_lens=sl, sinks=sinks,
                    out=out)
        args.update(kw)
        with pytest.raises(ValueError):
            fl.flint_attn_decode(L, args["q"], args["k_cache"], args["v_cache"],
                                 args["block_tables"], args["seq_lens"], 100, args["sinks"],
                                 args["out"])
    with pytest.raises(ValueError, match="k_in"):
        fl.flint_attn_decode_step(L, q, _z(B, 4, 64), _z(B, 4, 128), _z(128), _z(128),
                                  _z(B, dtype="int32"), kc, vc, bt, sl, 100, sinks, out)
    with pytest.raises(ValueError, match="positions"):
        fl.flint_qk_norm_rope_append(L, q, _z(B, 4, 128), _z(B, 4, 128), _z(128), _z(128),
                                     _z(B + 1, dtype="int32"), _z(B, dtype="int32"), q, kc, vc)
    with pytest.raises(ValueError, match="out"):
        fl.flint_attn_prefill(L, _z(5, 32, 128, dtype="int16"), _z(B + 1, dtype="int32"), 5,
                              kc, vc, bt, sl, 100, sinks, _z(4, 32, 128))
    with pytest.raises(ValueError, match="sinks"):
        fl.flint_attn_merge(L, _z(B, 3, 32, 128), _z(B, 3, 32), _z(8), out)
    M = fl.moe_layer(512, 16, 2, 512, 1)
    with pytest.raises(ValueError, match="w_down"):
        fl.flint_moe_forward(M, _z(1, 512), _z(16, 512, dtype="int16"),
                             _z(17, 2, 512, 512, dtype="int16"), _z(16, 512, 512, dtype="int16"))


def test_ceiling_library_exports_its_kernels():
    # the bench's measurement kernels live in a library of their own, which
    # the product library neither links nor calls
    from full_gqa_decode_amd import build as fb
    fl.lib()
    lib = C.CDLL(fb.SO_CEILING)
    for name in ("flint_ceiling_stream_bytes", "flint_ceiling_stream_read",
                 "flint_ceiling_page_walk", "flint_ceiling_empty", "flint_ceiling_atomics"):
        assert hasattr(lib, name), name
    lib.flint_ceiling_stream_bytes.restype = C.c_long
    assert lib.flint_ceiling_stream_bytes() == 256 * 8 * 96 * 1024
    # argument checks before any launch
    lib.flint_ceiling_stream_read.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    assert lib.flint_ceiling_stream_read(3, 1, None, None, None) == -1
    lib.flint_ceiling_page_walk.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                                            C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    assert lib.flint_ceiling_page_walk(None, None, None, 0, 4, 98, 0, None, None) == -1
    assert "ceiling" not in open(fb.SO, "rb").read().decode("latin-1")


C_CLIENT = r"""
#include <stdio.h>
#include "flint.h"

int main(void) {
  flint_attn_layer L = {32, 4, 128, 16, 0, 0, 10000.0f, 1e-6f, 0.08838834764831845f,
                        FLINT_KV_BF16, 1.0f, 1.0f};
  int32_t pps = 0, splits = 0;
  flint_status st = flint_attn_decode_plan(&L, 1, 100000, 0, &pps, &splits);
  size_t ws = flint_attn_decode_workspace_size(&L, 1, 100000);
  flint_status bad = flint_attn_decode_plan(NULL, 1, 100000, 0, &pps, &splits);
  printf("%d %d %d %d %zu %d\n", (int)flint_abi_version(), (int)st, (int)pps, (int)splits, ws,
         (int)bad);
  return 0;
}
"""


def test_header_is_c11_and_a_c_program_links_and_calls_the_library(tmp_path):
    # The boundary from plain C: include/flint.h compiles as strict C11 and a
    # program linked against libflint.so gets the same plan, workspace size
    # and error status as the Python binding (host-only calls, no GPU).
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(fl.LIB_PATH)
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", libdir, "-lflint", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, check=True)
    ver, st, pps, splits, ws, bad = (int(x) for x in out.stdout.split())
    L = fl.full_layer()
    assert ver == fl.lib().flint_abi_version()
    assert st == fl.FLINT_OK and (pps, splits) == fl.flint_attn_decode_plan(L, 1, 100000)
    assert ws == fl.flint_attn_decode_workspace_size(L, 1, 100000)
    assert fl.STATUS_NAMES[bad] == "FLINT_ERR_INVALID_ARGUMENT"
