"""Decode-attention bench for Flint's 49-layer stack on one MI355X.

Workload: one decode step at batch 1 and a 100,000-token context over all 49
attention layers -- 14 full-context NoPE layers reading 100,000 keys each and
35 RoPE sliding layers reading the last 513 keys -- from a bf16 paged KV cache
(16-token pages; every full layer's 6,250 pages in a seeded random physical
order; each sliding layer on a 33-page ring).  A step runs, per layer in
order, the fused norm/RoPE/append of the new token and then split-K decode
attention with the sink merge; the 49 layers are captured into one HIP graph.

Prints one JSON line.  `value` is microseconds per step (lower is better).
All inputs are seeded synthetic tensors (~N(0,1)); the KV pages are drawn on
the GPU by torch's seeded generator and are resident in HBM before timing
starts.
"""
from __future__ import annotations

import argparse
import contextlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "decode-attn µs/step & HBM GB/s (% of peak), bs1 100K ctx, 49 layers"
CTX = 100_000
LAYERS = 49
FULL_LAYERS = [l for l in range(LAYERS) if l % 7 in (3, 6)]   # 14 full, 35 sliding
WINDOW = 513
RING = 33
HQ, HKV, D, PAGE = 32, 4, 128, 16
HBM_PEAK_GBPS = 8000.0
BF16_DENSE_TFLOPS = 2500.0
SEED = 0
PARITY_TOL = 4e-3   # max |GPU - oracle| of the fp32 outputs over the step
KV_BYTES_PER_TOKEN_LAYER = 2 * HKV * D * 2   # K and V rows of one token, one layer
COPY_PROBE_BYTES = 256 << 20


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_full_layer_ctx100k_hbm_counters.md")
DECODE_SOURCES = ["decode.hip", "device.h", "launch.h", "api.hip"]


def measured_traffic(key="traffic_bytes_per_launch"):
    """HBM bytes from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary --
    per launch of K2 alone (traffic_bytes_per_launch) or per 49-layer step
    (step_traffic_bytes) -- or None once the decode sources differ from the
    ones those counters were taken on."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if ":" in line and line.split(":")[0] in (key, "source_sha256"):
            k, v = line.split(":", 1)
            vals[k] = v.strip()
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "full_gqa_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("source_sha256") != h.hexdigest() or key not in vals:
        return None
    return int(vals[key])


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@contextlib.contextmanager
def marker(name):
    """A roctx range (torch.cuda.nvtx maps to roctx on ROCm) around a phase of
    the bench, so that `rocprofv3 --marker-trace` ties each kernel to its leg
    and, in the eager step, to its layer.  Host-side only: graph replays carry
    none, and the timed loop gets one range around all of its steps."""
    import torch
    torch.cuda.nvtx.range_push(name)
    try:
        yield
    finally:
        torch.cuda.nvtx.range_pop()


def build_inputs(dev):
    """Seeded inputs for every layer, resident in HBM (the 2.9 GB of KV pages
    are drawn on the GPU by torch's generator; small tensors on the host)."""
    import torch
    pages = -(-CTX // PAGE)
    t = CTX - 1
    layers = []
    for l in range(LAYERS):
        full = l in FULL_LAYERS
        if full:
            bt, nb = synth.shuffled_block_table(SEED, (2, l, synth.PERM), 1, [pages], pages)
        else:
            bt, nb = synth.ring_block_table(SEED, (2, l, synth.PERM), 1, pages, RING, pages)
        kd = synth.normal_bf16_bits_torch(SEED, (2, l, synth.KC), (nb, HKV, PAGE, D), dev)
        vd = synth.normal_bf16_bits_torch(SEED, (2, l, synth.VC), (nb, HKV, D, PAGE), dev)
        q = synth.normal(SEED, (2, l, synth.Q), (1, HQ, D))
        k = synth.normal(SEED, (2, l, synth.K), (1, HKV, D))
        v = synth.normal(SEED, (2, l, synth.V), (1, HKV, D))
        sinks = synth.normal(SEED, (2, l, synth.SINK), HQ)
        slot = int(bt[0, t // PAGE]) * PAGE + t % PAGE
        up = lambda a: torch.from_numpy(np.ascontiguousarray(
            a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)
        layers.append(dict(
            full=full, host=dict(bt=bt, q=q, k=k, v=v, sinks=sinks, slot=slot),
            bt=up(bt), kc=kd, vc=vd, q_in=up(q), k_in=up(k), v_in=up(v),
            sinks=up(sinks), slots=up(np.array([slot], np.int32)),
            q_out=torch.empty((1, HQ, D), dtype=torch.float32, device=dev),
            out=torch.empty((1, HQ, D), dtype=torch.float32, device=dev)))
        if l % 7 == 6:
            log(f"bench: inputs for layers 0..{l} resident")
    return layers


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-moe", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads' legs (single-layer latency of a full layer at "
                         "4096 tokens and a sliding layer at 32768, 64 ragged requests, batches "
                         "of 2..16 at 100K context)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run the prefill leg (for counter runs of the prefill kernel)")
    ap.add_argument("--batch-legs", action="store_true",
                    help="only time batched decode: 64 ragged requests of 1024..131072 tokens "
                         "(one full and one sliding layer) and batches of 2..16 requests at "
                         "100K context (fused step), and print one JSON line")
    ap.add_argument("--ceilings", action="store_true",
                    help="only the machine-ceiling leg (launch, streaming reads, the split "
                         "kernel's loads alone, atomics), as one JSON line")
    ap.add_argument("--stamps", action="store_true",
                    help="only the phase stamps of the prefill and slice kernels, from the "
                         "instrumented libflint_stamps.so (python -m full_gqa_decode_amd.build "
                         "--stamps), as one JSON line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy three times (the "
                         "known-size kernel that calibrates HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decode path here is single-GPU (--gpus {args.gpus} "
              "is not supported; run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.ceilings:
        print(json.dumps({"ceilings": bench_ceilings(torch.device("cuda:0"))}), flush=True)
        return
    if args.copy_probe:
        copy_probe(torch.device("cuda:0"))
        return
    if args.stamps:
        print(json.dumps({"stamps": bench_stamps(torch.device("cuda:0"))}), flush=True)
        return
    import full_gqa_decode_amd as fl
    fl.lib()
    dev = torch.device("cuda:0")
    if args.prefill_only:
        print(json.dumps(bench_prefill(fl, dev, None)), flush=True)
        return
    if args.batch_legs:
        print(json.dumps(bench_batches(fl, dev)), flush=True)
        return
    eps = float(np.float32(1e-6))
    FULL = fl.layer(window=0, use_rope=0, rms_eps=eps)
    SLIDE = fl.layer(window=WINDOW, use_rope=1, rms_eps=eps)
    ones = torch.ones(D, dtype=torch.float32, device=dev)
    pos = torch.tensor([CTX - 1], dtype=torch.int32, device=dev)
    seq_lens = torch.tensor([CTX], dtype=torch.int32, device=dev)

    t0 = time.time()
    layers = build_inputs(dev)
    if not args.no_cpu_baseline:   # the oracle reads the same drawn pages
        for L in layers:
            L["kc0"] = L["kc"].cpu().numpy().view(np.uint16)
            L["vc0"] = L["vc"].cpu().numpy().view(np.uint16)
    log(f"bench: inputs ready in {time.time() - t0:.1f}s")
    ws_bytes = max(fl.flint_attn_decode_workspace_size(FULL, 1, CTX),
                   fl.flint_attn_decode_workspace_size(SLIDE, 1, CTX), 256)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)

    def layer_step_unfused(L):
        Ld = FULL if L["full"] else SLIDE
        fl.flint_qk_norm_rope_append(Ld, L["q_in"], L["k_in"], L["v_in"], ones, ones, pos,
                                     L["slots"], L["q_out"], L["kc"], L["vc"])
        fl.flint_attn_decode(Ld, L["q_out"], L["kc"], L["vc"], L["bt"], seq_lens, CTX,
                             L["sinks"], L["out"], workspace=ws)

    def layer_step(L):
        # one launch per layer (plus the split merge on full layers): the fused
        # norm/RoPE/append of the new token and the attention
        Ld = FULL if L["full"] else SLIDE
        fl.flint_attn_decode_step(Ld, L["q_in"], L["k_in"], L["v_in"], ones, ones, L["slots"],
                                  L["kc"], L["vc"], L["bt"], seq_lens, CTX, L["sinks"], L["out"],
                                  workspace=ws)

    def step():
        for idx, L in enumerate(layers):
            with marker(f"layer {idx} ({'full' if L['full'] else 'sliding'})"):
                layer_step(L)

    def step_unfused():
        for L in layers:
            layer_step_unfused(L)

    stream = torch.cuda.Stream()

    def capture(fn):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(gr, stream=stream):
                fn()
        return gr

    # eager once per path; both paths and their graphs must agree bit for bit
    step_unfused()
    torch.cuda.synchronize()
    eager = [L["out"].clone() for L in layers]
    step()
    torch.cuda.synchronize()
    for L, e in zip(layers, eager):
        assert torch.equal(L["out"], e), "fused step differs from append + decode"
    g = capture(step)
    g_unfused = capture(step_unfused)
    for _ in range(args.warmup):
        g.replay()
        g_unfused.replay()
    torch.cuda.synchronize()
    for L, e in zip(layers, eager):
        assert torch.equal(L["out"], e), "graph replay differs from eager"

    # timed region: K whole steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    with torch.cuda.stream(stream), marker(f"timed: {args.steps} steps of the 49-layer graph"):
        ev[0].record(stream)
        for i in range(args.steps):
            g.replay()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(args.steps)]
    us_step = ev[0].elapsed_time(ev[-1]) * 1e3 / args.steps
    log(f"bench: {args.steps} steps, {us_step:.1f} us/step (median {statistics.median(per):.1f}, "
        f"wall {wall * 1e6 / args.steps:.1f} us/step)")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(args.steps):
            g_unfused.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us_unfused = e0.elapsed_time(e1) * 1e3 / args.steps
    log(f"bench: unfused (append, then decode) {us_unfused:.1f} us/step")

    # K1 alone: the 49 appends of the new token, one graph
    def appends():
        for L in layers:
            fl.flint_qk_norm_rope_append(FULL if L["full"] else SLIDE, L["q_in"], L["k_in"],
                                         L["v_in"], ones, ones, pos, L["slots"], L["q_out"],
                                         L["kc"], L["vc"])
    g_app = capture(appends)
    g_app.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(args.steps):
            g_app.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us_append = e0.elapsed_time(e1) * 1e3 / args.steps
    log(f"bench: append alone (49 layers) {us_append:.1f} us/step")

    # dominant kernel: the split-K kernel (K2) of a full layer, alone, through
    # flint_attn_decode_partials -- 14 full layers back to back in one graph,
    # timed on the stream it runs on; and the launch pair of the fused step
    # (split kernel + merge) the same way
    full_layers = [L for L in layers if L["full"]]
    pps, nsplit = fl.flint_attn_decode_plan(FULL, 1, CTX)
    part_o = torch.empty((1, nsplit, HQ, D), dtype=torch.float32, device=dev)
    part_lse = torch.empty((1, nsplit, HQ), dtype=torch.float32, device=dev)

    def time_graph(fn, reps=20):
        gr = capture(fn)
        for _ in range(3):
            gr.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            t0.record(stream)
            for _ in range(reps):
                gr.replay()
            t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / (reps * len(full_layers))

    us_k2 = time_graph(lambda: [fl.flint_attn_decode_partials(
        FULL, L["q_out"], L["kc"], L["vc"], L["bt"], seq_lens, CTX, pps, part_o, part_lse)
        for L in full_layers])
    us_full = time_graph(lambda: [layer_step(L) for L in full_layers])
    kv_full = CTX * KV_BYTES_PER_TOKEN_LAYER
    table = (-(-CTX // PAGE)) * 4
    k2_bytes = kv_full + HQ * D * 4 + table                   # K/V, q, page table
    pair_bytes = kv_full + HQ * D * 4 * 2 + HQ * 4 + table    # + out, sinks
    achieved = k2_bytes / (us_k2 * 1e-6) / 1e9
    pair_achieved = pair_bytes / (us_full * 1e-6) / 1e9

    kv_step = sum(CTX * KV_BYTES_PER_TOKEN_LAYER if L["full"] else WINDOW * KV_BYTES_PER_TOKEN_LAYER
                  for L in layers)
    gbps_step = kv_step / (us_step * 1e-6) / 1e9

    step_traffic = measured_traffic("step_traffic_bytes")
    result = {
        "metric": METRIC,
        "value": round(us_step, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Flint decode attention, all 49 layers (14 full-context NoPE over "
                               "100,000 keys + 35 RoPE sliding over 513 keys), batch 1, one "
                               "decode step incl. norm/RoPE/append of the new token (fused, one "
                               "launch per layer + split merge), bf16 paged KV (16-token pages, "
                               "shuffled), HIP graph",
                   "global_batch": 1, "seq_len": CTX, "layers": LAYERS,
                   "full_layers": len(FULL_LAYERS), "window": WINDOW, "parallelism": "none"},
        # step-level rate over the algorithmic K/V bytes (not a counter
        # reading; the counter-based figure of the dominant kernel is
        # roofline.traffic)
        "hbm_gbps": round(gbps_step, 1),
        "hbm_gbps_kind": "analytic: algorithmic K/V bytes of the step / step time",
        "hbm_frac_of_peak": round(gbps_step / HBM_PEAK_GBPS, 4),
        # the step's HBM bytes by counters (fetch + write of its kernels, from
        # the committed summary while the sources match) over this run's time
        "hbm_gbps_counters": (None if step_traffic is None
                              else round(step_traffic / (us_step * 1e-6) / 1e9, 1)),
        "step_traffic_bytes": step_traffic,
        "kv_bytes_per_step": kv_step,
        "us_per_step_median": round(statistics.median(per), 2),
        "us_per_step_p10": round(float(np.percentile(per, 10)), 2),
        "us_per_step_p90": round(float(np.percentile(per, 90)), 2),
        "us_per_step_unfused": round(us_unfused, 2),
        "us_per_step_append_alone": round(us_append, 2),
        "roofline": {"kernel": "decode_split_kernel (K2, split-K flash decode) of one full "
                               "layer over 100,000 keys, alone: 64 splits x 4 KV heads, launched "
                               "through flint_attn_decode_partials",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(), "us_per_launch": round(us_k2, 2),
                     "bytes_per_launch": k2_bytes, "pages_per_split": pps, "splits": nsplit,
                     "pair": {"kernels": "split kernel (fused norm/RoPE/append) + LSE merge, "
                                         "the two launches of one full-layer "
                                         "flint_attn_decode_step",
                              "us_per_launch": round(us_full, 2), "bytes_per_launch": pair_bytes,
                              "achieved": round(pair_achieved, 1),
                              "frac": round(pair_achieved / HBM_PEAK_GBPS, 4)}},
        "context": "pages' end-to-end figure (model forward + LM head + sampling, 1x GB200, "
                   "vLLM): 2.06 ms/token ~ 485 tok/s at bs1, 100K ctx; not this metric",
    }

    if not args.no_fp8:
        with marker("fp8 cache leg"):
            result["fp8"] = bench_fp8(fl, dev, layers, ws, ones, seq_lens, capture, time_graph,
                                      args.steps, stream, eps)

    if not args.no_moe:
        with marker("MoE leg"):
            result["moe"] = bench_moe(fl, dev, capture, stream)

    if not args.no_configs:
        with marker("other workloads"):
            result["configs"] = bench_configs(fl, dev)
        with marker("machine ceilings"):
            result["ceilings"] = bench_ceilings(dev)
        walk = result["ceilings"]["page_walk"]["us_per_launch"]
        result["roofline"]["loads_alone_us"] = walk
        result["roofline"]["frac_of_loads_alone"] = round(walk / us_k2, 4)
        if "fp8" in result:
            k8 = result["fp8"]["split_kernel"]
            walk8 = result["ceilings"]["page_walk_fp8"]["us_per_launch"]
            k8["loads_alone_us"] = walk8
            k8["frac_of_loads_alone"] = round(walk8 / k8["us_per_launch"], 4)

    if not args.no_prefill:
        result["prefill"] = bench_prefill(fl, dev, stream)

    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_max_abs_err"] = cpu_baseline(layers, eps)
    print(json.dumps(result), flush=True)
    err = result.get("parity_max_abs_err")
    if err is not None and not err <= PARITY_TOL:
        log(f"bench: FAILED parity: max|gpu-oracle| {err:.3e} above {PARITY_TOL}")
        sys.exit(1)


FP8_SCALES = (1.0 / 16, 0.5)


def bench_fp8(fl, dev, layers, ws, ones, seq_lens, capture, time_graph, steps, stream, eps):
    """The same 49-layer step over an fp8 E4M3 KV cache (the pages' fp8
    KV-cache format; 14 KiB per token): fused step graph and the full-layer
    split kernel alone.  Cache codes are drawn uniformly over the E4M3 codes
    below 2.0 (a random sign, no NaN codes); the bf16 leg's q/k/v, tables and
    sinks are reused."""
    import torch
    ks, vs = FP8_SCALES
    FULL8 = fl.layer(window=0, use_rope=0, rms_eps=eps, kv_dtype=fl.FLINT_KV_FP8_E4M3,
                     k_scale=ks, v_scale=vs)
    SLIDE8 = fl.layer(window=WINDOW, use_rope=1, rms_eps=eps, kv_dtype=fl.FLINT_KV_FP8_E4M3,
                      k_scale=ks, v_scale=vs)
    l8 = []
    for l, L in enumerate(layers):
        nb = L["kc"].shape[0]
        l8.append(dict(L, kc=synth.fp8_codes_torch(SEED, (3, l, synth.KC), (nb, HKV, PAGE, D), dev),
                       vc=synth.fp8_codes_torch(SEED, (3, l, synth.VC), (nb, HKV, D, PAGE), dev),
                       out=torch.empty((1, HQ, D), dtype=torch.float32, device=dev)))

    def step8():
        for L in l8:
            fl.flint_attn_decode_step(FULL8 if L["full"] else SLIDE8, L["q_in"], L["k_in"],
                                      L["v_in"], ones, ones, L["slots"], L["kc"], L["vc"],
                                      L["bt"], seq_lens, CTX, L["sinks"], L["out"], workspace=ws)

    step8()
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(L["out"]).all()) for L in l8), "fp8 step output not finite"
    g8 = capture(step8)
    for _ in range(5):
        g8.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(steps):
            g8.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us_step = e0.elapsed_time(e1) * 1e3 / steps
    full8 = [L for L in l8 if L["full"]]
    pps, nsplit = fl.flint_attn_decode_plan(FULL8, 1, CTX)
    part_o = torch.empty((1, nsplit, HQ, D), dtype=torch.float32, device=dev)
    part_lse = torch.empty((1, nsplit, HQ), dtype=torch.float32, device=dev)
    us_k2 = time_graph(lambda: [fl.flint_attn_decode_partials(
        FULL8, L["q_out"], L["kc"], L["vc"], L["bt"], seq_lens, CTX, pps, part_o, part_lse)
        for L in full8])
    kv8 = CTX * KV_BYTES_PER_TOKEN_LAYER // 2
    k2_bytes = kv8 + HQ * D * 4 + (-(-CTX // PAGE)) * 4
    achieved = k2_bytes / (us_k2 * 1e-6) / 1e9
    kv_step = sum((CTX if L["full"] else WINDOW) * KV_BYTES_PER_TOKEN_LAYER // 2 for L in l8)
    log(f"bench: fp8 cache {us_step:.1f} us/step, full-layer split kernel {us_k2:.2f} us "
        f"({achieved:.0f} GB/s)")
    res = {"us_per_step": round(us_step, 2), "k_scale": ks, "v_scale": vs,
           "kv_bytes_per_step": kv_step,
           "hbm_gbps": round(kv_step / (us_step * 1e-6) / 1e9, 1),
           "split_kernel": {"us_per_launch": round(us_k2, 2), "bytes_per_launch": k2_bytes,
                            "achieved": round(achieved, 1),
                            "frac": round(achieved / HBM_PEAK_GBPS, 4)}}
    del l8, g8
    return res


MOE_LAYERS = 8


def bench_moe(fl, dev, capture, stream):
    """Flint's MoE sublayer at 1 and 8 tokens: 8 distinct layers of synthetic
    N(0, 1/fan_in) bf16 weights (1.6 GB each, so the 256 MB last-level cache
    cannot hold a cycle of them), each with its own x ~ N(0,1), in one graph.
    HBM bytes per layer are algorithmic: the router, the gate/up/down rows of
    every distinct expert the tokens selected plus the shared expert, x and
    the outputs."""
    import torch
    M = fl.moe_layer()
    H, E, I, S, K = M.hidden, M.num_experts, M.inter, M.num_shared, M.top_k
    res = {"workload": "MoE sublayer: hidden 2048, 256 routed experts, sigmoid top-6, one "
                       "shared expert, SwiGLU width 512 (a reading); 8 distinct layers",
           "bound": "hbm", "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    ws = torch.empty(fl.flint_moe_workspace_size(M, 8), dtype=torch.uint8, device=dev)
    layers = []
    for l in range(MOE_LAYERS):
        layers.append(dict(
            wr=synth.normal_bf16_bits_torch(SEED, (6, l, 1), (E, H), dev, std=H ** -0.5),
            wgu=synth.normal_bf16_bits_torch(SEED, (6, l, 2), (E + S, 2, I, H), dev,
                                             std=H ** -0.5),
            wd=synth.normal_bf16_bits_torch(SEED, (6, l, 3), (E + S, H, I), dev, std=I ** -0.5)))
    torch.cuda.synchronize()
    expert_bytes = (2 * I * H + H * I) * 2
    for T in (1, 8):
        for l, L in enumerate(layers):
            L["x"] = torch.from_numpy(synth.normal(SEED, (6, l, 4, T), (T, H))).to(dev)
            L["out"] = torch.empty((T, H), dtype=torch.float32, device=dev)
            L["ids"] = torch.empty((T, K), dtype=torch.int32, device=dev)
            L["w"] = torch.empty((T, K), dtype=torch.float32, device=dev)

        def run():
            for L in layers:
                fl.flint_moe_forward(M, L["x"], L["wr"], L["wgu"], L["wd"], out=L["out"],
                                     topk_ids=L["ids"], topk_weights=L["w"], workspace=ws)
        run()
        torch.cuda.synchronize()
        g = capture(run)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * MOE_LAYERS)
        nbytes = [E * H * 2 + (len(np.unique(L["ids"].cpu().numpy())) + S) * expert_bytes
                  + T * H * 4 * 2 + T * K * 8 for L in layers]
        per = float(np.mean(nbytes))
        gbps = per / (us * 1e-6) / 1e9
        finite = all(bool(torch.isfinite(L["out"]).all()) for L in layers)
        log(f"bench: MoE sublayer, {T} token(s): {us:.2f} us/layer, {per / 1e6:.1f} MB, "
            f"{gbps:.0f} GB/s")
        res[f"tokens_{T}"] = {"us_per_layer": round(us, 2), "bytes_per_layer": round(per),
                              "achieved": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                              "finite": finite}
    del layers
    torch.cuda.empty_cache()
    return res


def _time_launches(fn, reps=10, warm=3, warm_ms=30.0):
    """Mean µs per call of fn over reps calls after warm calls and at least
    warm_ms of calls (the core clock ramps up over tens of milliseconds of
    sustained work), with HIP events on the current stream."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    for _ in range(max(warm, math.ceil(warm_ms / max(e0.elapsed_time(e1), 1e-3)))):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def bench_batches(fl, dev):
    """Batched decode: the 64 ragged requests and the small batches at 100K
    context (bench_ragged_64, bench_small_batches), as one JSON object."""
    return {"workload": "batched decode: 64 ragged requests (1024..131072 tokens) on one full "
                        "and one sliding layer; batches of 2..16 at 100K context (fused step; "
                        "full layers over a bf16 and an fp8 cache, sliding over bf16)",
            "unit": "us", "peak_gbps": HBM_PEAK_GBPS, "ragged_64": bench_ragged_64(fl, dev),
            "small_batches_100k": bench_small_batches(fl, dev)}


def bench_configs(fl, dev):
    """The other workloads, each timed in its own graph or launch loop: one
    full layer at 4096 tokens and one sliding layer at 32768 tokens (single-
    layer latency), 64 ragged requests of 1024..131072 tokens, and batches of
    2..16 requests at 100K context."""
    out = bench_single_layers(fl, dev)
    out["ragged_64"] = bench_ragged_64(fl, dev)
    out["small_batches_100k"] = bench_small_batches(fl, dev, sizes=(2, 4, 8))
    return out


SINGLE_LAYER_ROTATION_BYTES = 512 << 20


def bench_single_layers(fl, dev):
    """One decode step of one layer at batch 1: a full (NoPE) layer over a
    4096-token context and a sliding (RoPE, 513-key) layer at a 32768-token
    context, each the fused step (norm/RoPE/append of the new token, then
    attention).  A layer's pages (8.4 MB / 1.05 MB) fit the 256 MB last-level
    cache, so each graph cycles through enough distinct copies -- their own
    caches, page tables and token inputs -- to touch more than 512 MB per
    replay: every step reads its pages from HBM."""
    import torch
    eps = float(np.float32(1e-6))
    stream = torch.cuda.Stream()
    res = {}
    for name, ctx, window in (("full_layer_ctx4096", 4096, 0), ("sliding_layer_ctx32768", 32768,
                                                                 WINDOW)):
        L = fl.layer(window=window, use_rope=1 if window else 0, rms_eps=eps)
        pages = ctx // PAGE
        t = ctx - 1
        kv_bytes = min(ctx, window or ctx) * KV_BYTES_PER_TOKEN_LAYER
        copies = -(-SINGLE_LAYER_ROTATION_BYTES // kv_bytes)
        tabs, nb0 = [], 0
        for c in range(copies):
            if window:
                bt, nb = synth.ring_block_table(SEED, (5, ctx, c, synth.PERM), 1, pages, RING, pages)
            else:
                bt, nb = synth.shuffled_block_table(SEED, (5, ctx, c, synth.PERM), 1, [pages],
                                                    pages)
            tabs.append(np.where(bt >= 0, bt + c * nb, -1).astype(np.int32))
            nb0 = nb
        kc = synth.normal_bf16_bits_torch(SEED, (5, ctx, synth.KC), (copies * nb0, HKV, PAGE, D), dev)
        vc = synth.normal_bf16_bits_torch(SEED, (5, ctx, synth.VC), (copies * nb0, HKV, D, PAGE), dev)
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        bts = [up(b) for b in tabs]
        slots = [up(np.array([int(b[0, t // PAGE]) * PAGE + t % PAGE], np.int32)) for b in tabs]
        q = up(synth.normal(SEED, (5, ctx, synth.Q), (copies, 1, HQ, D)))
        k = up(synth.normal(SEED, (5, ctx, synth.K), (copies, 1, HKV, D)))
        v = up(synth.normal(SEED, (5, ctx, synth.V), (copies, 1, HKV, D)))
        sinks = up(synth.normal(SEED, (5, ctx, synth.SINK), HQ))
        ones = torch.ones(D, dtype=torch.float32, device=dev)
        sl = torch.tensor([ctx], dtype=torch.int32, device=dev)
        out = torch.empty((copies, 1, HQ, D), dtype=torch.float32, device=dev)
        ws = torch.zeros(max(fl.flint_attn_decode_workspace_size(L, 1, ctx), 256), dtype=torch.uint8,
                         device=dev)

        def run():
            for c in range(copies):
                fl.flint_attn_decode_step(L, q[c], k[c], v[c], ones, ones, slots[c], kc, vc, bts[c],
                                          sl, ctx, sinks, out[c], workspace=ws)
        run()
        torch.cuda.synchronize()
        finite = bool(torch.isfinite(out).all())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                run()
            us = _time_launches(g.replay, reps=10) / copies
        nbytes = kv_bytes + HQ * D * 4 * 2 + HKV * D * 4 * 2 + HQ * 4 + (pages if not window
                                                                         else RING) * 4
        gbps = nbytes / us / 1e3
        res[name] = {"us_per_step": round(us, 2), "bytes_per_step": nbytes,
                     "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "copies_cycled": copies, "plan": list(fl.flint_attn_decode_plan(L, 1, ctx)),
                     "finite": finite}
        log(f"bench: one {name} step {us:.2f} us ({gbps:.0f} GB/s), {copies} copies cycled")
        del kc, vc, g
        torch.cuda.empty_cache()
    return res


def bench_ragged_64(fl, dev):
    """64 requests with lengths uniform in [1024, 131072] (seeded), pages in one
    random physical order, one full and one sliding layer, flint_attn_decode
    on a normalised q; algorithmic bytes from the drawn lengths."""
    import torch
    eps = float(np.float32(1e-6))
    FULL = fl.layer(window=0, use_rope=0, rms_eps=eps)
    SLIDE = fl.layer(window=WINDOW, use_rope=1, rms_eps=eps)
    B = 64
    lens = synth.uniform_ints(SEED, (3, 1), B, 1024, 131072).astype(np.int32)
    maxlen = int(lens.max())
    stride = -(-maxlen // PAGE)
    q = torch.randn((B, HQ, D), device=dev, generator=torch.Generator(device=dev).manual_seed(3))
    sinks = torch.randn(HQ, device=dev, generator=torch.Generator(device=dev).manual_seed(4))
    out = torch.empty((B, HQ, D), device=dev)
    sl = torch.from_numpy(lens).to(dev)
    ragged = {"requests": B, "min_len": int(lens.min()), "max_len": maxlen,
              "tokens": int(lens.sum())}
    for kind, L in (("full", FULL), ("sliding", SLIDE)):
        if kind == "full":
            bt, nb = synth.shuffled_block_table(SEED, (3, 2), B, [-(-int(x) // PAGE) for x in lens],
                                                stride)
            kv_bytes = int(lens.sum()) * KV_BYTES_PER_TOKEN_LAYER
        else:
            bt, nb = synth.ring_block_table(SEED, (3, 2), B, stride, RING, stride)
            kv_bytes = int(np.minimum(lens, WINDOW).sum()) * KV_BYTES_PER_TOKEN_LAYER
        kc = synth.normal_bf16_bits_torch(SEED, (3, 3, kind == "full"), (nb, HKV, PAGE, D), dev)
        vc = synth.normal_bf16_bits_torch(SEED, (3, 4, kind == "full"), (nb, HKV, D, PAGE), dev)
        bt_d = torch.from_numpy(np.ascontiguousarray(bt)).to(dev)
        ws = torch.zeros(max(fl.flint_attn_decode_workspace_size(L, B, maxlen), 256),
                         dtype=torch.uint8, device=dev)
        us = _time_launches(lambda: fl.flint_attn_decode(L, q, kc, vc, bt_d, sl, maxlen, sinks, out,
                                                         workspace=ws))
        assert torch.isfinite(out).all(), "non-finite output"
        ragged[kind] = {"us": round(us, 1), "kv_bytes": kv_bytes,
                        "gbps": round(kv_bytes / us / 1e3, 1),
                        "frac": round(kv_bytes / us / 1e3 / HBM_PEAK_GBPS, 4),
                        "plan": list(fl.flint_attn_decode_plan(L, B, maxlen))}
        log(f"bench: 64 ragged requests, {kind} layer: {us:.1f} us, {kv_bytes / 1e9:.3f} GB, "
            f"{kv_bytes / us / 1e3:.0f} GB/s")
        del kc, vc
    torch.cuda.empty_cache()
    return ragged


def bench_small_batches(fl, dev, sizes=(2, 4, 8, 16)):
    """B = 2, 4, 8, 16 (or `sizes`) requests at 100K context, one fused step of a full
    layer (bf16 and fp8 cache) and of a sliding layer each, in a graph of 6
    (full) or 20 (sliding) distinct layers so that no layer's pages stay in
    the caches between replays."""
    import torch
    eps = float(np.float32(1e-6))
    FULL = fl.layer(window=0, use_rope=0, rms_eps=eps)
    SLIDE = fl.layer(window=WINDOW, use_rope=1, rms_eps=eps)
    ones = torch.ones(D, dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    small = {}
    pages = -(-CTX // PAGE)
    t = CTX - 1
    FULL8 = fl.layer(window=0, use_rope=0, rms_eps=eps, kv_dtype=fl.FLINT_KV_FP8_E4M3,
                     k_scale=FP8_SCALES[0], v_scale=FP8_SCALES[1])
    for Bs in sizes:
        row = {}
        for kind, L in (("full", FULL), ("sliding", SLIDE), ("full_fp8", FULL8)):
            nlay = 20 if kind == "sliding" else 6
            lay = []
            for l in range(nlay):
                if kind == "full_fp8":
                    bt, nb = synth.shuffled_block_table(SEED, (9, Bs, l), Bs, [pages] * Bs, pages)
                    kc = synth.fp8_codes_torch(SEED, (9, Bs, l, 1), (nb, HKV, PAGE, D), dev)
                    vc = synth.fp8_codes_torch(SEED, (9, Bs, l, 2), (nb, HKV, D, PAGE), dev)
                    slots = np.array([int(bt[b, t // PAGE]) * PAGE + t % PAGE for b in range(Bs)],
                                     np.int32)
                    lay.append((torch.from_numpy(np.ascontiguousarray(bt)).to(dev), kc, vc,
                                torch.from_numpy(slots).to(dev)))
                    continue
                if kind == "full":
                    bt, nb = synth.shuffled_block_table(SEED, (8, Bs, l), Bs, [pages] * Bs, pages)
                else:
                    bt, nb = synth.ring_block_table(SEED, (8, Bs, l), Bs, pages, RING, pages)
                kc = synth.normal_bf16_bits_torch(SEED, (8, Bs, l, 1), (nb, HKV, PAGE, D), dev)
                vc = synth.normal_bf16_bits_torch(SEED, (8, Bs, l, 2), (nb, HKV, D, PAGE), dev)
                slots = np.array([int(bt[b, t // PAGE]) * PAGE + t % PAGE for b in range(Bs)],
                                 np.int32)
                lay.append((torch.from_numpy(np.ascontiguousarray(bt)).to(dev), kc, vc,
                            torch.from_numpy(slots).to(dev)))
            gen = torch.Generator(device=dev).manual_seed(5)
            qi = torch.randn((Bs, HQ, D), device=dev, generator=gen)
            ki = torch.randn((Bs, HKV, D), device=dev, generator=gen)
            vi = torch.randn((Bs, HKV, D), device=dev, generator=gen)
            sk = torch.randn(HQ, device=dev, generator=gen)
            sl = torch.full((Bs,), CTX, dtype=torch.int32, device=dev)
            o = torch.empty((Bs, HQ, D), device=dev)
            ws = torch.zeros(max(fl.flint_attn_decode_workspace_size(L, Bs, CTX), 256),
                             dtype=torch.uint8, device=dev)

            def run_all():
                for bt_d, kc, vc, slots in lay:
                    fl.flint_attn_decode_step(L, qi, ki, vi, ones, ones, slots, kc, vc, bt_d, sl, CTX,
                                              sk, o, workspace=ws)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    run_all()
            with torch.cuda.stream(stream):
                us = _time_launches(g.replay, reps=20) / nlay
            kv_bytes = Bs * (WINDOW if kind == "sliding" else CTX) * KV_BYTES_PER_TOKEN_LAYER
            if kind == "full_fp8":
                kv_bytes //= 2
            row[kind] = {"us_per_layer": round(us, 2), "gbps": round(kv_bytes / us / 1e3, 1),
                         "plan": list(fl.flint_attn_decode_plan(L, Bs, CTX))}
            del lay, g
            torch.cuda.empty_cache()
        small[f"B{Bs}"] = row
        log(f"bench: B={Bs} at 100K: full layer {row['full']['us_per_layer']:.1f} us "
            f"({row['full']['gbps']:.0f} GB/s), sliding layer {row['sliding']['us_per_layer']:.2f} us, "
            f"fp8 full layer {row['full_fp8']['us_per_layer']:.1f} us "
            f"({row['full_fp8']['gbps']:.0f} GB/s)")
    return small


def _ceiling_lib():
    """libflint_ceiling.so: the measurement kernels of the ceilings leg."""
    import ctypes as C

    import full_gqa_decode_amd as fl
    fl.lib()  # torch's HIP runtime first; raises if nothing was built
    from full_gqa_decode_amd import build as fb
    if not os.path.exists(fb.SO_CEILING):
        raise RuntimeError(f"{fb.SO_CEILING} is missing: build it with "
                           "`python -m full_gqa_decode_amd.build`")
    L = C.CDLL(fb.SO_CEILING)
    P, I = C.c_void_p, C.c_int
    L.flint_ceiling_stream_bytes.restype = C.c_long
    L.flint_ceiling_stream_read.argtypes = [I, I, P, P, P]
    L.flint_ceiling_page_walk.argtypes = [P, P, P, I, I, I, I, P, P]
    L.flint_ceiling_empty.argtypes = [P]
    L.flint_ceiling_atomics.argtypes = [P, I, I, P]
    return L


def bench_ceilings(dev):
    """Machine ceilings the decode kernels are compared against, measured with
    the kernels of libflint_ceiling.so (HIP graphs, events on the graph's
    stream):
      graph_launch_us  one empty kernel inside a graph (35 back to back);
      stream_read      every byte of 14 distinct ~201 MB buffers, in 4 KiB
                       chunks at pseudo-random offsets, nontemporal and
                       ordinary loads (the access shape of a paged cache);
      page_walk        the split-K kernel's loads alone in its own shape (64
                       splits x 4 KV heads, 8 waves, a shuffled page table,
                       6250 pages of 4 KiB K + 4 KiB V per head: one 100K
                       full layer), 14 distinct layers; page_walk_fp8 the
                       same over 2 KiB fp8 tiles;
      atomics          agent-scope atomic adds on one hot counter per us;
    plus torch's device-to-device copy of 204.8 MB (bytes read + written)."""
    import torch
    L = _ceiling_lib()
    stream = torch.cuda.Stream()

    def graph_time(fn, n, reps=10):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                fn()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * n)

    def ok(rc):
        if rc != 0:
            raise RuntimeError("ceiling kernel launch failed")

    sid = lambda: stream.cuda_stream
    us_launch = graph_time(lambda: [ok(L.flint_ceiling_empty(sid())) for _ in range(35)], 35, 20)

    nreg = 14
    rb = L.flint_ceiling_stream_bytes()
    buf = torch.empty(nreg * rb, dtype=torch.uint8, device=dev)
    out = torch.empty(256 * 4 * 512, dtype=torch.int32, device=dev)
    stream_read = {}
    for nt in (1, 0):
        us = graph_time(lambda: [ok(L.flint_ceiling_stream_read(4, nt, buf.data_ptr() + i * rb,
                                                                out.data_ptr(), sid()))
                                 for i in range(nreg)], nreg)
        stream_read["nontemporal" if nt else "ordinary"] = {
            "us_per_launch": round(us, 2), "gbps": round(rb / us / 1e3, 1),
            "frac": round(rb / us / 1e3 / HBM_PEAK_GBPS, 4)}
    del buf

    pages, heads, pps = -(-CTX // PAGE), HKV, 98
    tb = pages * heads * 4096
    k = [torch.empty(tb, dtype=torch.uint8, device=dev) for _ in range(nreg)]
    v = [torch.empty(tb, dtype=torch.uint8, device=dev) for _ in range(nreg)]
    gen = torch.Generator().manual_seed(SEED)
    tables = [torch.randperm(pages, generator=gen).to(torch.int32).to(dev) for _ in range(nreg)]
    us_walk = graph_time(lambda: [ok(L.flint_ceiling_page_walk(
        k[i].data_ptr(), v[i].data_ptr(), tables[i].data_ptr(), pages, heads, pps, 0,
        out.data_ptr(), sid())) for i in range(nreg)], nreg)
    walk_bytes = 2 * tb
    # the same walk over an fp8 cache's 2 KiB tiles (the first half of each buffer)
    us_walk8 = graph_time(lambda: [ok(L.flint_ceiling_page_walk(
        k[i].data_ptr(), v[i].data_ptr(), tables[i].data_ptr(), pages, heads, pps, 1,
        out.data_ptr(), sid())) for i in range(nreg)], nreg)
    walk8_bytes = tb
    del k, v

    ctr = torch.zeros(1, dtype=torch.int32, device=dev)
    wgs, per_wave = 1024, 16
    us_atom = graph_time(lambda: ok(L.flint_ceiling_atomics(ctr.data_ptr(), wgs, per_wave, sid())),
                         1, 5)
    n_atom = wgs * 4 * per_wave
    assert int(ctr.item()) == n_atom * (3 + 5), "atomic count"  # 3 warm-up + 5 timed replays

    nbytes = CTX * KV_BYTES_PER_TOKEN_LAYER
    src = [torch.ones(nbytes // 4, dtype=torch.float32, device=dev) for _ in range(nreg)]
    dst = [torch.empty_like(x) for x in src]

    def copy_all():
        for a, b in zip(dst, src):
            a.copy_(b)
    us_copy = _time_launches(copy_all, reps=5) / len(src)
    gbps = 2 * nbytes / us_copy / 1e3
    del src, dst
    torch.cuda.empty_cache()
    res = {"graph_launch_us": round(us_launch, 3),
           "stream_read": dict(stream_read, bytes_per_launch=rb, chunk_kib=4),
           "page_walk": {"us_per_launch": round(us_walk, 2), "bytes_per_launch": walk_bytes,
                         "gbps": round(walk_bytes / us_walk / 1e3, 1),
                         "frac": round(walk_bytes / us_walk / 1e3 / HBM_PEAK_GBPS, 4),
                         "pages_per_split": pps, "splits": -(-pages // pps)},
           "page_walk_fp8": {"us_per_launch": round(us_walk8, 2), "bytes_per_launch": walk8_bytes,
                             "gbps": round(walk8_bytes / us_walk8 / 1e3, 1),
                             "frac": round(walk8_bytes / us_walk8 / 1e3 / HBM_PEAK_GBPS, 4)},
           "atomics_per_us": round(n_atom / us_atom, 1),
           "copy_204_8MB_us": round(us_copy, 2), "copy_gbps_read_plus_write": round(gbps, 1)}
    log(f"bench: ceilings: graph launch {us_launch:.2f} us; random 4 KiB chunks "
        f"{stream_read['nontemporal']['gbps']:.0f} GB/s nontemporal, "
        f"{stream_read['ordinary']['gbps']:.0f} GB/s ordinary; split-kernel loads alone "
        f"{us_walk:.2f} us ({walk_bytes / us_walk / 1e3:.0f} GB/s), over an fp8 cache "
        f"{us_walk8:.2f} us ({walk8_bytes / us_walk8 / 1e3:.0f} GB/s); "
        f"{n_atom / us_atom:.0f} atomics/us on one counter; copy {gbps:.0f} GB/s (read + write)")
    return res


STAMP_NS = 10.0   # s_memrealtime counts at 100 MHz


def bench_stamps(dev):
    """Per-wave phase stamps (s_memrealtime) from the instrumented library:
    the 32,768-token prefill of a sliding and of a full layer (per work item:
    start-up, loop, epilogue, and the gaps between a workgroup's items) and one
    fused sliding-layer decode step at batch 1 (per slice workgroup: scalar
    inputs, start-up before the page loads, the pages, the epilogue)."""
    import ctypes
    import torch
    import full_gqa_decode_amd as fl
    path = os.path.join(ROOT, "full_gqa_decode_amd", "libflint_stamps.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: python -m full_gqa_decode_amd.build --stamps")
    fl.LIB_PATH = path
    lib = fl.lib()
    lib.flint_stamps_prefill.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.flint_stamps_slice.argtypes = [ctypes.c_void_p, ctypes.c_size_t]

    def read(fn, shape):
        buf = np.zeros(int(np.prod(shape)), np.uint64)
        assert fn(buf.ctypes.data, buf.nbytes) == 0
        return buf.reshape(shape).astype(np.int64)

    def stats(x):
        return {"mean": round(float(np.mean(x)), 3), "median": round(float(np.median(x)), 3)}

    out = {"clock": "s_memrealtime, 100 MHz; µs"}
    items, waves = 4096, 8
    for name, window in (("prefill_sliding_layer_32k", WINDOW), ("prefill_full_layer_32k", 0)):
        prefill_leg(fl, dev, window=window)
        torch.cuda.synchronize()
        st = read(lib.flint_stamps_prefill, (8192, waves, 8))[:items]
        t = (st[:, :, :6] - st[:, :, 0].min()) * STAMP_NS / 1e3
        npairs = st[:, 0, 7]
        ph = np.diff(t, axis=2).mean(1)   # per item, mean over waves
        grid = 256
        wg = st[:, 0, 6] >> 16            # the workgroup that ran the item
        start, end = t[:, :, 0].min(1), t[:, :, 5].max(1)
        gaps, ends = [], []
        for g in range(grid):
            idx = np.flatnonzero(wg == g)
            o = idx[np.argsort(start[idx])]
            gaps += list(start[o[1:]] - end[o[:-1]])
            ends.append(end[idx].max())
        out[name] = {
            "items": items, "workgroups": grid,
            "entry_to_lengths": stats(ph[:, 0]), "lengths_to_pair0_staged": stats(ph[:, 1]),
            "pair0_to_loop": stats(ph[:, 2]), "loop": stats(ph[:, 3]),
            "loop_per_pair": stats(ph[:, 3] / np.maximum(npairs, 1)),
            "epilogue": stats(ph[:, 4]), "gap_between_items": stats(np.array(gaps)),
            "workgroup_end_min_max": [round(float(min(ends)), 1), round(float(max(ends)), 1)],
            "workgroup_end_mean": round(float(np.mean(ends)), 1),
            "items_per_workgroup_min_max": [int(np.bincount(wg, minlength=grid).min()),
                                            int(np.bincount(wg, minlength=grid).max())]}
    # one fused sliding-layer step at batch 1 (32 slice workgroups)
    eps = float(np.float32(1e-6))
    L = fl.layer(window=WINDOW, use_rope=1, rms_eps=eps)
    ctx = 32768
    bt, nb = synth.ring_block_table(SEED, (6, ctx, synth.PERM), 1, ctx // PAGE, RING, ctx // PAGE)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    kc = synth.normal_bf16_bits_torch(SEED, (6, ctx, synth.KC), (nb, HKV, PAGE, D), dev)
    vc = synth.normal_bf16_bits_torch(SEED, (6, ctx, synth.VC), (nb, HKV, D, PAGE), dev)
    t_new = ctx - 1
    slots = up(np.array([int(bt[0, t_new // PAGE]) * PAGE + t_new % PAGE], np.int32))
    q = up(synth.normal(SEED, (6, ctx, synth.Q), (1, HQ, D)))
    k = up(synth.normal(SEED, (6, ctx, synth.K), (1, HKV, D)))
    v = up(synth.normal(SEED, (6, ctx, synth.V), (1, HKV, D)))
    sinks = up(synth.normal(SEED, (6, ctx, synth.SINK), HQ))
    ones = torch.ones(D, dtype=torch.float32, device=dev)
    sl = torch.tensor([ctx], dtype=torch.int32, device=dev)
    o = torch.empty((1, HQ, D), dtype=torch.float32, device=dev)
    btd = up(bt)
    for _ in range(3):   # the last call's stamps are read
        fl.flint_attn_decode_step(L, q, k, v, ones, ones, slots, kc, vc, btd, sl, ctx, sinks, o)
    torch.cuda.synchronize()
    nwg = HKV * 8
    st = read(lib.flint_stamps_slice, (1024, 16, 8))[:nwg, :8]
    t = (st[:, :, :5] - st[:, :, 0].min()) * STAMP_NS / 1e3
    ph = np.diff(t, axis=2).mean(1)
    out["decode_sliding_layer_fused_bs1"] = {
        "workgroups": nwg, "entry_to_scalars": stats(ph[:, 0]),
        "scalars_to_page_issue": stats(ph[:, 1]), "pages": stats(ph[:, 2]),
        "epilogue": stats(ph[:, 3]), "span": round(float(t[:, :, 4].max()), 3)}
    return out


def copy_probe(dev):
    """A plain copy of COPY_PROBE_BYTES (read once, written once), three times:
    its FETCH_SIZE and WRITE_SIZE per dispatch, against the known byte count,
    give the scale factor of those counters."""
    import torch
    n = COPY_PROBE_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: copy probe {COPY_PROBE_BYTES} bytes x 3 done")


def bench_prefill(fl, dev, stream):
    """Causal prefill of a 32,768-token prompt on one full layer (MFMA-bound)
    and on one sliding layer (window 513, RoPE; near the balance of MFMA and
    HBM): append all tokens (bf16 q), then time the attention kernel alone."""
    full = prefill_leg(fl, dev, window=0)
    full["sliding"] = prefill_leg(fl, dev, window=WINDOW)
    full["fp8"] = prefill_leg(fl, dev, window=0, fp8=True)
    return full


PREFILL_WARM_MS = 60.0
PREFILL_TIMED_MS = 20.0


def prefill_leg(fl, dev, window, fp8=False):
    with marker(f"prefill leg: 32768 tokens, window {window}{', fp8 cache' if fp8 else ''}"):
        return _prefill_leg(fl, dev, window, fp8)


def _prefill_leg(fl, dev, window, fp8=False):
    import torch
    T = 32768
    eps = float(np.float32(1e-6))
    kv = dict(kv_dtype=fl.FLINT_KV_FP8_E4M3, k_scale=FP8_SCALES[0], v_scale=FP8_SCALES[1]) \
        if fp8 else {}
    L = fl.layer(window=window, use_rope=1 if window else 0, rms_eps=eps, **kv)
    pages = T // PAGE
    bt, nb = synth.shuffled_block_table(SEED, (4, 0, synth.PERM), 1, [pages], pages)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q = up(synth.normal(SEED, (4, 0, synth.Q), (T, HQ, D)))
    k = up(synth.normal(SEED, (4, 0, synth.K), (T, HKV, D)))
    v = up(synth.normal(SEED, (4, 0, synth.V), (T, HKV, D)))
    sinks = up(synth.normal(SEED, (4, 0, synth.SINK), HQ))
    slots = up((bt[0, np.arange(T) // PAGE].astype(np.int64) * PAGE + np.arange(T) % PAGE)
               .astype(np.int32))
    pos = up(np.arange(T, dtype=np.int32))
    ones = torch.ones(D, dtype=torch.float32, device=dev)
    cdt = torch.uint8 if fp8 else torch.int16
    kc = torch.empty((nb, HKV, PAGE, D), dtype=cdt, device=dev)
    vc = torch.empty((nb, HKV, D, PAGE), dtype=cdt, device=dev)
    qb = torch.empty((T, HQ, D), dtype=torch.int16, device=dev)
    fl.flint_qk_norm_rope_append(L, q, k, v, ones, ones, pos, slots, qb, kc, vc)
    out = torch.empty((T, HQ, D), dtype=torch.float32, device=dev)
    cu = up(np.array([0, T], np.int32))
    sl = up(np.array([T], np.int32))
    btd = up(bt)
    ws = torch.zeros(max(8, fl.flint_attn_prefill_workspace_size(L, 1, T, T)), dtype=torch.uint8,
                     device=dev)
    run = lambda: fl.flint_attn_prefill(L, qb, cu, T, kc, vc, btd, sl, T, sinks, out, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    first_ms = e0.elapsed_time(e1)
    # The core clock ramps up over tens of milliseconds of sustained work: a
    # single 0.6 ms sliding-layer launch after idle runs at ~1.9 GHz instead
    # of ~2.35.  Warm up for PREFILL_WARM_MS of launches, then time at least
    # PREFILL_TIMED_MS of them.
    for _ in range(max(2, math.ceil(PREFILL_WARM_MS / first_ms))):
        run()
    reps = max(3, math.ceil(PREFILL_TIMED_MS / first_ms))
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # (query, key) pairs the causal (windowed) mask keeps, 4*D flops each
    i = np.arange(T, dtype=np.int64)
    pairs = int(np.minimum(i + 1, window).sum()) if window else T * (T + 1) // 2
    flops = 4.0 * D * pairs * HQ
    tflops = flops / (ms * 1e-3) / 1e12
    # HBM bytes the kernel must move: q (bf16) in, out (fp32), K/V read once
    nbytes = T * HQ * D * 2 + T * HQ * D * 4 + T * KV_BYTES_PER_TOKEN_LAYER // (2 if fp8 else 1)
    gbps = nbytes / (ms * 1e-3) / 1e9
    kind = f"sliding layer (window {window}, RoPE)" if window else "full layer"
    if fp8:
        kind += ", fp8 E4M3 cache"
    log(f"bench: prefill 32768 {kind} {ms:.2f} ms, {tflops:.1f} TFLOP/s, {gbps:.0f} GB/s")
    res = {"workload": f"causal prefill, 32,768-token prompt, one {kind} (32 q / 4 KV heads)",
           "ms": round(ms, 3), "flops": flops, "tflops": round(tflops, 1),
           "bound": "mfma", "peak_tflops": BF16_DENSE_TFLOPS,
           "mfma_frac": round(tflops / BF16_DENSE_TFLOPS, 4),
           "finite": bool(torch.isfinite(out).all().item())}
    if window:
        res.update({"bound": "mfma+hbm", "hbm_bytes": nbytes, "hbm_gbps": round(gbps, 1),
                    "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)})
    return res


def cpu_baseline(layers, eps):
    """The fp64 oracle on the host cores, over the same 49-layer step (its own
    append of the new token, then attention), timed; its outputs also give the
    step's parity check."""
    import oracle
    oracle.build(force=False)
    t = CTX - 1
    nthreads = oracle.default_threads()
    Lf = oracle.layer(window=0, use_rope=0, eps=eps)
    Ls = oracle.layer(window=WINDOW, use_rope=1, eps=eps)
    ones = np.ones(D, np.float32)
    worst = 0.0
    t0 = time.perf_counter()
    for L in layers:   # host copies of the drawn caches (pristine: taken before any append)
        L["host"]["kc"] = L["kc0"]
        L["host"]["vc"] = L["vc0"]
    for L in layers:
        h = L["host"]
        Lo = Lf if L["full"] else Ls
        kc, vc = h["kc"], h["vc"]   # the new token is appended in place
        qh = oracle.append(Lo, h["q"], h["k"], h["v"], ones, ones, np.array([t], np.int32),
                           np.array([h["slot"]], np.int32), kc, vc)
        ref = oracle.attn_decode(Lo, qh, kc, vc, h["bt"], np.array([CTX], np.int32), h["sinks"],
                                 nthreads=nthreads)
        L["ref"] = ref
    secs = time.perf_counter() - t0
    for L in layers:
        worst = max(worst, float(np.max(np.abs(L["out"].cpu().numpy().astype(np.float64)
                                               - L["ref"]))))
    # one thread: the attention of one full and one sliding layer (the append is
    # negligible beside it), extrapolated to the step and labelled as such
    one = {}
    for full in (True, False):
        L = next(L for L in layers if L["full"] == full)
        h = L["host"]
        Lo = Lf if full else Ls
        qh = oracle.append(Lo, h["q"], h["k"], h["v"], ones, ones, np.array([t], np.int32),
                           np.array([-1], np.int32), h["kc"], h["vc"])
        t1 = time.perf_counter()
        oracle.attn_decode(Lo, qh, h["kc"], h["vc"], h["bt"], np.array([CTX], np.int32),
                           h["sinks"], nthreads=1)
        one["full" if full else "sliding"] = (time.perf_counter() - t1) * 1e6
    n_full = len(FULL_LAYERS)
    single = {"us_full_layer": round(one["full"], 1), "us_sliding_layer": round(one["sliding"], 1),
              "us_per_step_extrapolated": round(n_full * one["full"] +
                                                (LAYERS - n_full) * one["sliding"], 1),
              "threads": 1}
    log(f"bench: oracle step {secs:.2f} s on {nthreads} threads; one thread: full layer "
        f"{one['full'] / 1e6:.2f} s, sliding layer {one['sliding'] / 1e3:.1f} ms; "
        f"max|gpu-oracle| {worst:.2e}")
    return ({"value": round(secs * 1e6, 1), "unit": "us/step", "cores": nthreads,
             "kind": "oracle",
             "sample": "the whole 49-layer step (append of the new token + attention for all "
                       "32 heads of every layer), fp64, once",
             "single_thread": single}, worst)


if __name__ == "__main__":
    main()
