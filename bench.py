#!/usr/bin/env python3
"""Benchmark of one MLA decode step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic inputs:
    mla_absorb_q -> mla_decode_attn (split-KV attention + LSE combine)
    -> mla_up_proj_v
with every input already resident in HBM.  The latent cache (>= 768 MB in
total) and W^UK / W^UV are replicated and the replicas are used round-robin,
so each step reads its cache and weights from HBM rather than from the
256 MB memory-side cache.

Prints ONE JSON line.  `value` is decode tokens/s (B*T query tokens per
step / step time).  `roofline` describes the dominant kernel (the attention
kernel), timed with HIP events on the stream it runs on; `cpu_baseline`
times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
DEFAULT_WORKLOAD = "v2_b32_l4k_bf16"
ATTN_PER_GRAPH = 20                     # attention calls captured per graph
STEPS_PER_GRAPH = 10                    # decode steps captured per graph
COPY_PROBE_BYTES = 512 * 2 ** 20        # calibration copy of the traffic probe
COPY_CEILING_BYTES = 2 ** 30            # plain device copy reported as the practical ceiling
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
_CSRC = os.path.join(ROOT, "head_latent_attention_11_amd", "csrc")
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in
                  ("decode_mfma.hip", "decode_mfma_asm.inc", "decode_small.hip",
                   "kernels_misc.hip", "mla_common.hpp", "plan_device.hpp", "mla_api.hip")]
LITE_WORKLOAD = "v2lite_b64_l8k_bf16"   # DeepSeek-V2-Lite shapes (16 heads)


def algorithmic(w, seq_lens):
    """Bytes and flops the absorbed method must move / compute per attention
    launch: the latent cache rows, the absorbed queries, the latent output
    and the LSE; 2 * rows * L * (d_c + d_h^R + d_c) flops per sequence."""
    D = w.d_latent + w.d_rope
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[w.kv_dtype]
    row_bytes = D * esz + (4 if w.kv_dtype == "fp8" else 0)
    total_tokens = int(sum(seq_lens))
    q_bytes = w.batch * w.q_tokens * w.n_heads * D * (4 if w.q_dtype == "f32" else 2)
    out_bytes = w.batch * w.q_tokens * w.n_heads * (w.d_latent + 1) * 4
    cache_bytes = total_tokens * row_bytes
    flops = 0
    for L in seq_lens:
        # causal: query tau sees L - T + tau + 1 tokens
        for tau in range(w.q_tokens):
            n = L - w.q_tokens + tau + 1
            flops += 2 * w.n_heads * n * (D + w.d_latent)
    return cache_bytes, q_bytes + out_bytes, flops


def kernel_sources_sha256() -> str:
    """Digest of the attention kernels' sources (decode + combine): counters
    taken on other sources do not describe the kernels being timed."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for_current_kernel(workload: str):
    """HBM traffic per attention call measured with rocprofv3 counters
    (bench_traffic.py), if taken on this workload and on the current kernel
    sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        if rec.get("workload") == workload and rec.get("sources_sha256") == kernel_sources_sha256():
            return rec
    except (OSError, ValueError):
        pass
    return None


def cpu_baseline(w, gen, budget_s: float):
    """Time the CPU oracle (as it is) on a bounded sample: whole-length
    (sequence, head) evaluations, scaled to the full step."""
    from threadpoolctl import threadpool_info

    from oracle import mla as omla
    t0 = time.perf_counter()
    n_eval = 0
    seqs = list(range(w.batch))
    h = 0
    b_i = 0
    d = None
    cur_b = None
    while True:
        b = seqs[b_i % len(seqs)]
        if b != cur_b:
            d = omla.logical_inputs(gen, w, seqs=[b])
            cur_b = b
        omla.decode(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["c_rows"], d["kr_rows"],
                    d["row_offsets"], d["seq_lens"], w.q_tokens, seqs=[b], heads=[h])
        n_eval += 1
        h += 1
        if h == w.n_heads:
            h = 0
            b_i += 1
        if time.perf_counter() - t0 >= budget_s and n_eval >= 2:
            break
    elapsed = time.perf_counter() - t0
    per_eval = elapsed / n_eval                       # one (sequence, head) incl. all T
    full_step = per_eval * w.batch * w.n_heads
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": w.batch * w.q_tokens / full_step,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{n_eval} whole-length (sequence, head) evaluations of the literal "
                   f"fp64 oracle in {elapsed:.1f} s, scaled to B*n_h = "
                   f"{w.batch * w.n_heads} evaluations per step"),
    }


def time_out_proj(w, buf, stream):
    """The attention output projection u = W^O [o_1; ...; o_{n_h}] that follows
    the step (not part of it): its own HIP-event time over graph replays of 20
    calls on the step's o (as bf16), W^O [d_model, n_h d_h] bf16 drawn by the
    input generator and replicated so that the memory-side cache cannot hold
    it.  Bound: streaming W^O from HBM."""
    import numpy as np
    import torch
    from head_latent_attention_11_amd import binding as B
    from mla_inputs import output_weights
    K = w.n_heads * w.d_head
    w_bytes = w.d_model * K * 2
    reps = max(2, -(-512 * 2 ** 20 // w_bytes))
    w0 = torch.from_numpy(output_weights(w).view(np.int16)).to("cuda").view(torch.bfloat16)
    w_o = [w0] + [w0.clone() for _ in range(reps - 1)]
    o = buf.o.to(torch.bfloat16).contiguous()
    u = torch.empty((buf.n_tok, w.d_model), dtype=torch.float32, device="cuda")
    wsb = B.out_proj_workspace_size(buf.dims, w.d_model, buf.n_tok, B.BF16)
    ws = torch.empty(((wsb + 15) // 16 * 4,), dtype=torch.float32, device="cuda") if wsb else None
    calls = 20

    def fn():
        for i in range(calls):
            B.out_proj(buf.dims, o, w_o[i % reps], w.d_model, u, buf.n_tok, ws, wsb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / (5 * calls)
    byts = w_bytes + buf.n_tok * K * 2 + buf.n_tok * w.d_model * 4
    res = {"us": round(t * 1e6, 2), "d_model": w.d_model, "n_tokens": buf.n_tok,
           "bytes_alg": byts, "achieved_GBps": round(byts / t / 1e9, 1),
           "frac_hbm": round(byts / t / 1e9 / HBM_PEAK_GBPS, 4)}
    del w_o, g
    return res


def time_kv_produce(w, buf, stream):
    """The cache producer that precedes the step (not part of it): the rows
    [RMSNorm(W^DKV h) ; RoPE(W^KR h)] of the step's B*T new tokens appended
    into a cache of the step's format (a scratch one, so the step's cache is
    left as it is); HIP-event time over graph replays of 20 calls."""
    import torch
    from head_latent_attention_11_amd import binding as B
    from head_latent_attention_11_amd.runner import to_device
    from mla_inputs import producer_inputs
    n = buf.n_tok
    inp = producer_inputs(w, n)
    D = w.d_latent + w.d_rope
    h = to_device(inp["h"], "bf16", "cuda")
    wk = to_device(inp["w_dkv_kr"], "bf16", "cuda")
    gain = torch.from_numpy(inp["gain"]).cuda()
    seq = torch.arange(n, dtype=torch.int32, device="cuda") // w.q_tokens
    pos = (torch.arange(n, dtype=torch.int32, device="cuda") % w.q_tokens)
    B_, ml = w.batch, w.q_tokens
    if w.kv_dtype == "fp8":
        cache = torch.zeros((B_ * ml, D), dtype=torch.uint8, device="cuda")
        scale = torch.zeros((B_ * ml,), dtype=torch.float32, device="cuda")
    else:
        cache = torch.zeros((B_ * ml, D), dtype=torch.bfloat16, device="cuda")
        scale = None
    wsb = B.kv_produce_workspace_size(buf.dims, w.d_model, n)
    ws = torch.empty(((wsb + 15) // 16 * 4,), dtype=torch.float32, device="cuda")
    calls = 20

    def fn():
        for _ in range(calls):
            B.kv_produce(buf.dims, h, w.d_model, wk, gain, 1e-6, seq, pos, None, B_, 0, ml,
                         B_ * ml, True, cache, scale, n, ws, wsb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / (5 * calls)
    byts = D * w.d_model * 2 + n * w.d_model * 2 + n * (D * (1 if w.kv_dtype == "fp8" else 2))
    return {"us": round(t * 1e6, 2), "d_model": w.d_model, "n_rows": n, "bytes_alg": byts,
            "achieved_GBps": round(byts / t / 1e9, 1),
            "frac_hbm": round(byts / t / 1e9 / HBM_PEAK_GBPS, 4)}


def time_lite(stream, steps: int):
    """DeepSeek-V2-Lite attention shapes (16 heads: the 16-row attention
    kernel), reported next to the main line: the whole step (absorb ->
    attention -> up-projection) and the attention call alone, HIP-event
    timed over graph replays with the cache replicated past the memory-side
    cache."""
    import torch
    from head_latent_attention_11_amd.runner import DecodeBuffers
    from mla_inputs import WORKLOADS, generate
    w = WORKLOADS[LITE_WORKLOAD]
    gen = generate(w)
    seq_lens = [int(x) for x in gen["seq_lens"]]
    cache_b, io_b, flops = algorithmic(w, seq_lens)
    reps = max(2, -(-768 * 2 ** 20 // cache_b))
    buf = DecodeBuffers(w, gen, device="cuda", poison=False, cache_replicas=reps,
                        weight_replicas=reps)
    per = 10

    def timed(call):
        def fn():
            for i in range(per):
                call(i % reps)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(2):
            g.replay()
        n = max(2, steps // per)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / (n * per)

    t_step = timed(lambda r: buf.step(replica=r))
    t_attn = timed(lambda r: buf.attend(replica=r))
    del buf
    byts = cache_b + io_b
    return {"workload": w.name, "batch": w.batch, "kv_len": w.kv_len, "n_heads": w.n_heads,
            "step_us": round(t_step * 1e6, 2),
            "tokens_per_s": round(w.batch * w.q_tokens / t_step, 1),
            "attn_us": round(t_attn * 1e6, 2),
            "latent_cache_GBps": round(cache_b / t_attn / 1e9, 1),
            "bytes_alg_per_launch": byts,
            "frac_hbm": round(byts / t_attn / 1e9 / HBM_PEAK_GBPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the cpu_baseline sample")
    ap.add_argument("--no-out-proj", action="store_true",
                    help="skip the timings of the cache producer and of the output "
                         "projection around the step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lite", action="store_true",
                    help="skip the DeepSeek-V2-Lite (16-head) attention line")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a calibration copy and a few attention calls for "
                         "rocprofv3 counter runs (see bench_traffic.py), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from head_latent_attention_11_amd.runner import DecodeBuffers
    from mla_inputs import WORKLOADS, generate

    w = WORKLOADS[args.workload]
    gen = generate(w)
    seq_lens = [int(x) for x in gen["seq_lens"]]
    cache_b, io_b, flops = algorithmic(w, seq_lens)
    replicas = max(1, -(-768 * 2 ** 20 // max(cache_b, 1)))
    torch.cuda.set_device(0)
    buf = DecodeBuffers(w, gen, device="cuda", poison=False, cache_replicas=replicas,
                        weight_replicas=replicas)
    torch.cuda.synchronize()

    # Each step is captured once per cache replica as a HIP graph and
    # replayed: the library calls are asynchronous launches on the current
    # stream, and replay removes the per-call host overhead of the binding.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()                      # warm up outside the graph
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        return g

    # A serving loop captures many launches per graph (a decode step of the
    # whole model runs this layer once per layer), so the host-side cost of a
    # graph launch is shared: STEPS_PER_GRAPH steps per graph, cache replicas
    # round-robin.  n_steps(k) replays graphs for exactly k steps.
    def steps_fn(first, n):
        def fn():
            for i in range(n):
                buf.step(replica=(first + i) % replicas)
        return fn

    step_graphs = [capture(steps_fn(j * STEPS_PER_GRAPH, STEPS_PER_GRAPH))
                   for j in range(replicas)]
    tail_graphs = {}

    def n_steps(k):
        for j in range(k // STEPS_PER_GRAPH):
            step_graphs[j % replicas].replay()
        rem = k % STEPS_PER_GRAPH
        if rem:
            if rem not in tail_graphs:
                tail_graphs[rem] = capture(steps_fn(0, rem))
            tail_graphs[rem].replay()

    if args.steps % STEPS_PER_GRAPH:
        n_steps(args.steps % STEPS_PER_GRAPH)    # capture the tail graph now
    torch.cuda.synchronize()
    # the attention call alone: ATTN_PER_GRAPH calls (replicas round-robin) per
    # graph, so the gap between graph launches is amortised and the per-call
    # time is the kernels' own (decode + combine)
    def attn_calls():
        for i in range(ATTN_PER_GRAPH):
            buf.attend(replica=i % replicas)
    attn_graph = capture(attn_calls)
    stream = torch.cuda.current_stream()

    if args.traffic_probe:
        # For rocprofv3 counter runs: a plain copy of known size (the
        # calibration kernel), then a few attention calls.  Nothing is timed.
        src = torch.empty(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        for i in range(3):
            buf.attend(replica=i % replicas)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "copy_bytes": COPY_PROBE_BYTES,
                          "workload": w.name, "sources_sha256": kernel_sources_sha256(),
                          "bytes_alg_per_launch": cache_b + io_b}), flush=True)
        return

    n_steps(args.warmup)
    torch.cuda.synchronize()

    # ---- timed region: K whole steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    n_steps(args.steps)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    ms_step_events = e0.elapsed_time(e1) / args.steps

    # ---- the attention launches alone, back to back (same stream)
    n_rep = max(1, -(-args.steps // ATTN_PER_GRAPH))
    for i in range(max(1, args.warmup // ATTN_PER_GRAPH)):
        attn_graph.replay()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a0.record(stream)
    for i in range(n_rep):
        attn_graph.replay()
    a1.record(stream)
    torch.cuda.synchronize()
    attn_ms = a0.elapsed_time(a1) / (n_rep * ATTN_PER_GRAPH)
    attn_s = attn_ms * 1e-3
    bytes_alg = cache_b + io_b
    achieved_gbps = bytes_alg / attn_s / 1e9
    tflops = flops / attn_s / 1e12
    mfma_peak = MFMA_PEAK_TFLOPS["bf16"]          # the MFMA precision issued
    t_hbm = bytes_alg / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (mfma_peak * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(tflops / mfma_peak, 4)}
    tr = traffic_for_current_kernel(w.name)
    roof["traffic"] = tr["hbm_bytes_per_launch"] if tr else None
    roof["kernel"] = ("mla_decode_attn (decode_mfma_kernel, or decode_small_kernel for "
                      "query-row counts that are no multiple of 128, + combine_kernel when "
                      "split), per call, HIP-event timed over back-to-back graph replays")
    roof["bytes_alg_per_launch"] = bytes_alg
    roof["flops_alg_per_launch"] = flops

    # Practical HBM ceiling on this GPU, for context: a plain 1 GiB device
    # copy (read + write bytes over its time).  Not part of any step.
    cp_src = torch.empty(COPY_CEILING_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    cp_dst = torch.empty_like(cp_src)
    for _ in range(3):
        cp_dst.copy_(cp_src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(10):
        cp_dst.copy_(cp_src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * COPY_CEILING_BYTES / (c0.elapsed_time(c1) * 1e-3 / 10) / 1e9
    del cp_src, cp_dst

    # Achievable dense bf16 matrix throughput on this GPU, for context: a
    # library GEMM (torch.mm -> hipBLASLt) of 8192^3 with contiguous
    # operands.  Not part of any step.
    n_g = 8192
    ga = torch.randn(n_g, n_g, device="cuda").to(torch.bfloat16)
    gb = torch.randn(n_g, n_g, device="cuda").to(torch.bfloat16)
    gc = torch.mm(ga, gb)
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(10):
        torch.mm(ga, gb, out=gc)
    c1.record(stream)
    torch.cuda.synchronize()
    gemm_tflops = 2 * n_g ** 3 / (c0.elapsed_time(c1) * 1e-3 / 10) / 1e12
    del ga, gb, gc

    out = {
        "metric": "MLA decode tokens/s and latent-cache GB/s (% of HBM/MFMA roofline)",
        "value": round(w.batch * w.q_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype if w.kv_dtype != "f32" else "f32",
        "data": "synthetic (seeded N(0,1) latent cache and queries, N(0,1/d_c) weights)",
        "config": {"workload": w.name, "batch": w.batch, "q_tokens": w.q_tokens,
                   "kv_len": w.kv_len or None, "n_heads": w.n_heads, "d_head": w.d_head,
                   "d_latent": w.d_latent, "d_rope": w.d_rope, "kv_dtype": w.kv_dtype,
                   "layout": w.layout, "cache_replicas": replicas,
                   "steps_per_graph": STEPS_PER_GRAPH},
        "latent_cache_GBps": round(cache_b / attn_s / 1e9, 1),
        "hbm_copy_GBps": round(copy_gbps, 1),
        "gemm_bf16_TFLOPs": round(gemm_tflops, 1),
        "attn_us": round(attn_ms * 1e3, 2),
        "step_us_events": round(ms_step_events * 1e3, 2),
        "roofline": roof,
    }
    if w.q_dtype == "bf16" and not args.no_out_proj:
        out["out_proj"] = time_out_proj(w, buf, stream)
        out["kv_produce"] = time_kv_produce(w, buf, stream)
    if not args.no_lite and w.name != LITE_WORKLOAD:
        out["v2lite"] = time_lite(stream, args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, gen, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
