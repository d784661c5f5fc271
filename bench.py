#!/usr/bin/env python3
"""Benchmark of one MLA decode step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic inputs:
    mla_absorb_append (mla_absorb_q and mla_cache_append of the B*T new rows,
    one launch) -> mla_decode_attn (split-KV attention + LSE combine)
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
DEFAULT_WORKLOAD = "v2_fp8_t4_b64_l8k"       # B=64, T=4, L=8192, fp8 cache
COMPANION_WORKLOAD = "v2_b64_l8k_bf16"      # B=64, T=1, L=8192, bf16 cache
ATTN_PER_GRAPH = 20                     # attention calls captured per graph
STEPS_PER_GRAPH = 10                    # decode steps captured per graph
COPY_PROBE_BYTES = 512 * 2 ** 20        # calibration copy of the traffic probe
COPY_CEILING_BYTES = 2 ** 30            # plain device copy reported as the practical ceiling
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
_CSRC = os.path.join(ROOT, "head_latent_attention_11_amd", "csrc")
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in
                  ("decode_mfma.hip", "decode_fp8.hip", "decode_mfma_asm.inc", "decode_small.hip",
                   "decode_x2.hip", "decode_tile.hpp", "kernels_misc.hip", "mla_common.hpp",
                   "plan_device.hpp", "mla_api.hip")]
LITE_WORKLOAD = "v2lite_b64_l8k_bf16"   # DeepSeek-V2-Lite shapes (16 heads)
FP6_WORKLOAD = "v2_fp6_t4_b64_l8k"      # the headline shape on the 6-bit cache


def algorithmic(w, seq_lens):
    """Bytes and flops the absorbed method must move / compute per attention
    launch: the latent cache rows, the absorbed queries, the latent output
    and the LSE; 2 * rows * L * (d_c + d_h^R + d_c) flops per sequence."""
    D = w.d_latent + w.d_rope
    if w.kv_dtype == "fp6":
        row_bytes = 452                  # 576 six-bit codes, 18 exponent bytes, 2 pad
    else:
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
    (sequence, head) evaluations, scaled to the full step.  BLAS runs one
    thread per core of this process's affinity set."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import mla as omla
    cores, model = host_info()
    with threadpool_limits(limits=cores):
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
            omla.decode(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["c_rows"],
                        d["kr_rows"], d["row_offsets"], d["seq_lens"], w.q_tokens, seqs=[b],
                        heads=[h])
            n_eval += 1
            h += 1
            if h == w.n_heads:
                h = 0
                b_i += 1
            if time.perf_counter() - t0 >= budget_s and n_eval >= 2:
                break
        elapsed = time.perf_counter() - t0
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    per_eval = elapsed / n_eval                       # one (sequence, head) incl. all T
    full_step = per_eval * w.batch * w.n_heads
    return {
        "value": w.batch * w.q_tokens / full_step,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{n_eval} whole-length (sequence, head) evaluations of the literal "
                   f"fp64 oracle (all T={w.q_tokens} query tokens each) in {elapsed:.1f} s, "
                   f"scaled to B*n_h = {w.batch * w.n_heads} evaluations per step"),
        "host_cores_affinity": cores,
        "cpu_model": model,
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
    t_rm = e0.elapsed_time(e1) * 1e-3 / (5 * calls)
    del g
    # the same projection with W^O in the panel layout (packed once, as at
    # weight-load time, outside the timed region)
    w_p = [torch.empty_like(x) for x in w_o]
    for a, b in zip(w_o, w_p):
        B.out_proj_pack(buf.dims, a, w.d_model, b)
    del w_o

    def fnp():
        for i in range(calls):
            B.out_proj_packed(buf.dims, o, w_p[i % reps], w.d_model, u, buf.n_tok, ws, wsb)
    with torch.cuda.stream(side):
        fnp()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fnp()
    g.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / (5 * calls)
    byts = w_bytes + buf.n_tok * K * 2 + buf.n_tok * w.d_model * 4
    res = {"us": round(t * 1e6, 2), "w_o_layout": "panels (mla_out_proj_packed)",
           "us_row_major": round(t_rm * 1e6, 2), "d_model": w.d_model, "n_tokens": buf.n_tok,
           "bytes_alg": byts, "achieved_GBps": round(byts / t / 1e9, 1),
           "frac_hbm": round(byts / t / 1e9 / HBM_PEAK_GBPS, 4)}
    del w_p, g
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


def host_info():
    """Host CPU context of the oracle timing: the cores this process may run
    on (its affinity set) and the CPU model."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90))}


def roofline(bytes_alg, flops, attn_s):
    """Fraction of the binding roofline for one attention call: HBM bytes
    against 8 TB/s, or flops against the dense peak of the matrix precision
    the kernels issue (bf16: fp8 caches are decoded to bf16 before the
    products); the fp8 dense peak is given next to it."""
    achieved_gbps = bytes_alg / attn_s / 1e9
    tflops = flops / attn_s / 1e12
    peak = MFMA_PEAK_TFLOPS["bf16"]
    t_hbm = bytes_alg / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (peak * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                "frac_fp8_peak": round(tflops / MFMA_PEAK_TFLOPS["fp8"], 4)}
    roof["achieved_GBps"] = round(achieved_gbps, 1)
    roof["achieved_TFLOPs"] = round(tflops, 1)
    return roof


class Timer:
    """A workload resident on the GPU, its decode step and attention call
    captured in HIP graphs (cache and weights replicated to >= 768 MB and
    used round-robin, so each step reads them from HBM), timed with HIP
    events on the stream the graphs are launched on."""

    def __init__(self, name, precision="auto"):
        import torch
        from head_latent_attention_11_amd.runner import DecodeBuffers
        from mla_inputs import WORKLOADS, generate
        self.w = w = WORKLOADS[name]
        self.gen = generate(w)
        self.seq_lens = [int(x) for x in self.gen["seq_lens"]]
        self.cache_b, self.io_b, self.flops = algorithmic(w, self.seq_lens)
        self.replicas = reps = max(2, -(-768 * 2 ** 20 // max(self.cache_b, 1)))
        self.buf = DecodeBuffers(w, self.gen, device="cuda", poison=False, cache_replicas=reps,
                                 weight_replicas=reps, precision=precision)
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream()
        buf = self.buf

        # A serving loop captures many launches per graph (a decode step of
        # the whole model runs this layer once per layer), so the host-side
        # cost of a graph launch is shared: STEPS_PER_GRAPH steps per graph,
        # cache replicas round-robin.
        def steps_fn(first, n):
            def fn():
                for i in range(n):
                    buf.step(replica=(first + i) % reps)
            return fn
        self.step_graphs = [self.capture(steps_fn(j * STEPS_PER_GRAPH, STEPS_PER_GRAPH))
                            for j in range(reps)]
        self.tail_graphs = {}

        def attn_calls():
            for i in range(ATTN_PER_GRAPH):
                buf.attend(replica=i % reps)
        self.attn_graph = self.capture(attn_calls)
        self.steps_fn = steps_fn

    @staticmethod
    def capture(fn):
        import torch
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

    def graphs_for(self, k):
        """The graph replays that run exactly k steps, with their step counts."""
        out = [(self.step_graphs[j % self.replicas], STEPS_PER_GRAPH)
               for j in range(k // STEPS_PER_GRAPH)]
        rem = k % STEPS_PER_GRAPH
        if rem:
            if rem not in self.tail_graphs:
                self.tail_graphs[rem] = self.capture(self.steps_fn(0, rem))
            out.append((self.tail_graphs[rem], rem))
        return out

    def time_steps(self, k, warmup):
        """K steps: one HIP event before and after each graph replay (per-step
        percentiles), the whole region bracketed by device synchronisations."""
        import torch
        for g, _ in self.graphs_for(warmup):
            g.replay()
        plan = self.graphs_for(k)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(self.stream)
        for i, (g, _) in enumerate(plan):
            g.replay()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        per_step = [ev[i].elapsed_time(ev[i + 1]) * 1e-3 / n for i, (_, n) in enumerate(plan)]
        total_ev = ev[0].elapsed_time(ev[-1]) * 1e-3
        return {"wall_s": t1 - t0, "events_s": total_ev, "per_step_s": per_step}

    def time_attention(self, n_graphs, warmup_graphs=3):
        import torch
        for _ in range(warmup_graphs):
            self.attn_graph.replay()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_graphs + 1)]
        torch.cuda.synchronize()
        ev[0].record(self.stream)
        for i in range(n_graphs):
            self.attn_graph.replay()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        per_call = [ev[i].elapsed_time(ev[i + 1]) * 1e-3 / ATTN_PER_GRAPH for i in range(n_graphs)]
        return {"mean_s": ev[0].elapsed_time(ev[-1]) * 1e-3 / (n_graphs * ATTN_PER_GRAPH),
                "per_call_s": per_call}

    def release(self):
        import torch
        del self.buf, self.step_graphs, self.tail_graphs, self.attn_graph
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def side_line(name, steps):
    """Step and attention-call numbers of another workload (same method as
    the main line), reported as a field next to it."""
    t = Timer(name)
    w = t.w
    st = t.time_steps(max(steps, 2 * STEPS_PER_GRAPH), 2 * STEPS_PER_GRAPH)
    at = t.time_attention(max(3, steps // ATTN_PER_GRAPH))
    step_s = st["events_s"] / max(steps, 2 * STEPS_PER_GRAPH)
    attn_s = at["mean_s"]
    ps, pa = percentiles(st["per_step_s"]), percentiles(at["per_call_s"])
    out = {"workload": w.name, "batch": w.batch, "q_tokens": w.q_tokens, "kv_len": w.kv_len,
           "n_heads": w.n_heads, "kv_dtype": w.kv_dtype,
           "step_us": round(step_s * 1e6, 2),
           "step_us_p10_p90": [round(ps["p10"] * 1e6, 2), round(ps["p90"] * 1e6, 2)],
           "tokens_per_s": round(w.batch * w.q_tokens / step_s, 1),
           "attn_us": round(attn_s * 1e6, 2),
           "attn_us_p10_p90": [round(pa["p10"] * 1e6, 2), round(pa["p90"] * 1e6, 2)],
           "latent_cache_GBps": round(t.cache_b / attn_s / 1e9, 1),
           "bytes_alg_per_launch": t.cache_b + t.io_b, "flops_alg_per_launch": t.flops,
           "roofline": roofline(t.cache_b + t.io_b, t.flops, attn_s)}
    t.release()
    return out


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
    ap.add_argument("--precision", default="auto", choices=["auto", "bf16", "bf16x2", "fp32"],
                    help="precision mode of the library (mla_dims_t.precision)")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the companion (bf16, T=1) and DeepSeek-V2-Lite lines")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a calibration copy and a few attention calls for "
                         "rocprofv3 counter runs (see bench_traffic.py), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    t = Timer(args.workload, args.precision)
    w, buf, stream = t.w, t.buf, t.stream
    cache_b, io_b, flops = t.cache_b, t.io_b, t.flops

    if args.traffic_probe:
        # For rocprofv3 counter runs: a plain copy of known size (the
        # calibration kernel), then a few attention calls.  Nothing is timed.
        src = torch.empty(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        for i in range(3):
            buf.attend(replica=i % t.replicas)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "copy_bytes": COPY_PROBE_BYTES,
                          "workload": w.name, "sources_sha256": kernel_sources_sha256(),
                          "bytes_alg_per_launch": cache_b + io_b}), flush=True)
        return

    # ---- timed region: K whole steps (absorb, append, attention, up-projection)
    st = t.time_steps(args.steps, args.warmup)
    ms_step = st["wall_s"] * 1e3 / args.steps
    ms_step_events = st["events_s"] * 1e3 / args.steps
    ps = percentiles(st["per_step_s"])

    # ---- the attention launches alone, back to back (same stream)
    at = t.time_attention(max(3, -(-args.steps // ATTN_PER_GRAPH)),
                          max(1, args.warmup // ATTN_PER_GRAPH))
    attn_s = at["mean_s"]
    pa = percentiles(at["per_call_s"])
    bytes_alg = cache_b + io_b
    roof = roofline(bytes_alg, flops, attn_s)
    tr = traffic_for_current_kernel(w.name)
    roof["traffic"] = tr["hbm_bytes_per_launch"] if tr else None
    roof["kernel"] = ("mla_decode_attn (decode_fp8_kernel for fp8 caches, else decode_mfma_kernel; "
                      "decode_small_kernel for "
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
        "dtype": "bf16" if w.kv_dtype in ("bf16", "fp8", "fp6") else "f32",
        "data": "synthetic (seeded N(0,1) latent cache and queries, N(0,1/d_c) weights)",
        "config": {"workload": w.name, "batch": w.batch, "q_tokens": w.q_tokens,
                   "kv_len": w.kv_len or None, "n_heads": w.n_heads, "d_head": w.d_head,
                   "d_latent": w.d_latent, "d_rope": w.d_rope, "kv_dtype": w.kv_dtype,
                   "layout": w.layout, "precision": args.precision,
                   "cache_replicas": t.replicas,
                   "steps_per_graph": STEPS_PER_GRAPH,
                   "step": "absorb_append (absorb_q + cache_append of B*T rows) + decode_attn + up_proj_v"},
        "step_us_events": round(ms_step_events * 1e3, 2),
        "step_us_median_p10_p90": [round(ps["median"] * 1e6, 2), round(ps["p10"] * 1e6, 2),
                                   round(ps["p90"] * 1e6, 2)],
        "attn_us": round(attn_s * 1e6, 2),
        "attn_us_median_p10_p90": [round(pa["median"] * 1e6, 2), round(pa["p10"] * 1e6, 2),
                                   round(pa["p90"] * 1e6, 2)],
        "latent_cache_GBps": round(cache_b / attn_s / 1e9, 1),
        "hbm_copy_GBps": round(copy_gbps, 1),
        "gemm_bf16_TFLOPs": round(gemm_tflops, 1),
        "roofline": roof,
    }
    if w.q_dtype == "bf16" and not args.no_out_proj:
        out["out_proj"] = time_out_proj(w, buf, stream)
        out["kv_produce"] = time_kv_produce(w, buf, stream)
    t.release()
    if not args.no_side:
        if w.name != COMPANION_WORKLOAD:
            out["companion"] = side_line(COMPANION_WORKLOAD, args.steps)
        if w.name != LITE_WORKLOAD:
            out["v2lite"] = side_line(LITE_WORKLOAD, args.steps)
        if w.name != FP6_WORKLOAD:
            out["fp6_cache"] = side_line(FP6_WORKLOAD, args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(t.w, t.gen, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
