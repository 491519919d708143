"""Decode-step benchmark of libmlra on one MI355X.

A step is one pass of the whole decode path over one batch: query absorption,
split-K latent attention over the paged cache, log-sum-exp combine with the
value up-projection (plus the latent append for the ragged workload, and the
query path and RoPE key before it for the whole-layer workload). Inputs are
seeded synthetic data with the workload's shapes, resident in HBM before timing.
Several independent cache pools are rotated so the 256 MB Infinity Cache cannot
serve the cache stream.

Prints one JSON line. `value` is decode tokens/s (batch / step time over K
steps timed back to back with one event pair around all of them). The
`roofline` object reports the attention kernel (the one that streams the cache):
algorithmic cache bytes per launch / its mean duration over a second pass of the
same K steps, each attention launch dispatched with a HIP event pair that its
dispatch fills with the kernel's own start and stop times (mlra_attend_timed),
against the 8 TB/s HBM3E peak; `roofline.trace` gives the same ratio from the
committed rocprofv3 kernel-trace summary of this workload when that summary was
taken on the current attention source. `cpu_baseline` times the CPU oracle
(test infrastructure, used here only for this baseline) on a bounded sample of
the same workload, and on the tiny fp32 workload with one thread.

The W warm-up steps are followed by more untimed steps until --warmup-seconds
(0.5 s) of wall time has passed, so the timed steps run at settled clocks.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--warmup-seconds S] [--workload 2]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "decode tokens/s + latent-cache HBM GB/s (% of peak), MLRA-4 B=32 ctx=8K, 1 GPU"
# the attention kernels' sources: a committed profile counts for the current
# build only when it was taken on these exact files
KERNEL_SOURCES = [os.path.join(ROOT, "compressed_kv_cache_mlra_amd", "csrc", f)
                  for f in ("attend_mfma.hip", "attend_generic.hip", "common.h")]
# rocprofv3 summaries of the attention kernel, per workload:
# profiles/attend_<tag>_kernel_stats.txt (kernel trace) and _counters.txt (HBM bytes)
PROFILE_TAGS = {1: "tiny_fp32", 2: "mlra4_b32_ctx8k", 3: "mla_b32_ctx8k", 4: "tpshare_b64_ctx32k",
                5: "mlra2_ragged_append", 6: "mlra4_fp8_b32_ctx8k", 7: "mlra4_b32_ctx8k_layer",
                8: "mlra4_fp8_block_scaled_b32_ctx8k", 9: "readb_k2_b32_ctx8k", 10: "readb_k4_b32_ctx8k",
                11: "h24_b32_ctx8k", 12: "h24_readb_k4_b32_ctx8k", 13: "tp2share_mlra2_b64_ctx32k",
                14: "mla_tpshare_b64_ctx32k"}


def _profile_file(workload: int, kind: str) -> str:
    tag = PROFILE_TAGS.get(workload, "none")
    return os.path.join(ROOT, "profiles", f"attend_{tag}_{kind}.txt")
COPY_BYTES = 1 << 30


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--warmup-seconds", type=float, default=0.5,
                   help="keep running untimed steps after the W warm-up steps until this much wall time has "
                        "passed (the GPU's clocks take about 0.1 s of load to settle; 0 for counter runs)")
    p.add_argument("--workload", type=int, default=2, choices=list(range(1, 15)))
    p.add_argument("--pools", type=int, default=3, help="cache pool instances rotated per step")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-baseline duration")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the graph-replay and streaming-read legs (for profiler runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy (known bytes), to scale HBM counters")
    return p.parse_args()


def _copy_calibration(steps: int):
    """A plain copy kernel of known size: reads and writes COPY_BYTES per launch.
    Profiling it with the same counters as the attention kernel gives the factor
    that turns FETCH_SIZE / WRITE_SIZE readings into bytes."""
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": COPY_BYTES, "launches": steps}), flush=True)


def _source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def _profile_text(workload: int, kind: str):
    """A committed profile summary of this workload, if it was taken on the
    current attention source."""
    path = _profile_file(workload, kind)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != _source_hash():
        return None
    return text


def _trace(bytes_alg: float, workload: int):
    """The attention kernel's mean duration in the committed rocprofv3
    kernel-trace summary of this workload (same source) and the HBM fraction
    it gives."""
    text = _profile_text(workload, "kernel_stats")
    m = text and re.search(r"attend_trace_mean_ns:\s*([0-9.eE+]+)", text)
    if not m:
        return None
    ns = float(m.group(1))
    gbps = bytes_alg / (ns * 1e-9) / 1e9
    return {"mean_us": round(ns / 1e3, 3), "achieved": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "source": os.path.relpath(_profile_file(workload, "kernel_stats"), ROOT)}


def _traffic(bytes_alg: float, workload: int):
    """HBM bytes per launch of the attention kernel from the committed rocprofv3
    counter summary of this workload, when it was taken on the current kernel
    source."""
    text = _profile_text(workload, "counters")
    if text is None:
        return None
    f = re.search(r"hbm_read_bytes_per_launch:\s*([0-9.eE+]+)", text)
    w = re.search(r"hbm_write_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not f or not w:
        return None
    return {"read_bytes": float(f.group(1)), "write_bytes": float(w.group(1)),
            "algorithmic_bytes": bytes_alg,
            "read_over_algorithmic": float(f.group(1)) / bytes_alg}


def main():
    args = _args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the decode path "
              "has no multi-GPU component.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        _copy_calibration(args.steps)
        return

    import numpy as np
    import torch

    import compressed_kv_cache_mlra_amd as mlra
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    t0 = time.time()
    inp = synth.workload_inputs(args.workload, pool_copies=args.pools)
    pools_np = inp.pool if isinstance(inp.pool, list) else [inp.pool]
    s = inp.shape

    def dev(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.to("cuda")

    pools = [dev(p) for p in pools_np]
    page_table = None if inp.page_table is None else dev(inp.page_table)
    seq_lens, q_c, q_r = dev(inp.seq_lens), dev(inp.q_c), dev(inp.q_r)
    w_uk, w_uv = dev(inp.w_uk), dev(inp.w_uv)
    append = inp.x is not None
    qpath = append and s.d_cq > 0
    if append:
        positions, x, kr_new = dev(inp.positions), dev(inp.x), dev(inp.kr_new)
        # one copy of the step's weights per pool instance, rotated with it, so
        # that they stream from HBM as a different layer's weights would
        w_dkv = [dev(inp.w_dkv) for _ in pools]
    qp_bytes = 0.0
    if qpath:
        qpw = [tuple(dev(a) for a in (inp.w_dq, inp.w_uq, inp.w_qr, inp.w_kr)) for _ in pools]
        et = torch.bfloat16 if s.dtype != "f32" else torch.float32
        c_q = torch.empty((s.batch, s.d_cq), dtype=torch.float32, device="cuda")
        q_c = torch.empty((s.batch, s.n_heads, s.d_h), dtype=et, device="cuda")
        q_r = torch.empty((s.batch, s.n_heads, s.d_r), dtype=et, device="cuda")
        kr_new = torch.empty((s.batch, s.d_r), dtype=et, device="cuda")
        qp_bytes = float(sum(a.numel() * a.element_size() for a in qpw[0]) +
                         w_dkv[0].numel() * w_dkv[0].element_size())
    desc = mlra.make_desc(batch=s.batch, n_heads=s.n_heads, d_h=s.d_h, d_c=s.d_c, n_blocks=s.n_blocks,
                          d_r=s.d_r, max_pages_per_seq=inp.max_pages_per_seq,
                          num_pages=pools_np[0].shape[0], dtype=s.dtype, page_size=s.page_size,
                          blocks_per_head=s.blocks_per_head, d_model=s.d_model, cache_scale=s.cache_scale,
                          d_cq=s.d_cq, rope_base=s.rope_base)
    ws = mlra.alloc_workspace(desc, inp.max_seq_len)
    out = torch.empty((s.batch, s.n_heads, s.d_h), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    setup_s = time.time() - t0

    def launch(i, cs, mark=lambda k: None, kev=None):
        """One step on pool instance i % pools, enqueued on cs; mark(k) is
        called at the kernel boundaries 0 (start) .. 4 (end); kev: an event
        pair that the attention's dispatch fills with its own start and stop."""
        p = i % len(pools)
        mark(0)
        if qpath:
            # the token's projections: latent append, RoPE key, query path
            w_dq, w_uq, w_qr, w_kr = qpw[p]
            mlra.project_token(desc, x, positions, pools[p], page_table, w_dkv[p], w_kr, kr_new, None, w_dq,
                               w_uq, w_qr, c_q, q_c, q_r, ws, cs)
            mark(1)
        elif append:
            mlra.append_latent(desc, pools[p], page_table, positions, x, w_dkv[p], kr_new, None, ws, cs)
        mlra.absorb_query(desc, seq_lens, q_c, q_r, w_uk, ws, cs)
        mark(2)
        if kev is None:
            mlra.attend(desc, pools[p], page_table, ws, cs)
        else:
            mlra.attend_timed(desc, pools[p], page_table, ws, kev[0], kev[1], cs)
        mark(3)
        mlra.combine(desc, ws, w_uv, out, None, cs)
        mark(4)

    def step(i, ev=None, kev=None):
        launch(i, stream, (lambda k: ev[k].record(stream)) if ev is not None else (lambda k: None), kev)

    # Warm-up: W steps, then more untimed steps in chunks until the floor of
    # wall time has passed. From idle the first ~0.1 s of steps run up to 10%
    # slower while the clocks rise; the timed steps should see steady clocks.
    t_warm = time.time()
    warm_steps = 0
    while warm_steps < args.warmup or time.time() - t_warm < args.warmup_seconds:
        for _ in range(args.warmup if warm_steps < args.warmup else 50):
            step(warm_steps)
            warm_steps += 1
        torch.cuda.synchronize()
    warm_s = time.time() - t_warm

    # Timed region 1: K whole steps back to back, bracketed by two events only
    # (events between the kernels would add their own packets to the step).
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # Timed region 2: the same K steps with HIP events around every launch on the
    # launch stream (per-kernel durations, each including its dispatch).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    # Timed region 3: the same K steps, the attention dispatched with an event
    # pair that records the kernel's own start and stop (the roofline's
    # duration); no other events in these steps.
    kevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, None, kevs[i])
    torch.cuda.synchronize()
    attend_kernel_ms = [k[0].elapsed_time(k[1]) for k in kevs]
    qp_ms = [e[0].elapsed_time(e[1]) for e in evs] if qpath else [0.0]
    pre_ms = [e[1 if qpath else 0].elapsed_time(e[2]) for e in evs]
    attend_ms = [e[2].elapsed_time(e[3]) for e in evs]
    comb_ms = [e[3].elapsed_time(e[4]) for e in evs]
    step_ev_ms = [e[0].elapsed_time(e[4]) for e in evs]

    graph_ms_per_step, read_gbps = None, None
    if not args.no_extras:
        graph_ms_per_step, read_gbps = _extras(args, torch, mlra, launch, len(pools), stream,
                                               _cache_bytes(inp, s))

    n_tokens = int(np.sum(inp.seq_lens.astype(np.int64)))
    cache_bytes = _cache_bytes(inp, s)
    heads_per_block = s.n_heads * s.blocks_per_head // s.n_blocks
    # per token: every (head, attended block) pair scores w + d_r and accumulates w
    attn_flops = float(n_tokens) * s.n_heads * s.blocks_per_head * (4.0 * s.w + 2.0 * s.d_r)
    attend_mean_ms = float(np.mean(attend_kernel_ms))
    achieved = cache_bytes / (attend_mean_ms * 1e-3) / 1e9
    # the roofline's duration: the committed kernel-trace mean of this workload
    # when it was taken on the current attention source (over the same pass of
    # dispatch-timed launches), else the live dispatch-timed mean
    trace = _trace(cache_bytes, args.workload)
    roof_gbps = trace["achieved"] if trace else achieved
    roof_duration = ("rocprofv3 kernel-trace mean of the attention launches in the dispatch-timed pass "
                     "(committed summary, same source hash)" if trace else
                     "kernel start to stop recorded by its dispatch (mlra_attend_timed), mean over K whole steps")
    tokens_per_s = s.batch / (ms_per_step * 1e-3)

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the MFMA operand type: bf16 caches multiply in bf16, E4M3 caches widen to f16
        "dtype": {"f32": "f32", "fp8": "f16", "fp8b": "f16"}.get(s.dtype, "bf16"),
        "data": "synthetic",
        "config": {"workload": wl["name"], "workload_id": args.workload, "cache_dtype": s.dtype, "batch": s.batch, "n_heads": s.n_heads, "d_h": s.d_h,
                   "d_c": s.d_c, "n_blocks": s.n_blocks, "d_r": s.d_r, "page_size": s.page_size,
                   "context_tokens": n_tokens, "heads_per_block": heads_per_block,
                   "pool_instances": len(pools), "parallelism": "single GPU"},
        "cache_gbps_full_step": round(cache_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "graph_ms_per_step": None if graph_ms_per_step is None else round(graph_ms_per_step, 5),
        "step_us_with_events": {"p10": round(1e3 * float(np.percentile(step_ev_ms, 10)), 2),
                                "p50": round(1e3 * float(np.percentile(step_ev_ms, 50)), 2),
                                "p90": round(1e3 * float(np.percentile(step_ev_ms, 90)), 2)},
        "stream_read_gbps_same_device": None if read_gbps is None else round(read_gbps, 1),
        "attend_frac_of_stream_read": None if read_gbps is None else round(achieved / read_gbps, 4),
        "cache_pct_of_hbm_peak_full_step": round(100.0 * cache_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "attend_kernel_us": {"mean": round(1e3 * attend_mean_ms, 2),
                             "p10": round(1e3 * float(np.percentile(attend_kernel_ms, 10)), 2),
                             "p50": round(1e3 * float(np.percentile(attend_kernel_ms, 50)), 2),
                             "p90": round(1e3 * float(np.percentile(attend_kernel_ms, 90)), 2)},
        "kernel_us_with_events": {"append_absorb": round(1e3 * float(np.mean(pre_ms)), 2),
                      "attend": round(1e3 * float(np.mean(attend_ms)), 2),
                      "attend_p50": round(1e3 * float(np.percentile(attend_ms, 50)), 2),
                      "attend_p10": round(1e3 * float(np.percentile(attend_ms, 10)), 2),
                      "attend_p90": round(1e3 * float(np.percentile(attend_ms, 90)), 2),
                      "combine": round(1e3 * float(np.mean(comb_ms)), 2),
                      "token_projections": round(1e3 * float(np.mean(qp_ms)), 2) if qpath else None},
        "roofline": {
            "kernel": "attend_generic_kernel" if s.dtype == "f32" else "attend_mfma_kernel",
            "bound": "hbm",
            "achieved": round(roof_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(roof_gbps / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes_per_launch": cache_bytes,
            "algorithmic_flops_per_launch": attn_flops,
            "duration": roof_duration,
            "live": {"mean_us": round(1e3 * attend_mean_ms, 2), "achieved": round(achieved, 1),
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "duration": "kernel start to stop recorded by its dispatch (mlra_attend_timed), "
                                 "mean over K whole steps, this run"},
            "trace": trace,
            "traffic": _traffic(cache_bytes, args.workload),
            "mfma_tflops": round(attn_flops / (attend_mean_ms * 1e-3) / 1e12, 2),
            "mfma_frac_of_bf16_peak": round(attn_flops / (attend_mean_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
        },
        "setup_s": round(setup_s, 1),
    }
    if qpath:
        # project_token (latent append, RoPE key, query path): its five weight
        # matrices are its HBM bytes
        qms = float(np.mean(qp_ms))
        result["token_projections"] = {"weight_bytes": qp_bytes, "us": round(1e3 * qms, 2),
                                "gbps": round(qp_bytes / (qms * 1e-3) / 1e9, 1),
                                "frac_of_hbm_peak": round(qp_bytes / (qms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(inp, args.cpu_seconds)
        result["cpu_baseline"]["one_thread_tiny"] = _cpu_one_thread_tiny()
    print(json.dumps(result), flush=True)


def _cache_bytes(inp, s):
    """Algorithmic cache bytes of one step: every attended token's row once
    (k^R is read once for all blocks)."""
    import numpy as np
    return float(np.sum(inp.seq_lens.astype(np.int64))) * s.row_bytes


def _extras(args, torch, mlra, launch, n_pools, stream, cache_bytes):
    """(1) The same K steps replayed from HIP graphs, one graph per pool
    instance; (2) a plain streaming read of as many bytes as the attention's
    algorithmic cache bytes, with the attention's loads and launch shape,
    rotated over as many buffers as there are pool instances."""
    graphs = []
    for p in range(n_pools):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            launch(p, torch.cuda.current_stream())
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / args.steps
    del graphs

    rbytes = int(cache_bytes) // 16 * 16
    rbufs = [torch.empty(rbytes, dtype=torch.uint8, device="cuda") for _ in range(n_pools)]
    sink = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    for i in range(args.warmup):
        mlra.stream_read(rbufs[i % len(rbufs)], sink, stream)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for i in range(args.steps):
        mlra.stream_read(rbufs[i % len(rbufs)], sink, stream)
    r1.record(stream)
    torch.cuda.synchronize()
    read_gbps = rbytes / (r0.elapsed_time(r1) / args.steps * 1e-3) / 1e9
    return graph_ms, read_gbps


def _cpu_baseline(inp, target_s: float):
    """The oracle, as it stands, on whole sequences of the same workload (all
    heads of sequence 0, then 1, ...) until about target_s seconds of work."""
    import oracle

    s = inp.shape
    pool = inp.pool[0] if isinstance(inp.pool, list) else inp.pool
    done, spent = 0, 0.0
    order = list(range(s.batch))
    while done < len(order) and spent < target_s:
        b = order[done]
        t = time.perf_counter()
        oracle.decode_unabsorbed(inp, [(b, i) for i in range(s.n_heads)], pool=pool)
        spent += time.perf_counter() - t
        done += 1
    tokens = sum(int(inp.seq_lens[b]) for b in order[:done])
    return {"value": round(done / spent, 4), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{done} of {s.batch} sequences, all {s.n_heads} heads each "
                      f"({tokens} cached tokens), un-absorbed fp64 oracle, {spent:.1f} s"}


def _cpu_one_thread_tiny(target_s: float = 2.0):
    """The oracle on one thread over the whole tiny fp32 workload (every head
    of its one 256-token sequence), repeated for about target_s seconds."""
    import oracle
    import synth

    inp = synth.workload_inputs(1)
    n0 = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < target_s:
            oracle.decode_unabsorbed(inp)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
    finally:
        oracle.set_num_threads(n0)
    return {"workload": synth.WORKLOADS[1]["name"], "us_per_step": round(dt * 1e6, 1),
            "tokens_per_s": round(inp.shape.batch / dt, 1), "cores": 1, "steps_timed": reps}


if __name__ == "__main__":
    main()
