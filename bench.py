#!/usr/bin/env python
"""Decode-attention benchmark on one MI355X.

Default workload: single-sequence bucketed decode at 4K context -- 42 layers,
32 q / 8 kv heads, head_dim 128, bf16, bucket 4096 with an identity block
table, 4096 live keys.  One step is one replay of a captured graph holding, for
every layer, the append of this token's K/V at position 4095 and the attention
of its query over all 4096 keys (the step rewrites the same slot each replay,
so replays at a fixed length are idempotent).

Printed on one JSON line:
  value          KV GB/s: the live K+V bytes a step must read (42 x 2 x 4096 x
                 8 x 128 x 2 B = 704.6 MB), divided by the measured step time;
  ms_per_step    graph replay time (HIP events, averaged over --steps);
  roofline       the per-layer attention call: algorithmic bytes per launch /
                 its average duration, measured with HIP events around graph
                 replays of 42 back-to-back calls, against 8 TB/s HBM;
  cpu_baseline   the fp64 CPU oracle on the same step's bits, timed on the host.

Other workloads (--config c3 / c4 / c5 / c5d) print the same kind of line for
the 64-sequence batched decode, the column-store step and the long-context
passes; --config prefix times the prefill hand-over copies (import of a
4096-token prefill cache into every layer, export back out).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode attention KV GB/s (% of HBM peak) + µs/step at 4K ctx, 1×MI355X"


# Sources that decide a workload's dominant kernel: the kernel's own file,
# the shared device headers and the host plan that sets its launch.
TRAFFIC_SOURCES = {
    "decode_step_4k": ["attn_vec.hip", "device_util.h", "internal.h", "api.hip"],
    "prefix_import_4k": ["prefix_copy.hip", "device_util.h", "internal.h", "api.hip"],
    "batched64": ["attn_vec.hip", "device_util.h", "internal.h", "api.hip"],
    "long_decode_d256": ["attn_mfma.hip", "device_util.h", "internal.h", "api.hip"],
    "column_store": ["attn_mfma.hip", "device_util.h", "internal.h", "api.hip"],
    "draft_verify_d256": ["attn_mfma.hip", "device_util.h", "internal.h", "api.hip"],
}
# bench --config of each traffic record
TRAFFIC_KEY = {"c2": "decode_step_4k", "prefix": "prefix_import_4k", "c3": "batched64",
               "c5d": "long_decode_d256", "c4": "column_store", "c5": "draft_verify_d256"}


def kernel_source_hash(workload: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_194_amd", "csrc")
    for name in sorted(TRAFFIC_SOURCES[workload]):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def profile_record(workload: str) -> dict:
    """The committed PMC record of the workload's dominant kernel, if it was
    taken on the current sources of that kernel; else {}."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        data = json.load(f)
    rec = data.get(workload)
    if not rec or rec.get("kernel_source_sha") != kernel_source_hash(workload):
        return {}
    return rec


def traffic_from_profiles(workload: str):
    """HBM bytes per launch from committed PMC summaries, if they were taken on
    the current sources of the workload's kernel; else None."""
    return profile_record(workload).get("hbm_bytes_per_launch")


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def host_info() -> dict:
    """Cores the oracle may use and what they are."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"affinity_cpus": len(os.sched_getaffinity(0)), "blas_threads": cpu_threads(),
            "cpu_model": model}


def copy_ceiling_gbs(torch, nbytes=4 << 30, reps=5) -> float:
    """A plain device-to-device copy: read + write bytes over time."""
    a = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    sec = s.elapsed_time(e) / 1e3 / reps
    del a, b
    return 2 * (nbytes // 2) / sec / 1e9


def time_graph(torch, graph, reps: int) -> float:
    """Average seconds per replay, HIP events on the current stream."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        graph.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / 1e3 / reps


def time_call(torch, fn, args) -> float:
    """Average seconds per call: graph replays, or with --eager plain launches
    (hardware counters are taken per dispatch)."""
    if args.eager:
        for _ in range(max(1, args.warmup)):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(args.steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / 1e3 / args.steps
    g = capture(torch, fn)
    time_graph(torch, g, max(1, args.warmup))
    return time_graph(torch, g, args.steps)


def capture(torch, fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


# ---------------------------------------------------------------------------
# 42-layer single-sequence decode at a fixed context
# ---------------------------------------------------------------------------

def bench_decode_step(args, torch):
    import paged_kv_cache_194_amd as pkv
    import workloads
    from paged_kv_cache_194_amd.harness import DecodeStepGraph, PagedDecodeCache

    m = workloads.DecodeModel()
    L = args.ctx
    dev = torch.device("cuda:0")
    cache = PagedDecodeCache(m.layers, m.q_heads, m.kv_heads, m.head_dim, L, dev, m.dtype,
                             num_splits=args.splits)
    for i in range(m.layers):   # the stored prefix (and stale tail) of every layer
        cache.k[i].copy_(workloads.randn(cache.k[i].shape, m.dtype, workloads.SEED_BASE + 200 + 2 * i, dev))
        cache.v[i].copy_(workloads.randn(cache.v[i].shape, m.dtype, workloads.SEED_BASE + 201 + 2 * i, dev))
    cache.set_length(L)
    inputs = workloads.c2_step_inputs(1, m, dev)[0].contiguous()       # [layers, Hq+2Hkv, D]
    out = torch.zeros(m.layers, m.q_heads, m.head_dim, dtype=m.dtype, device=dev)
    runner = DecodeStepGraph(cache, inputs, out)

    if args.eager:
        # plain launches, one step at a time (hardware counters are taken per dispatch)
        for _ in range(max(1, args.warmup)):
            runner.forward()
        torch.cuda.synchronize()
        t_wall0 = time.perf_counter()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(args.steps):
            runner.forward()
        e.record()
        torch.cuda.synchronize()
        sec_step = s.elapsed_time(e) / 1e3 / args.steps
        wall = time.perf_counter() - t_wall0
    else:
        for _ in range(max(1, args.warmup)):
            runner.step()
        torch.cuda.synchronize()
        graph = runner._graphs[(cache.bucket, cache.generation)]
        t_wall0 = time.perf_counter()
        sec_step = time_graph(torch, graph, args.steps)
        wall = time.perf_counter() - t_wall0

    kv_bytes_layer = 2 * L * m.kv_heads * m.head_dim * 2
    kv_bytes_step = m.layers * kv_bytes_layer

    # Dominant kernel: the per-layer attention call, 42 back-to-back in a graph.
    ws = cache.workspace
    if args.eager:
        result_eager = {"metric": METRIC, "eager_us_per_step": round(sec_step * 1e6, 2), "wall_s": round(wall, 3)}
        return result_eager

    def attn_only():
        for i in range(m.layers):
            x = inputs[i]
            pkv.paged_decode_attn(out[i].unsqueeze(0), x[:m.q_heads].unsqueeze(0), cache.k[i], cache.v[i],
                                  cache.block_table, cache.seqused, max_seqlen_k=cache.bucket,
                                  num_splits=args.splits, workspace=ws)
    g_attn = capture(torch, attn_only)
    time_graph(torch, g_attn, 3)
    sec_call = time_graph(torch, g_attn, max(5, args.steps // 2)) / m.layers
    achieved = kv_bytes_layer / sec_call / 1e9

    result = {
        "metric": METRIC,
        "value": round(kv_bytes_step / sec_step / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_step * 1e3, 5),
        "us_per_step": round(sec_step * 1e6, 2),
        "pct_hbm_peak": round(100 * kv_bytes_step / sec_step / 1e9 / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "single-sequence bucketed paged decode, 42 layers, append + attend per layer",
                   "context": L, "bucket": cache.bucket, "layers": m.layers, "q_heads": m.q_heads,
                   "kv_heads": m.kv_heads, "head_dim": m.head_dim, "block_size": 16,
                   "num_splits": pkv.attn_num_splits(1, 1, cache.bucket, m.q_heads, m.kv_heads,
                                                     m.head_dim, args.splits),
                   "kv_bytes_per_step": kv_bytes_step},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles("decode_step_4k"),
                     "kernel": "paged_decode_attn call (one layer, 4096 keys)",
                     "bytes_per_launch": kv_bytes_layer, "us_per_launch": round(sec_call * 1e6, 3)},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(args, torch, cache, inputs, L, kv_bytes_step)
    return result


def cpu_baseline_decode(args, torch, cache, inputs, L, kv_bytes_step):
    """The oracle, as it stands, on the same bits: every layer of one step."""
    import numpy as np

    import oracle

    m_layers = cache.num_layers
    hq, hkv, D = cache.q_heads, cache.kv_heads, cache.head_dim
    layers = list(range(min(m_layers, args.cpu_layers)))
    host = []
    for i in layers:
        host.append((inputs[i, :hq].unsqueeze(0).cpu().view(torch.int16).numpy().view(np.uint16),
                     cache.k[i].cpu().view(torch.int16).numpy().view(np.uint16),
                     cache.v[i].cpu().view(torch.int16).numpy().view(np.uint16)))
    bt = cache.block_table.cpu().numpy()
    cu = np.array([0, 1])
    used = np.array([L])
    t0 = time.perf_counter()
    for q, k, v in host:
        oracle.paged_attention(q, k, v, bt, cu, used, dtype="bf16", scale=1.0 / D ** 0.5,
                               max_seqlen_k=cache.bucket)
    sec = (time.perf_counter() - t0) / len(layers) * m_layers
    return {"value": round(kv_bytes_step / sec / 1e9, 4), "unit": "GB/s", "cores": cpu_threads(),
            "kind": "oracle", "sec_per_step": round(sec, 3), **host_info(),
            "sample": f"{len(layers)} of {m_layers} layers of one step at {L} keys, scaled to the step"}


# ---------------------------------------------------------------------------
# One-call workloads: batched paged decode, column store, long context
# ---------------------------------------------------------------------------

def host_bits(torch, t):
    """A device tensor's raw bits on the host (bf16 as uint16), as the oracle takes them."""
    import numpy as np
    h = t.cpu()
    return h.view(torch.int16).numpy().view(np.uint16) if h.dtype == torch.bfloat16 else h.numpy()


def cpu_baseline_call(run, fraction: float, kv_bytes: int, sample: str) -> dict:
    """The oracle, as it stands, on the same bits: ``run()`` computes the
    sampled part of the call, ``fraction`` is that part's share of the call's
    work (visible query-key pairs), and the time is scaled to the whole call."""
    t0 = time.perf_counter()
    run()
    sec = (time.perf_counter() - t0) / fraction
    return {"value": round(kv_bytes / sec / 1e9, 4), "unit": "GB/s", "cores": cpu_threads(),
            "kind": "oracle", "sec_per_call": round(sec, 3), **host_info(), "sample": sample}


def bench_single_call(args, torch):
    import numpy as np

    import paged_kv_cache_194_amd as pkv
    import workloads

    dev = torch.device("cuda:0")
    if args.config == "c3":
        inp = workloads.c3_batched(device=dev)
        used = inp.seqused_k.cpu().numpy().astype(np.int64)
        kv_bytes = int(used.sum()) * inp.kv_heads * inp.head_dim * 2 * 2
        ws = torch.zeros(max(1, pkv.attn_workspace_bytes(inp.num_seqs, 1, inp.max_seqlen_k, inp.q_heads,
                                                         inp.kv_heads, inp.head_dim, args.splits)),
                         dtype=torch.uint8, device=dev)
        out = torch.empty_like(inp.q)

        def call():
            pkv.paged_decode_attn(out, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                                  max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale,
                                  num_splits=args.splits, workspace=ws)
        name = "batched paged decode, 64 sequences, lengths U[1,8192], 40000-block pool"
        extra = {"sum_len": int(used.sum())}

        def oracle_run():
            import oracle
            oracle.paged_attention(host_bits(torch, inp.q), host_bits(torch, inp.k_cache),
                                   host_bits(torch, inp.v_cache), inp.block_table.cpu().numpy(),
                                   inp.cu_seqlens_q.cpu().numpy(), used, dtype="bf16", scale=inp.scale,
                                   max_seqlen_k=inp.max_seqlen_k)
        oracle_fraction, oracle_sample = 1.0, "all 64 sequences (host copies of the inputs included)"
    elif args.config == "c5d":
        inp = workloads.c5_long(device=dev, decode=True)
        used = inp.seqused_k.cpu().numpy().astype(np.int64)
        kv_bytes = int(used.sum()) * inp.kv_heads * inp.head_dim * 2 * 2
        splits = args.splits or 16
        ws = torch.zeros(max(1, pkv.attn_workspace_bytes(inp.num_seqs, 1, inp.max_seqlen_k, inp.q_heads,
                                                         inp.kv_heads, inp.head_dim, splits)),
                         dtype=torch.uint8, device=dev)
        out = torch.empty_like(inp.q)

        def call():
            pkv.paged_decode_attn(out, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                                  max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, causal=True,
                                  num_splits=splits, workspace=ws)
        name = "long-context decode, 4 sequences 32K/64K, 64 q / 8 kv heads, D 256, 16 splits"
        extra = {}

        def oracle_run():
            import oracle
            oracle.paged_attention(host_bits(torch, inp.q), host_bits(torch, inp.k_cache),
                                   host_bits(torch, inp.v_cache), inp.block_table.cpu().numpy(),
                                   inp.cu_seqlens_q.cpu().numpy(), used, dtype="bf16", scale=inp.scale,
                                   causal=True, max_seqlen_k=inp.max_seqlen_k, seqs=[0, 1])
        oracle_fraction = float(used[:2].sum()) / float(used.sum())
        oracle_sample = (f"sequences 0 and 1 ({int(used[0])} + {int(used[1])} keys) of 4, scaled by "
                         "live keys (host copies of the inputs included)")
    elif args.config in ("c4", "c5"):
        return bench_multirow(args, torch)
    else:
        raise SystemExit(f"unknown --config {args.config}")
    sec = time_call(torch, call, args)
    gbs = kv_bytes / sec / 1e9
    res = {"metric": f"{name}: KV GB/s", "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 5),
           "us_per_call": round(sec * 1e6, 2), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": name, "kv_bytes": kv_bytes, **extra},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": traffic_from_profiles(TRAFFIC_KEY[args.config]),
                        "bytes_per_launch": kv_bytes}}
    if not args.no_cpu_baseline and not args.eager:
        res["cpu_baseline"] = cpu_baseline_call(oracle_run, oracle_fraction, kv_bytes, oracle_sample)
    return res


def bench_prefix(args, torch):
    """Prefill hand-over of the 42-layer decode model: every layer's 4096-token
    [1, 8, 4096, 128] bf16 prefill K/V imported into an 8192 bucket (identity
    table), then the same 4096 positions exported back to dense tensors.  One
    step = 84 copy launches in one graph; bytes = what the copies must read and
    write (4 x 704.6 MB)."""
    import numpy as np

    import paged_kv_cache_194_amd as pkv
    import workloads
    from paged_kv_cache_194_amd.harness import PagedDecodeCache

    m = workloads.DecodeModel()
    n = args.ctx
    dev = torch.device("cuda:0")
    keys = [workloads.randn((1, m.kv_heads, n, m.head_dim), m.dtype, workloads.SEED_BASE + 300 + i, dev)
            for i in range(m.layers)]
    vals = [workloads.randn((1, m.kv_heads, n, m.head_dim), m.dtype, workloads.SEED_BASE + 400 + i, dev)
            for i in range(m.layers)]
    cache = PagedDecodeCache(m.layers, m.q_heads, m.kv_heads, m.head_dim, n + 1, dev, m.dtype)
    k_out = [torch.empty_like(k) for k in keys]
    v_out = [torch.empty_like(v) for v in vals]

    def import_all():
        for i in range(m.layers):
            pkv.prefix_import(cache.k[i], cache.v[i], keys[i], vals[i], cache.block_table, n,
                              seqused_k=cache.seqused if i == m.layers - 1 else None)

    def export_all():
        for i in range(m.layers):
            pkv.prefix_export(k_out[i], v_out[i], cache.k[i], cache.v[i], cache.block_table)

    def step():
        import_all()
        export_all()

    layer_bytes = 2 * n * m.kv_heads * m.head_dim * 2          # K + V of one layer
    step_bytes = 4 * m.layers * layer_bytes                      # import r+w, export r+w
    if args.eager:
        # plain launches (hardware counters are taken per dispatch)
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(args.steps):
            step()
        e.record()
        torch.cuda.synchronize()
        res = {"metric": "prefill hand-over copy GB/s (import + export)",
               "eager_us_per_step": round(s.elapsed_time(e) * 1e3 / args.steps, 2)}
        return res
    g = capture(torch, step)
    time_graph(torch, g, max(1, args.warmup))
    t_wall0 = time.perf_counter()
    sec = time_graph(torch, g, args.steps)
    wall = time.perf_counter() - t_wall0
    for i in (0, m.layers - 1):     # a cheap end-to-end check on the last replay
        if not (torch.equal(k_out[i].view(torch.int16), keys[i].view(torch.int16))
                and torch.equal(v_out[i].view(torch.int16), vals[i].view(torch.int16))):
            raise SystemExit(f"prefix round trip differs at layer {i}")
    g_imp, g_exp = capture(torch, import_all), capture(torch, export_all)
    reps = max(5, args.steps // 2)
    time_graph(torch, g_imp, 2)
    sec_imp = time_graph(torch, g_imp, reps) / m.layers
    time_graph(torch, g_exp, 2)
    sec_exp = time_graph(torch, g_exp, reps) / m.layers
    per_launch = 2 * layer_bytes                                 # read + write of one call
    gbs = step_bytes / sec / 1e9
    name = "prefix import + export, 42 layers x [1, 8, 4096, 128] bf16, identity table"
    res = {"metric": "prefill hand-over copy GB/s (import + export)", "value": round(gbs, 2),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(sec * 1e3, 5), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": name, "layers": m.layers, "positions": n, "kv_heads": m.kv_heads,
                      "head_dim": m.head_dim, "bytes_per_step": step_bytes},
           "roofline": {"bound": "hbm", "achieved": round(per_launch / sec_imp / 1e9, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(per_launch / sec_imp / 1e9 / HBM_PEAK_GBS, 4),
                        "traffic": traffic_from_profiles("prefix_import_4k"),
                        "kernel": "prefix_import call (one layer, 4096 positions)",
                        "bytes_per_launch": per_launch, "us_per_launch": round(sec_imp * 1e6, 3)},
           "roofline_export": {"bound": "hbm", "achieved": round(per_launch / sec_exp / 1e9, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(per_launch / sec_exp / 1e9 / HBM_PEAK_GBS, 4),
                               "us_per_launch": round(sec_exp * 1e6, 3)},
           "wall_s_timed": round(wall, 4)}
    if not args.no_cpu_baseline:
        import oracle
        layers = list(range(min(m.layers, args.cpu_layers)))
        host = [(keys[i].cpu().view(torch.int16).numpy(), vals[i].cpu().view(torch.int16).numpy(),
                 cache.k[i].cpu().view(torch.int16).numpy().reshape(-1, m.kv_heads, m.head_dim),
                 cache.v[i].cpu().view(torch.int16).numpy().reshape(-1, m.kv_heads, m.head_dim))
                for i in layers]
        bt = cache.block_table.cpu().numpy()
        t0 = time.perf_counter()
        for ks, vs, kc, vc in host:
            ki, vi = oracle.prefix_import(kc, vc, ks, vs, bt, n)
            oracle.prefix_export(ki, vi, bt, 1, n)
        csec = (time.perf_counter() - t0) / len(layers) * m.layers
        res["cpu_baseline"] = {"value": round(step_bytes / csec / 1e9, 4), "unit": "GB/s",
                               "cores": cpu_threads(), "kind": "oracle", "sec_per_step": round(csec, 3),
                               **host_info(),
                               "sample": f"import + export of {len(layers)} of {m.layers} layers, "
                                         "scaled to the step"}
    return res


def visible_pairs(E: int, L: int, causal: bool, window: int):
    """(union of visible keys, number of visible (query, key) pairs) of one unit."""
    lo_u, hi_u, pairs = None, 0, 0
    for i in range(L):
        p = E - L + i
        hi = min(E, p + 1) if causal else E
        lo = max(0, p - window + 1) if window > 0 else 0
        if hi > lo:
            pairs += hi - lo
            lo_u = lo if lo_u is None else min(lo_u, lo)
            hi_u = max(hi_u, hi)
    return (0 if lo_u is None else hi_u - lo_u), pairs


def bench_multirow(args, torch):
    """Column store with decode + chunked-prefill segments (c4), or the
    long-context draft-verify pass (c5): one attention call per step."""
    import numpy as np

    import paged_kv_cache_194_amd as pkv
    import workloads

    dev = torch.device("cuda:0")
    if args.config == "c4":
        inp = workloads.c4_column(device=dev)
        info = inp.seq_info.cpu().numpy()
        units = [(int(r[1]), int(r[3])) for r in info]          # (L, E)
        causal, window = True, 4096
        mk = window + inp.max_seqlen_q - 1
        out = torch.empty_like(inp.q)
        ws = torch.zeros(max(1, pkv.attn_workspace_bytes(len(units), inp.max_seqlen_q, mk, inp.q_heads,
                                                         inp.kv_heads, inp.head_dim, args.splits)),
                         dtype=torch.uint8, device=dev)

        def call():
            pkv.varlen_attn(out, inp.q, inp.k_store, inp.v_store, seq_info=inp.seq_info,
                            max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=mk, softmax_scale=inp.scale,
                            causal=True, window=window, num_splits=args.splits, workspace=ws)
        name = "column store [8192,32,8,128]: 24 decode + 8 chunked-prefill segments, causal, window 4096"

        def oracle_run():
            import oracle
            oracle.column_attention(host_bits(torch, inp.q), host_bits(torch, inp.k_store),
                                    host_bits(torch, inp.v_store), info, dtype="bf16", scale=inp.scale,
                                    causal=True, window=window, max_seqlen_q=inp.max_seqlen_q)
        oracle_seqs = None
    else:
        inp = workloads.c5_long(device=dev)
        used = inp.seqused_k.cpu().numpy()
        units = [(16, int(e)) for e in used]
        causal, window = False, 0
        out = torch.empty_like(inp.q)
        ws = torch.zeros(max(1, pkv.attn_workspace_bytes(inp.num_seqs, inp.max_seqlen_q, inp.max_seqlen_k,
                                                         inp.q_heads, inp.kv_heads, inp.head_dim, args.splits)),
                         dtype=torch.uint8, device=dev)

        def call():
            pkv.varlen_attn(out, inp.q, inp.k_cache, inp.v_cache, cu_seqlens_q=inp.cu_seqlens_q,
                            seqused_k=inp.seqused_k, block_table=inp.block_table, max_seqlen_q=16,
                            max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, causal=False,
                            num_splits=args.splits, workspace=ws)
        name = "long-context draft verify: 4 x 16-token blocks over 32K/64K keys, 64 q / 8 kv heads, D 256"

        def oracle_run():
            import oracle
            oracle.paged_attention(host_bits(torch, inp.q), host_bits(torch, inp.k_cache),
                                   host_bits(torch, inp.v_cache), inp.block_table.cpu().numpy(),
                                   inp.cu_seqlens_q.cpu().numpy(), used, dtype="bf16", scale=inp.scale,
                                   causal=False, max_seqlen_q=16, max_seqlen_k=inp.max_seqlen_k,
                                   seqs=[0, 1])
        oracle_seqs = [0, 1]
    keys = pairs = sample_pairs = 0
    for u, (L, E) in enumerate(units):
        k_u, p_u = visible_pairs(E, L, causal, window)
        keys += k_u
        pairs += p_u
        if oracle_seqs is None or u in oracle_seqs:
            sample_pairs += p_u
    kv_bytes = keys * inp.kv_heads * inp.head_dim * 2 * 2
    flops = 4 * inp.head_dim * inp.q_heads * pairs
    sec = time_call(torch, call, args)
    gbs, tfs = kv_bytes / sec / 1e9, flops / sec / 1e12
    hbm_frac, mfma_frac = gbs / HBM_PEAK_GBS, tfs / 2500.0
    bound = "hbm" if kv_bytes / (HBM_PEAK_GBS * 1e9) >= flops / 2.5e15 else "mfma"
    prof = profile_record(TRAFFIC_KEY[args.config])
    roof = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(hbm_frac, 4)} if bound == "hbm" else
            {"bound": "mfma", "achieved": round(tfs, 2), "peak": 2500.0, "unit": "TFLOP/s",
             "frac": round(mfma_frac, 4)})
    roof.update({"traffic": prof.get("hbm_bytes_per_launch"), "bytes_per_launch": kv_bytes,
                 "flops_per_launch": flops,
                 # busy cycles of every MFMA issued (masked keys included) over the
                 # kernel's SIMD-cycles, from the committed counter record
                 "mfma_busy_pct": prof.get("mfma_busy_pct")})
    res = {"metric": f"{name}: KV GB/s", "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 5),
           "us_per_call": round(sec * 1e6, 2), "pct_hbm_peak": round(100 * hbm_frac, 2),
           "tflops": round(tfs, 2), "pct_mfma_peak": round(100 * mfma_frac, 2),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": name, "kv_bytes": kv_bytes, "flops": flops},
           "roofline": roof}
    if not args.no_cpu_baseline and not args.eager:
        sample = ("all 32 segments" if oracle_seqs is None else
                  f"sequences {oracle_seqs} of {len(units)}, scaled by visible query-key pairs")
        res["cpu_baseline"] = cpu_baseline_call(oracle_run, sample_pairs / pairs, kv_bytes,
                                                sample + " (host copies of the inputs included)")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2", choices=["c2", "c3", "c4", "c5", "c5d", "prefix"])
    ap.add_argument("--ctx", type=int, default=4096, help="live keys of the 42-layer decode step")
    ap.add_argument("--splits", type=int, default=0, help="split-K partitions (0: library choice)")
    ap.add_argument("--cpu-layers", type=int, default=42, help="layers the CPU oracle times")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip the 4 GiB device copy timed as the practical HBM ceiling")
    ap.add_argument("--copy-ceiling", action="store_true", help="time the device copy (the default)")
    ap.add_argument("--eager", action="store_true",
                    help="plain launches instead of graph replays (for per-dispatch counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the benchmark runs the single-GPU hot path, so --gpus must be 1"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    import paged_kv_cache_194_amd as pkv
    pkv.lib()        # fail loudly if the library is missing
    if args.config == "c2":
        res = bench_decode_step(args, torch)
    elif args.config == "prefix":
        res = bench_prefix(args, torch)
    else:
        res = bench_single_call(args, torch)
    if not args.no_copy_ceiling:
        ceil = copy_ceiling_gbs(torch)
        res["copy_ceiling_gbs"] = round(ceil, 1)
        if "value" in res and res.get("unit") == "GB/s":
            res["pct_copy_ceiling"] = round(100 * res["value"] / ceil, 2)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
