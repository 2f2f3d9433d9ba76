#!/usr/bin/env python3
"""Benchmark: one batch-invariant decode step of a Llama-3.1-8B-shaped attention layer.

Step (every row of the hot path, on one batch of synthetic input resident in HBM):
  RMSNorm(x) -> QKV GEMM [B,4096]x[6144,4096]^T -> slot mapping + KV write of the
  new token -> paged attention (split phase and fixed-order merge; at this batch one
  launch of the row-group mapping) -> O GEMM [B,4096]x[4096,4096]^T
Geometry: 32 query / 8 KV heads, head_dim 128, pages of 16 tokens, fixed key split
256, context lengths ~ U{512..8192}, K/V/x ~ N(0,1) bf16, weights ~ N(0, 0.02),
gamma ~ N(1, 0.1).  Random-init, synthetic data.

Prints ONE JSON line.  `value` = algorithmic HBM bytes of the whole step / step
time (GB/s).  `roofline` is for the dominant kernel (the attention launch),
timed with HIP events recorded on the stream it is launched on.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

Other workloads (one JSON line each, same keys; not the headline):
  --workload decode-sweep   the same attention layer at batch 1, 8, 64 and 256 (MALL
                            flushed before every timed repetition), vs split-K
  --workload gemm           RMSNorm + GEMM, hidden 4096, M in {1, 7, 64, 256, 1024},
                            N in {14336 (bf16 out), 128256 (fp32 logits)}, vs split-K
  --workload prefill        chunked prefill with a shared 1024-token prefix (8
                            requests), chunk budgets {16, 128, 512} and token by token
  --workload gemma          one decode step of a 34-layer Gemma-3-4B-shaped decoder
                            (replayed as one HIP graph)
  --workload agentic        4 sessions x 6 turns through the engine on that decoder:
                            16K-token prompts over an 8K cached shared prefix, +256
                            input and 768 output tokens per turn, 0.5 s user delay
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "batch-invariant paged-attn decode HBM GB/s (% peak) + overhead vs split-K"
# bi_paged_attention_mapping's answer, by value.
MAPPING_NAMES = {0: "split + merge", 1: "row-group"}
PEAK_HBM_GBPS = 8000.0
HQ, HKV, D, P, S = 32, 8, 128, 16, 256
DEFAULT_LOCAL_SPLIT = 128  # the decoder shape's windowed-layer split size
DEFAULT_GLOBAL_SPLIT = 256  # and its global layers'
HIDDEN = 4096
QKV_N = (HQ + 2 * HKV) * D
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_decode_b256_traffic.json")
KERNEL_SOURCES = ["deterministic_paged_attention_amd/csrc/attention.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(batch: int):
    """HBM bytes per attention launch (the row-group kernel at batch 256) from
    committed rocprofv3 counter runs, if they were taken on the current kernel
    source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_source_hash() or t.get("batch") != batch:
        return None
    return t.get("hbm_bytes_per_launch")


def measured_stream_read(stream, nbytes=4 << 30, reps=10):
    """Bandwidth of the library's plain streaming-read reference kernel over one
    contiguous 4 GiB buffer (about the split kernel's 4.5 GB), timed with HIP
    events on the stream it runs on; median of `reps` launches: the same GPU's
    practical read ceiling, quoted beside the published 8 TB/s."""
    import torch
    import deterministic_paged_attention_amd as bi
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(bi.lib.bi_bench_stream_read_sink_words(), dtype=torch.int32, device="cuda")
    for _ in range(3):
        bi.bi_bench_stream_read(src, sink, stream)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        bi.bi_bench_stream_read(src, sink, stream)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    ts.sort()
    del src
    torch.cuda.empty_cache()
    t = ts[len(ts) // 2]
    return {"gbps": round(nbytes / t / 1e9, 1), "bytes": nbytes, "us": round(t * 1e6, 1)}


def measured_mfma_peak(rounds=4096, reps=10):
    """Rate of the library's MFMA throughput reference (the GEMM's own bf16
    16x16x32 instruction, eight independent accumulators per wave, a full grid),
    timed with HIP events on the current stream; median of `reps` launches of
    about 1.1 TFLOP each: the matrix-core rate this GPU sustains, quoted beside
    the published dense peak."""
    import torch
    import deterministic_paged_attention_amd as bi
    stream = torch.cuda.current_stream()
    sink, flops = bi.bi_bench_mfma_peak(rounds, 0.0, stream=stream)
    for _ in range(2):
        bi.bi_bench_mfma_peak(rounds, 0.0, sink, stream)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        bi.bi_bench_mfma_peak(rounds, 0.0, sink, stream)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    ts.sort()
    t = ts[len(ts) // 2]
    return {"tflops": round(flops / t / 1e12, 1), "flops_per_launch": flops, "us": round(t * 1e6, 1)}


def split_bytes(lengths):
    """Algorithmic bytes of one split-phase launch: K+V of every visible key,
    Q, and the page-table entries read."""
    kv = sum(2 * L * HKV * D * 2 for L in lengths)
    q = len(lengths) * HQ * D * 2
    pt = sum(4 * ((L + P - 1) // P) for L in lengths)
    return kv + q + pt


def step_bytes(lengths):
    B = len(lengths)
    rms = 2 * B * HIDDEN * 2 + 2 * HIDDEN
    qkv = 2 * B * HIDDEN + 2 * QKV_N * HIDDEN + 2 * B * QKV_N
    slot = B * (4 + 4 + 4) + 4 * B
    kvw = 2 * (B * HKV * D * 2) * 2
    merge = B * HQ * D * 2
    oproj = 2 * B * HIDDEN + 2 * HIDDEN * HIDDEN + 2 * B * HIDDEN
    return rms + qkv + slot + kvw + split_bytes(lengths) + merge + oproj


def cpu_baseline(wl, sample_seqs: int):
    """The oracle, as it stands, on the first `sample_seqs` sequences of the workload
    (each sequence copied to the host untimed, then attended by the oracle timed)."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    dt = 0.0
    lens = []
    for s in range(sample_seqs):
        kk, vv, table, L = wl.host_sequence(s)
        q = synth.to_f64(wl.q[s:s + 1].cpu())
        t0 = time.perf_counter()
        oracle.attention_ref(q, kk, vv, table, [L], [0, 1], HKV, P)
        dt += time.perf_counter() - t0
        lens.append(L)
    nbytes = split_bytes(lens) + sample_seqs * HQ * D * 2
    out = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"float64 numpy attention oracle over {sample_seqs} of the {wl.batch} decode sequences of the "
                     f"same workload (same bytes-per-sequence accounting as the GPU), {dt:.1f} s of oracle time",
           "affinity_cores": len(os.sched_getaffinity(0))}
    # The same oracle on one BLAS thread, over the first few sequences.
    try:
        from threadpoolctl import threadpool_limits
        n1 = min(64, sample_seqs)
        dt1, lens1 = 0.0, []
        with threadpool_limits(limits=1, user_api="blas"):
            for s in range(n1):
                kk, vv, table, L = wl.host_sequence(s)
                q = synth.to_f64(wl.q[s:s + 1].cpu())
                t0 = time.perf_counter()
                oracle.attention_ref(q, kk, vv, table, [L], [0, 1], HKV, P)
                dt1 += time.perf_counter() - t0
                lens1.append(L)
        out["single_core"] = {"value": round((split_bytes(lens1) + n1 * HQ * D * 2) / dt1 / 1e9, 4), "unit": "GB/s",
                              "cores": 1, "sample": f"the first {n1} sequences, {dt1:.1f} s of oracle time"}
    except ImportError:  # pragma: no cover
        pass
    return out


def bench_decode(args):
    import torch
    import deterministic_paged_attention_amd as bi
    import synth
    from synth.workloads import build_decode_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    B = args.batch
    cfg = bi.AttnConfig(HQ, HKV, D, page_size=P, split_size=S)
    wl = build_decode_workload(HQ, HKV, D, batch=B, seed=args.seed)
    lengths = wl.lengths
    x = synth.normal_bf16_device((B, HIDDEN), args.seed + 10)
    gamma = synth.normal_bf16_device((HIDDEN,), args.seed + 11, std=0.1, mean=1.0)
    w_qkv = synth.normal_bf16_device((QKV_N, HIDDEN), args.seed + 12, std=0.02)
    w_o = synth.normal_bf16_device((HIDDEN, HQ * D), args.seed + 13, std=0.02)
    torch.cuda.synchronize()

    xn = torch.empty((B, HIDDEN), dtype=torch.bfloat16, device=dev)
    qkv = torch.empty((B, QKV_N), dtype=torch.bfloat16, device=dev)
    q = qkv[:, : HQ * D].view(B, HQ, D)
    k_new = qkv[:, HQ * D: (HQ + HKV) * D].view(B, HKV, D)
    v_new = qkv[:, (HQ + HKV) * D:].view(B, HKV, D)
    attn = torch.empty((B, HQ, D), dtype=torch.bfloat16, device=dev)
    y = torch.empty((B, HIDDEN), dtype=torch.bfloat16, device=dev)
    ws = bi.alloc_workspace(bi.bi_paged_attention_workspace_size(cfg, B, B, wl.max_seq_len))
    stream = torch.cuda.current_stream()

    # slot mapping + KV write as one launch (bi_kv_write_paged: slots from the page table);
    # attention through bi_paged_attention, which runs the row-group mapping (split
    # and merge in one launch, partials in LDS) for a batch that fills the GPU, else
    # the split and merge phases
    mapping = bi.bi_paged_attention_mapping(cfg, B, B, wl.max_seq_len)
    names = ["rmsnorm", "gemm_qkv", "kv_write", "attention", "gemm_o"]
    launches = [
        lambda: bi.bi_rmsnorm(x, gamma, 1e-5, out=xn),
        lambda: bi.bi_gemm(xn, w_qkv, out=qkv),
        lambda: bi.bi_kv_write_paged(cfg, k_new, v_new, wl.page_table, wl.seq_lens, wl.qsl, wl.k_cache, wl.v_cache),
        lambda: bi.bi_paged_attention(cfg, q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.qsl,
                                      wl.max_seq_len, workspace=ws, out=attn),
        lambda: bi.bi_gemm(attn.view(B, HQ * D), w_o, out=y),
    ]

    ATTN = names.index("attention")

    def step(events=None):
        """One decode step.  events: (before, after) the attention launch(es), on their stream."""
        for i, f in enumerate(launches):
            if events is not None and i == ATTN:
                events[0].record(stream)
            f()
            if events is not None and i == ATTN:
                events[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps; the only events inside bracket the attention
    # launch (its duration feeds the roofline).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(ev[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    attn_launch_us = statistics.mean(ev[k][0].elapsed_time(ev[k][1]) for k in range(args.steps)) * 1e3

    # Per-kernel breakdown, after the timed region: events around every launch.
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        for i, f in enumerate(launches):
            bev[k][i].record(stream)
            f()
        bev[k][-1].record(stream)
    torch.cuda.synchronize()
    per_kernel = {n: statistics.mean(bev[k][i].elapsed_time(bev[k][i + 1]) for k in range(args.steps)) * 1e3
                  for i, n in enumerate(names)}

    # Algorithmic bytes of the attention launch: K+V of every visible key, Q,
    # page-table entries, and the output rows.
    sb = split_bytes(lengths) + B * HQ * D * 2
    achieved = sb / (attn_launch_us * 1e-6) / 1e9
    value = step_bytes(lengths) / (ms_per_step * 1e-3) / 1e9
    attn_us = per_kernel["attention"]
    attn_gbps = sb / (attn_us * 1e-6) / 1e9

    splitk = None
    if not args.no_splitk:
        # The comparator is the fastest of the split counts a batch-aware kernel
        # could pick (the heuristic's choice among them), so the overhead is
        # measured against the best non-invariant schedule, not a weak one.
        props = torch.cuda.get_device_properties(0)
        heur = bi.bi_splitk_attention_heuristic(cfg, B, wl.max_seq_len, props.multi_processor_count, 8)
        candidates = sorted({heur, 1, 2, 4, 8, 16, 32})
        out_k = torch.empty_like(attn)

        def run_inv():
            launches[ATTN]()

        def splitk_runner(n):
            ws_k = bi.alloc_workspace(bi.bi_paged_attention_splitk_workspace_size(cfg, B, B, wl.max_seq_len, n))

            def run():
                bi.bi_paged_attention_splitk(cfg, q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.qsl,
                                             wl.max_seq_len, n, workspace=ws_k, out=out_k)
            return run

        def timeit(f, reps=max(10, args.steps)):
            for _ in range(3):
                f()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(reps):
                f()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps * 1e3

        t_inv = timeit(run_inv)
        per_n = {n: timeit(splitk_runner(n)) for n in candidates}
        best = min(per_n, key=per_n.get)
        splitk = {"invariant_us": round(t_inv, 2), "splitk_us": round(per_n[best], 2), "splitk_num_splits": best,
                  "heuristic_num_splits": heur, "splitk_us_by_num_splits": {str(n): round(v, 2) for n, v in per_n.items()},
                  "overhead": round(t_inv / per_n[best] - 1.0, 4)}

    read_ref = measured_stream_read(stream)

    # The oracle runs after the GPU timing: its BLAS threads keep spinning for a
    # while after each call and would delay the host launching the timed steps.
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, min(args.cpu_sample, B))

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 2
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3.1-8b-shaped attention layer, batch-invariant decode step",
                   "batch": B, "context_lengths": "U{512..8192}", "mean_context": round(sum(lengths) / B, 1),
                   "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "page_size": P, "split_size": S,
                   "hidden": HIDDEN, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(B),
                     "kernel": "attn_rowgroup_kernel<128>" if mapping == 1 else
                               "attn_split_kernel<128, 1> + attn_merge_kernel<128>",
                     "algorithmic_bytes_per_launch": sb,
                     "avg_launch_us": round(attn_launch_us, 2), "mapping": MAPPING_NAMES[mapping],
                     "measured_stream_read_gbps": read_ref["gbps"],
                     "frac_of_measured_stream_read": round(achieved / read_ref["gbps"], 4)},
        "cpu_baseline": cpu,
        "attention_gbps": round(attn_gbps, 2),
        "attention_frac_of_peak": round(attn_gbps / PEAK_HBM_GBPS, 4),
        "splitk": splitk,
        "kernels_us": {k: round(v, 2) for k, v in per_kernel.items()},
        "kernel_sha": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# Secondary workloads (not the headline line).
# ---------------------------------------------------------------------------
PEAK_BF16_TFLOPS = 2500.0
FLUSH_BYTES = 1 << 30   # > the 256 MB MALL


def _torch_env():
    import torch
    import deterministic_paged_attention_amd as bi
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    return torch, bi, synth


def rep_times_ms(fn, reps, flush=None):
    """Duration (ms) of each of `reps` calls of fn, from HIP events recorded on the
    current stream around each call; `flush()` runs before each call, untimed."""
    import torch
    stream = torch.cuda.current_stream()
    pairs = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def pct(ts):
    import numpy as np
    return {"median": float(np.median(ts)), "p10": float(np.percentile(ts, 10)), "p90": float(np.percentile(ts, 90))}


def mall_flusher():
    """Evicts the MALL and L2 by reading 1 GiB.  A read, not a write: a write
    would leave the caches full of dirty lines whose write-back the next timed
    kernel would pay for."""
    import torch
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty((), dtype=torch.int32, device="cuda")
    return lambda: torch.amax(buf, dim=0, out=sink)


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        return 1


def bench_decode_sweep(args):
    """Batch-invariant attention (bi_paged_attention: the split and merge phases, or
    the row-group mapping once the batch fills the GPU) of the 8B-shaped decode layer
    at batch 1, 8, 64 and 256 (the first B sequences of one 256-sequence pool), MALL
    flushed before each repetition, against the fastest split-K split count."""
    torch, bi, synth = _torch_env()
    from synth.workloads import build_decode_workload
    cfg = bi.AttnConfig(HQ, HKV, D, page_size=P, split_size=S)
    pool = synth.llama8b_decode_lengths(256, args.seed)
    flush = mall_flusher()
    reps = max(args.steps, 20)
    props = torch.cuda.get_device_properties(0)
    rows = []
    for B in [int(b) for b in args.batches.split(",")]:
        wl = build_decode_workload(HQ, HKV, D, batch=B, seed=args.seed, lengths=pool[:B])
        ws = bi.alloc_workspace(bi.bi_paged_attention_workspace_size(cfg, B, B, wl.max_seq_len))
        out = torch.empty((B, HQ, D), dtype=torch.bfloat16, device="cuda")

        def inv():
            bi.bi_paged_attention(cfg, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.qsl,
                                  wl.max_seq_len, workspace=ws, out=out)
        inv()
        t_inv = pct(rep_times_ms(inv, reps, flush))
        heur = bi.bi_splitk_attention_heuristic(cfg, B, wl.max_seq_len, props.multi_processor_count, 8)
        per_n = {}
        for n in sorted({heur, 1, 2, 4, 8, 16, 32}):
            ws_k = bi.alloc_workspace(bi.bi_paged_attention_splitk_workspace_size(cfg, B, B, wl.max_seq_len, n))

            def sk():
                bi.bi_paged_attention_splitk(cfg, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.qsl,
                                             wl.max_seq_len, n, workspace=ws_k, out=out)
            sk()
            per_n[n] = pct(rep_times_ms(sk, reps, flush))["median"]
            del ws_k
        best = min(per_n, key=per_n.get)
        nbytes = split_bytes(wl.lengths) + B * HQ * D * 2
        gbps = nbytes / (t_inv["median"] * 1e-3) / 1e9
        mapping = bi.bi_paged_attention_mapping(cfg, B, B, wl.max_seq_len)
        rows.append({"batch": B, "mapping": MAPPING_NAMES[mapping],
                     "algorithmic_bytes": nbytes, "invariant_ms": {k: round(v, 4) for k, v in t_inv.items()},
                     "gbps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
                     "splitk_ms": round(per_n[best], 4), "splitk_num_splits": best, "heuristic_num_splits": heur,
                     "overhead_vs_splitk": round(t_inv["median"] / per_n[best] - 1.0, 4)})
        print(json.dumps({"progress": rows[-1]}), file=sys.stderr, flush=True)
        del wl, ws
        torch.cuda.empty_cache()
    top = rows[-1]
    print(json.dumps({
        "metric": METRIC, "value": top["gbps"], "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": top["invariant_ms"]["median"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3.1-8b-shaped decode attention (split + merge), batch sweep, MALL flushed per rep",
                   "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "page_size": P, "split_size": S,
                   "context_lengths": "U{512..8192}"},
        "rows": rows}), flush=True)


def bench_gemm(args):
    """RMSNorm (hidden 4096) then the M-independent GEMM against [N, 4096] weights,
    per (N, M); MALL flushed before each repetition.  Comparator: the fastest of
    the split-K counts {1, 2, 4, 8, 16} whose fp32 partials fit in 2 GiB."""
    torch, bi, synth = _torch_env()
    K = 4096
    reps = max(args.steps, 20)
    flush = mall_flusher()
    rows = []
    cpu = None
    for N, odt in ((14336, torch.bfloat16), (128256, torch.float32)):
        W = synth.normal_bf16_device((N, K), args.seed + 40 + N % 7, std=0.02)
        for M in [int(m) for m in args.ms.split(",")]:
            x = synth.normal_bf16_device((M, K), args.seed + 50 + M)
            g = synth.normal_bf16_device((K,), args.seed + 49, std=0.1, mean=1.0)
            xn = torch.empty_like(x)
            c = torch.empty((M, N), dtype=odt, device="cuda")
            rms = lambda: bi.bi_rmsnorm(x, g, 1e-5, out=xn)  # noqa: E731
            gem = lambda: bi.bi_gemm(xn, W, out=c)  # noqa: E731
            rms()
            gem()
            t_rms = pct(rep_times_ms(rms, reps, flush))
            t_gemm = pct(rep_times_ms(gem, reps, flush))
            per_k = {}
            for ks in (1, 2, 4, 8, 16):
                if K % (32 * ks) or M * N * 4 * ks > (2 << 30) or (args.no_splitk and ks > 1):
                    continue
                ws = torch.empty(M * N * ks, dtype=torch.float32, device="cuda")
                c2 = torch.empty_like(c)
                sk = lambda: bi.bi_gemm_splitk(xn, W, ks, out=c2, workspace=ws)  # noqa: E731
                sk()
                per_k[ks] = pct(rep_times_ms(sk, reps, flush))["median"]
                del ws, c2
            best = min(per_k, key=per_k.get)
            flops = 2.0 * M * N * K
            nbytes = 2 * M * K + 2 * N * K + (4 if odt == torch.float32 else 2) * M * N
            t_mfma, t_hbm = flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBPS * 1e9)
            tm = t_gemm["median"] * 1e-3
            rows.append({
                "N": N, "M": M, "out": "fp32" if odt == torch.float32 else "bf16",
                "rmsnorm_us": round(t_rms["median"] * 1e3, 2),
                "rmsnorm_gbps": round((4 * M * K + 2 * K) / (t_rms["median"] * 1e-3) / 1e9, 1),
                "gemm_us": {k: round(v * 1e3, 2) for k, v in t_gemm.items()},
                "gemm_tflops": round(flops / tm / 1e12, 1), "gemm_gbps": round(nbytes / tm / 1e9, 1),
                "bound": "mfma" if t_mfma > t_hbm else "hbm",
                "roofline_us": round(max(t_mfma, t_hbm) * 1e6, 2),
                "frac_of_roofline": round(max(t_mfma, t_hbm) / tm, 4),
                "mfma_frac_of_bf16_peak": round(flops / tm / 1e12 / PEAK_BF16_TFLOPS, 4),
                "splitk_us": round(per_k[best] * 1e3, 2), "splitk_k_splits": best,
                "overhead_vs_splitk": round(t_gemm["median"] / per_k[best] - 1.0, 4)})
            print(json.dumps({"progress": rows[-1]}), file=sys.stderr, flush=True)
            del x, xn, c
        if not args.no_cpu_baseline and N == 14336:
            w_host = W.cpu()          # the oracle runs after all GPU timing (its BLAS threads spin on)
        del W
        torch.cuda.empty_cache()
    mfma_ref = measured_mfma_peak()
    for r in rows:
        r["mfma_frac_of_measured_peak"] = round(r["gemm_tflops"] / mfma_ref["tflops"], 4)
    if not args.no_cpu_baseline:
        cpu = gemm_cpu_baseline(w_host, args.seed)
    head = ([r for r in rows if r["N"] == 14336 and r["M"] == 256] or rows)[0]
    print(json.dumps({
        "metric": "batch-invariant RMSNorm + GEMM: GEMM fraction of roofline", "value": head["frac_of_roofline"],
        "unit": "fraction of min(bf16 MFMA peak, HBM) roofline", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": head["gemm_us"]["median"] / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "rmsnorm + gemm, K 4096, M {1,7,64,256,1024} x N {14336 bf16, 128256 fp32}, "
                               "MALL flushed per rep", "value_row": "N 14336, M 256"},
        "measured_mfma_peak": mfma_ref, "rows": rows, "cpu_baseline": cpu}), flush=True)


def gemm_cpu_baseline(W, seed):
    """The oracle's RMSNorm + matmul (fp64 numpy) for M = 64 rows against the
    [14336, 4096] weight, timed on the host."""
    import oracle
    import synth
    x = synth.to_f64(synth.normal_bf16((64, W.shape[1]), seed + 77))
    g = synth.to_f64(synth.normal_bf16((W.shape[1],), seed + 78, std=0.1, mean=1.0))
    w = synth.to_f64(W)
    t0 = time.perf_counter()
    xn = oracle.rmsnorm_ref(x, g, 1e-5)
    oracle.gemm_ref(xn, w)
    dt = time.perf_counter() - t0
    flops = 2.0 * 64 * W.shape[0] * W.shape[1]
    return {"value": round(flops / dt / 1e9, 2), "unit": "GFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"float64 numpy rmsnorm + matmul, M 64 x N {W.shape[0]} x K {W.shape[1]}, {dt:.2f} s"}


def prefill_schedule(unique, budget):
    """Steps of a chunked prefill: request 0 computes the 1024-token prefix alone,
    then every request continues from it (shared pages).  A step takes up to
    `budget` tokens in request order; budget 0 means token by token (one row per
    live request).  Each step is a list of (request, first position, tokens)."""
    total = [1024 + u for u in unique]
    steps = []
    pos = 0
    while pos < 1024:
        n = 1 if budget == 0 else min(budget, 1024 - pos)
        steps.append([(0, pos, n)])
        pos += n
    done = [1024] * len(unique)
    while any(d < t for d, t in zip(done, total)):
        st, left = [], budget
        for r in range(len(unique)):
            if done[r] >= total[r]:
                continue
            if budget == 0:
                n = 1
            else:
                if left == 0:
                    break
                n = min(left, total[r] - done[r])
                left -= n
            st.append((r, done[r], n))
            done[r] += n
        steps.append(st)
    return steps


def bench_prefill(args):
    """Attention (split + merge) over every step of a chunked-prefill schedule of
    8 requests sharing a 1024-token prefix, each with U{256..2048} unique tokens.
    The paged cache is filled beforehand; each schedule is captured as one HIP
    graph and replayed."""
    torch, bi, synth = _torch_env()
    cfg = bi.AttnConfig(HQ, HKV, D, page_size=P, split_size=S)
    nreq = 8
    unique = synth.uniform_ints(nreq, 256, 2048, args.seed + 60)
    total = [1024 + u for u in unique]
    shared = synth.pages_needed(1024, P)
    perm = synth.permutation(shared + sum(synth.pages_needed(u, P) for u in unique) + 16, args.seed + 61)
    prefix_pages, cur = perm[:shared], shared
    tables = []
    for u in unique:
        n = synth.pages_needed(u, P)
        tables.append(prefix_pages + perm[cur:cur + n])
        cur += n
    num_pages = len(perm)
    k_cache = synth.normal_bf16_device(cfg.k_cache_shape(num_pages), args.seed + 62)
    v_cache = synth.normal_bf16_device(cfg.v_cache_shape(num_pages), args.seed + 63)
    q_all = synth.normal_bf16_device((1024 + max(total), HQ, D), args.seed + 64)
    stride = max(len(t) for t in tables)
    flush = mall_flusher()
    rows = []
    for budget in [int(b) for b in args.budgets.split(",")]:
        steps = prefill_schedule(unique, budget)
        meta = []
        max_ws = 0
        for st in steps:
            pt = torch.tensor([tables[r] + [-1] * (stride - len(tables[r])) for r, _, _ in st], dtype=torch.int32)
            sl = [s0 + n for _, s0, n in st]
            ql = [n for _, _, n in st]
            T = sum(ql)
            qsl = [0]
            for n in ql:
                qsl.append(qsl[-1] + n)
            meta.append((pt.cuda(), torch.tensor(sl, dtype=torch.int32, device="cuda"),
                         torch.tensor(qsl, dtype=torch.int32, device="cuda"), T, max(sl), q_all[:T]))
            max_ws = max(max_ws, bi.bi_paged_attention_workspace_size(cfg, len(st), T, max(sl)))
        ws = bi.alloc_workspace(max_ws)
        outs = [torch.empty((m[3], HQ, D), dtype=torch.bfloat16, device="cuda") for m in meta]

        def run_all():
            for (pt, sl, qsl, T, msl, q), o in zip(meta, outs):
                bi.bi_paged_attention(cfg, q, k_cache, v_cache, pt, sl, qsl, msl, workspace=ws, out=o)
        run_all()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_all()
        graph.replay()
        torch.cuda.synchronize()
        t = pct(rep_times_ms(graph.replay, max(3, min(args.steps, 10)), flush))
        flops = 0
        kv_bytes = 0
        tokens = 0
        for st in steps:
            for _, s0, n in st:
                tokens += n
                flops += sum(4 * D * HQ * (s0 + j + 1) for j in range(n))
                kv_bytes += 2 * (s0 + n) * HKV * D * 2
        sec = t["median"] * 1e-3
        rows.append({"budget": budget or "token-by-token", "steps": len(steps), "tokens": tokens,
                     "ms": {k: round(v, 3) for k, v in t.items()}, "tokens_per_s": round(tokens / sec, 1),
                     "tflops": round(flops / sec / 1e12, 2), "mfma_frac_of_bf16_peak": round(flops / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "kv_gbps": round(kv_bytes / sec / 1e9, 1), "algorithmic_flops": flops, "kv_bytes": kv_bytes})
        print(json.dumps({"progress": rows[-1]}), file=sys.stderr, flush=True)
        del graph, meta, outs, ws
        torch.cuda.empty_cache()
    head = ([r for r in rows if r["budget"] == 512] or rows)[0]
    print(json.dumps({
        "metric": "batch-invariant chunked prefill attention tokens/s", "value": head["tokens_per_s"],
        "unit": "tokens/s", "n_gpus": 1, "steps": len(rows), "warmup": 1, "ms_per_step": head["ms"]["median"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "8 requests, shared 1024-token prefix + U{256..2048} unique tokens, llama3.1-8b-shaped "
                               "attention layer, chunk budgets {16,128,512} and token by token",
                   "unique_tokens": unique, "value_row": "budget 512"},
        "rows": rows}), flush=True)


def bench_gemma(args):
    """One decode step (one new token per sequence) of the 34-layer Gemma-3-4B-shaped
    decoder over a paged cache, captured as one HIP graph and replayed."""
    torch, bi, synth = _torch_env()
    from deterministic_paged_attention_amd.decoder import Decoder, DecoderShape
    from synth.workloads import decoder_weights
    s = DecoderShape(split_size=args.global_split, split_size_local=args.local_split)
    B = args.batch
    ctx = synth.uniform_ints(B, 512, 4096, args.seed + 70)
    w = decoder_weights(s.layers, s.hidden, s.q_heads, s.kv_heads, s.head_dim, s.ffn, s.vocab, seed=args.seed + 71)
    dec = Decoder(s, w)
    k_lens = [L + 1 for L in ctx]
    need = [synth.pages_needed(L, s.page_size) for L in k_lens]
    num_pages = sum(need) + 16
    perm = synth.permutation(num_pages, args.seed + 72)
    tables, cur = [], 0
    for n in need:
        tables.append(perm[cur:cur + n])
        cur += n
    stride = max(need)
    pt = torch.tensor([t + [-1] * (stride - len(t)) for t in tables], dtype=torch.int32, device="cuda")
    caches = dec.new_caches(num_pages)
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed + 73)
    for k, v in caches:
        k.normal_(generator=g)
        v.normal_(generator=g)
    ids = torch.tensor(synth.uniform_ints(B, 0, s.vocab - 1, args.seed + 74), dtype=torch.int32, device="cuda")
    sl = torch.tensor(k_lens, dtype=torch.int32, device="cuda")
    qsl = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    step = lambda: dec.step(ids, caches, pt, sl, qsl, max(k_lens))  # noqa: E731
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        logits = step()
    for _ in range(max(1, args.warmup)):
        graph.replay()
    torch.cuda.synchronize()
    ts = rep_times_ms(graph.replay, args.steps)
    t = pct(ts)
    eager = pct(rep_times_ms(step, 3))
    per_layer = s.qkv_width * s.hidden + s.hidden * s.q_heads * s.head_dim + 2 * s.ffn * s.hidden + s.hidden * s.ffn
    n_global = sum(1 for l in range(s.layers) if s.is_global(l))
    n_local = s.layers - n_global
    w_bytes = 2 * (s.layers * per_layer + s.vocab * s.hidden)
    kv_token = 2 * s.kv_heads * s.head_dim * 2
    kv_read = sum(kv_token * (n_local * min(L, s.window) + n_global * L) for L in k_lens)
    kv_write = s.layers * B * kv_token
    logits_bytes = B * s.vocab * 4
    nbytes = w_bytes + kv_read + kv_write + logits_bytes
    sec = t["median"] * 1e-3
    cpu = None if args.no_cpu_baseline else gemma_cpu_baseline(dec, ctx[0], args.seed)
    print(json.dumps({
        "metric": "batch-invariant decoder decode step: tokens/s", "value": round(B / sec, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t["median"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gemma-3-4b-shaped decoder (random init), one decode token per sequence, HIP graph",
                   "batch": B, "context_lengths": "U{512..4096}", "mean_context": round(sum(ctx) / B, 1),
                   "layers": s.layers, "hidden": s.hidden, "q_heads": s.q_heads, "kv_heads": s.kv_heads,
                   "head_dim": s.head_dim, "ffn": s.ffn, "vocab": s.vocab, "window": s.window,
                   "global_layers": n_global, "split_size": s.split_size, "split_size_local": s.split_size_local},
        "step_ms": {k: round(v, 4) for k, v in t.items()}, "eager_step_ms": round(eager["median"], 4),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / sec / 1e9, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(nbytes / sec / 1e9 / PEAK_HBM_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_step": nbytes, "weight_bytes": w_bytes, "kv_read_bytes": kv_read},
        "logits_shape": list(logits.shape), "cpu_baseline": cpu}), flush=True)


def gemma_cpu_baseline(dec, ctx_len, seed):
    """The oracle's per-op chain for one layer (layer 0, local) at batch 1 with a
    context of ctx_len tokens (fp64 numpy), timed on the host."""
    import numpy as np
    import oracle
    import synth
    s = dec.shape
    W = {k: synth.to_f64(v.cpu()) for k, v in dec.w["layers"][0].items()}
    L = ctx_len + 1
    h = synth.to_f64(synth.normal_bf16((1, s.hidden), seed + 80))
    kc = synth.to_f64(synth.normal_bf16((synth.pages_needed(L, s.page_size), s.page_size, s.kv_heads, s.head_dim),
                                        seed + 81))
    vc = synth.to_f64(synth.normal_bf16(kc.shape, seed + 82))
    Hq, Hk, D = s.q_heads, s.kv_heads, s.head_dim
    t0 = time.perf_counter()
    xn = oracle.rmsnorm_ref(h, W["g_attn"], s.eps)
    qkv = oracle.gemm_ref(xn, W["w_qkv"])
    q, k = oracle.qk_norm_rope_ref(qkv[:, :Hq * D].reshape(1, Hq, D), qkv[:, Hq * D:(Hq + Hk) * D].reshape(1, Hk, D),
                                   W["g_q"], W["g_k"], s.eps, [L - 1], s.theta_local)
    table = np.arange(kc.shape[0])[None, :]
    o = oracle.attention_ref(q, kc, vc, table, [L], [0, 1], Hk, s.page_size, window=s.window)
    h2 = oracle.add_ref(h, oracle.gemm_ref(o.reshape(1, -1), W["w_o"]))
    gu = oracle.gemm_ref(oracle.rmsnorm_ref(h2, W["g_mlp"], s.eps), W["w_gu"])
    oracle.add_ref(h2, oracle.gemm_ref(oracle.gated_gelu_ref(gu), W["w_down"]))
    dt = time.perf_counter() - t0
    per_layer = sum(int(np.prod(v.shape)) for v in W.values()) * 2 + 2 * min(L, s.window) * Hk * D * 2
    return {"value": round(per_layer / dt / 1e9, 3), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"float64 numpy per-op chain of one local layer at batch 1, context {L}: {dt:.3f} s "
                      f"(bf16-equivalent bytes of that layer / time)"}


def bench_agentic(args):
    """Agentic sessions on the 34-layer Gemma-3-4B-shaped decoder through the
    engine (prefix cache, chunked prefill, decode steps replayed as HIP graphs):
    a shared reference prefix is cached first; S sessions then each run T
    turns: the first prefills a prompt that starts with the shared prefix, each
    later turn appends new user tokens to the retained conversation (its pages
    are found in the prefix cache), and every turn generates a fixed number of
    tokens greedily.  A session waits a fixed user delay between turns; the
    clock is simulated (engine time is measured, the delay is added, nothing
    sleeps).  Reports session time and the share of engine time spent in
    decode-only steps."""
    torch, bi, synth = _torch_env()
    from deterministic_paged_attention_amd.decoder import Decoder, DecoderShape
    from deterministic_paged_attention_amd.engine import Engine
    from synth.workloads import decoder_weights
    s = DecoderShape(split_size=args.global_split, split_size_local=args.local_split)
    S, T = args.sessions, args.turns
    shared_len, prompt_len, turn_in, turn_out = args.shared_tokens, args.prompt_tokens, args.turn_input, args.turn_output
    delay = args.user_delay
    w = decoder_weights(s.layers, s.hidden, s.q_heads, s.kv_heads, s.head_dim, s.ffn, s.vocab, seed=args.seed + 90)
    dec = Decoder(s, w)
    ctx_max = prompt_len + T * (turn_in + turn_out) + 64
    num_pages = (shared_len + S * ctx_max) // s.page_size + 256
    eng = Engine(dec, num_pages=num_pages, budget=args.prefill_budget, check_writes=False, graphs=True,
                 record_logits=False)
    V = s.vocab
    shared = synth.uniform_ints(shared_len, 0, V - 1, args.seed + 91)
    # cache the shared prefix: one request over it (its pages are registered as they fill)
    eng.add(-1, shared + [0], 1)
    while eng.step():
        pass
    torch.cuda.synchronize()
    conv = {k: shared + synth.uniform_ints(prompt_len - shared_len, 0, V - 1, args.seed + 100 + k) for k in range(S)}
    ready = {k: 0.0 for k in range(S)}       # simulated time the session's next turn arrives
    turn = {k: 0 for k in range(S)}
    active = {}                              # request id -> session
    clock = 0.0
    t_decode = t_mixed = 0.0
    n_decode_steps = n_mixed_steps = 0
    generated = 0
    done_at = {}
    rid = 0
    while len(done_at) < S:
        for k in range(S):
            if k not in done_at and k not in active.values() and ready[k] <= clock:
                eng.add(rid, conv[k], turn_out)
                active[rid] = k
                rid += 1
        if not active:
            clock = min(ready[k] for k in range(S) if k not in done_at)
            continue
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        eng.step()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        clock += dt
        if eng.last_step_decode_only:
            t_decode += dt
            n_decode_steps += 1
        else:
            t_mixed += dt
            n_mixed_steps += 1
        for r_id in [r for r in active if r in eng.finished]:
            k = active.pop(r_id)
            req = eng.finished[r_id]
            generated += len(req.tokens)
            turn[k] += 1
            conv[k] = conv[k] + req.tokens
            print(json.dumps({"progress": {"session": k, "turn": turn[k], "clock_s": round(clock, 3)}}),
                  file=sys.stderr, flush=True)
            if turn[k] == T:
                done_at[k] = clock
            else:
                conv[k] = conv[k] + synth.uniform_ints(turn_in, 0, V - 1, args.seed + 1000 * k + turn[k])
                ready[k] = clock + delay
    engine_time = t_decode + t_mixed
    reused = sum(r.reused_pages for r in eng.finished.values() if r.rid >= 0)
    print(json.dumps({
        "metric": "agentic sessions: decode share of engine time and output tokens/s", "value": round(generated / engine_time, 1),
        "unit": "output tokens/s (engine time)", "n_gpus": 1, "steps": eng.steps, "warmup": 0,
        "ms_per_step": round(engine_time / max(eng.steps, 1) * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "agentic sessions on a gemma-3-4b-shaped decoder (random init) through the engine",
                   "sessions": S, "turns": T, "shared_prefix_tokens": shared_len, "first_prompt_tokens": prompt_len,
                   "turn_input_tokens": turn_in, "turn_output_tokens": turn_out, "user_delay_s": delay,
                   "prefill_budget": args.prefill_budget, "split_size": s.split_size,
                   "split_size_local": s.split_size_local},
        "session_time_s": round(max(done_at.values()), 3), "engine_time_s": round(engine_time, 3),
        "decode_share_of_engine_time": round(t_decode / engine_time, 4),
        "decode_steps": n_decode_steps, "steps_with_prefill": n_mixed_steps,
        "decode_ms_per_step": round(t_decode / max(n_decode_steps, 1) * 1e3, 3),
        "generated_tokens": generated, "prefix_pages_reused": reused, "graph_replays": eng.graph_replays,
        "graphs_captured": len(eng._graphs), "cache_stats": list(eng.cache.stats())}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "decode-sweep", "gemm", "prefill", "gemma", "agentic"])
    ap.add_argument("--sessions", type=int, default=4)
    ap.add_argument("--turns", type=int, default=6)
    ap.add_argument("--shared-tokens", type=int, default=8192)
    ap.add_argument("--prompt-tokens", type=int, default=16384)
    ap.add_argument("--turn-input", type=int, default=256)
    ap.add_argument("--turn-output", type=int, default=768)
    ap.add_argument("--user-delay", type=float, default=0.5)
    ap.add_argument("--prefill-budget", type=int, default=2048)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--local-split", type=int, default=DEFAULT_LOCAL_SPLIT,
                    help="gemma and agentic workloads: fixed KV split size of the windowed layers")
    ap.add_argument("--global-split", type=int, default=DEFAULT_GLOBAL_SPLIT,
                    help="gemma and agentic workloads: fixed KV split size of the global layers")
    ap.add_argument("--batches", default="1,8,64,256", help="decode-sweep workload: batch sizes to run")
    ap.add_argument("--ms", default="1,7,64,256,1024", help="gemm workload: token counts M to run")
    ap.add_argument("--budgets", default="16,128,512,0",
                    help="prefill workload: chunk budgets to run (0 = token by token)")
    ap.add_argument("--seed", type=int, default=2000)
    ap.add_argument("--cpu-sample", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-splitk", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the method is single-GPU and this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    {"decode": bench_decode, "decode-sweep": bench_decode_sweep, "gemm": bench_gemm, "prefill": bench_prefill,
     "gemma": bench_gemma, "agentic": bench_agentic}[args.workload](args)


if __name__ == "__main__":
    main()
