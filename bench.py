#!/usr/bin/env python3
"""Benchmark: one batch-invariant decode step of a Llama-3.1-8B-shaped attention layer.

Step (every row of the hot path, on one batch of synthetic input resident in HBM):
  RMSNorm(x) -> QKV GEMM [B,4096]x[6144,4096]^T -> slot mapping -> KV write of the
  new token -> paged attention split phase -> merge phase -> O GEMM [B,4096]x[4096,4096]^T
Geometry: 32 query / 8 KV heads, head_dim 128, pages of 16 tokens, fixed key split
256, context lengths ~ U{512..8192}, K/V/x ~ N(0,1) bf16, weights ~ N(0, 0.02),
gamma ~ N(1, 0.1).  Random-init, synthetic data.

Prints ONE JSON line.  `value` = algorithmic HBM bytes of the whole step / step
time (GB/s).  `roofline` is for the dominant kernel (attention split phase),
timed with HIP events recorded on the stream it is launched on.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
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
PEAK_HBM_GBPS = 8000.0
HQ, HKV, D, P, S = 32, 8, 128, 16, 256
HIDDEN = 4096
QKV_N = (HQ + 2 * HKV) * D
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_split_traffic.json")
KERNEL_SOURCES = ["deterministic_paged_attention_amd/csrc/attention.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(batch: int):
    """HBM bytes per split launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_source_hash() or t.get("batch") != batch:
        return None
    return t.get("hbm_bytes_per_launch")


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
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 numpy attention oracle over {sample_seqs} of the {wl.batch} decode sequences of the "
                      f"same workload (same bytes-per-sequence accounting as the GPU), {dt:.1f} s of oracle time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=256)
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

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, min(args.cpu_sample, B))

    xn = torch.empty((B, HIDDEN), dtype=torch.bfloat16, device=dev)
    qkv = torch.empty((B, QKV_N), dtype=torch.bfloat16, device=dev)
    q = qkv[:, : HQ * D].view(B, HQ, D)
    k_new = qkv[:, HQ * D: (HQ + HKV) * D].view(B, HKV, D)
    v_new = qkv[:, (HQ + HKV) * D:].view(B, HKV, D)
    slots = torch.empty(B, dtype=torch.int32, device=dev)
    attn = torch.empty((B, HQ, D), dtype=torch.bfloat16, device=dev)
    y = torch.empty((B, HIDDEN), dtype=torch.bfloat16, device=dev)
    ws = bi.alloc_workspace(bi.bi_paged_attention_workspace_size(cfg, B, B, wl.max_seq_len))
    stream = torch.cuda.current_stream()

    names = ["rmsnorm", "gemm_qkv", "slot_mapping", "kv_write", "attn_split", "attn_merge", "gemm_o"]
    launches = [
        lambda: bi.bi_rmsnorm(x, gamma, 1e-5, out=xn),
        lambda: bi.bi_gemm(xn, w_qkv, out=qkv),
        lambda: bi.bi_slot_mapping(wl.page_table, wl.seq_lens, wl.qsl, B, P, wl.num_pages, out=slots),
        lambda: bi.bi_kv_write(cfg, k_new, v_new, slots, wl.k_cache, wl.v_cache),
        lambda: bi.bi_paged_attention_split(cfg, q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.qsl,
                                            wl.max_seq_len, ws),
        lambda: bi.bi_paged_attention_merge(cfg, wl.seq_lens, wl.qsl, B, wl.max_seq_len, ws, out=attn),
        lambda: bi.bi_gemm(attn.view(B, HQ * D), w_o, out=y),
    ]

    def step(events=None):
        for i, f in enumerate(launches):
            if events is not None:
                events[i].record(stream)
            f()
        if events is not None:
            events[-1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)] for _ in range(args.steps)]
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
    per_kernel = {n: statistics.mean(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)) * 1e3
                  for i, n in enumerate(names)}

    sb = split_bytes(lengths)
    split_us = per_kernel["attn_split"]
    achieved = sb / (split_us * 1e-6) / 1e9
    value = step_bytes(lengths) / (ms_per_step * 1e-3) / 1e9
    attn_us = per_kernel["attn_split"] + per_kernel["attn_merge"]
    attn_gbps = (sb + B * HQ * D * 2) / (attn_us * 1e-6) / 1e9

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
            launches[4]()
            launches[5]()

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
                     "kernel": "attn_split_kernel<128>", "algorithmic_bytes_per_launch": sb,
                     "avg_launch_us": round(split_us, 2)},
        "cpu_baseline": cpu,
        "attention_gbps": round(attn_gbps, 2),
        "attention_frac_of_peak": round(attn_gbps / PEAK_HBM_GBPS, 4),
        "splitk": splitk,
        "kernels_us": {k: round(v, 2) for k, v in per_kernel.items()},
        "kernel_sha": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
