"""Benchmark of batched paged attention on one MI355X.

Default line: the batched decode workload (64 sequences, lengths uniform in
[512, 4096], 32 q heads / 8 kv heads, head dim 128, block size 16, f16 K/V, 8 forks
sharing a 256-token prefix).  One step = pa_write_kv of the 64 new tokens + pa_decode
(split-KV, partitions of 512 positions, then the log-sum-exp reduce).  The value is
decode KV bytes per second: sum over sequences and kv heads of the visible positions
times (head_dim_k + head_dim_v) * 2 bytes, divided by the step time.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|long|varlen|mla]

Prints one JSON line.  The roofline object times the decode call alone with HIP
events on its stream, with a 512 MiB buffer rewritten between launches so that the
pool is read from HBM; the cpu_baseline object times the CPU oracle on the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged-decode KV GB/s (% HBM peak); varlen prefill TFLOP/s (% MFMA peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode", "long", "varlen", "mla"])
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    return ap.parse_args()


def dev(a, dtype=None):
    import torch

    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda")


def decode_bytes(w):
    """Algorithmic KV bytes of one decode call: every visible position of every
    (sequence, kv head) read once, K and V."""
    eb = 4 if w.dtype == "f32" else 2
    n = w.seq_lens.astype(np.int64)
    if w.sliding_window > 0:
        n = np.minimum(n, w.sliding_window)
    return int(n.sum()) * w.num_kv_heads * (w.dk + w.dv) * eb


def time_calls(fn, reps, flush=None):
    """Average duration of fn() in ms from HIP events on the current stream; the
    optional flush runs between calls, outside the events."""
    import torch

    durs = []
    for _ in range(reps):
        if flush is not None:
            flush()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        durs.append(s.elapsed_time(e))
    return float(np.mean(durs)), float(np.median(durs))


def cpu_baseline_decode(w, budget_s):
    """The oracle (as it stands) on a bounded prefix of the sequences, all host cores."""
    from oracle import oracle as orc_mod

    orc = orc_mod.get()
    threads = os.cpu_count() or 1
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    orc.write_kv(kp, vp, w.dtype, w.k_new, w.v_new, w.slot_mapping)
    S = w.num_seqs
    take = S
    # calibrate on 4 sequences, then size the sample to the budget
    t0 = time.perf_counter()
    orc.decode(kp, vp, w.dtype, w.q[:4], w.dtype, w.block_tables[:4], w.seq_lens[:4], w.scale, threads=threads)
    per_seq = (time.perf_counter() - t0) / 4
    take = int(max(4, min(S, budget_s / max(per_seq, 1e-9))))
    t0 = time.perf_counter()
    orc.decode(kp, vp, w.dtype, w.q[:take], w.dtype, w.block_tables[:take], w.seq_lens[:take], w.scale,
               threads=threads)
    dt = time.perf_counter() - t0
    eb = 4 if w.dtype == "f32" else 2
    nbytes = int(w.seq_lens[:take].astype(np.int64).sum()) * w.num_kv_heads * (w.dk + w.dv) * eb
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {take} of {S} sequences, whole decode call (gather + two-pass fp64), {dt:.2f} s"}


def varlen_flops(w):
    """Algorithmic flops of one varlen call: visible (query, key) pairs times
    2 * (head_dim_k + head_dim_v), summed over q heads."""
    total = 0
    for s in range(w.num_seqs):
        t0, t1 = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
        pos = w.positions[t0:t1].astype(np.int64)
        end = pos + 1 if w.causal else np.full(t1 - t0, int(w.seq_lens[s]))
        start = np.maximum(0, end - w.sliding_window) if w.sliding_window > 0 else np.zeros_like(end)
        total += int((end - start).sum())
    return total * w.num_heads * 2 * (w.dk + w.dv)


def chunked_flops(cp):
    total = 0
    for ctx, n in zip(cp.ctx_lens.astype(np.int64), cp.new_lens.astype(np.int64)):
        total += n * ctx + n * (n + 1) // 2
    return int(total) * cp.num_heads * 2 * (cp.dk + cp.dv)


def run_prefill(args):
    """Secondary workloads: mixed varlen (config of 4 prefill chunks + 12 decode
    tokens) or the MLA-style chunked prefill.  Prints one JSON line in TFLOP/s."""
    import torch

    from paged_kv_attention_table_amd import pa_varlen, pa_write_kv
    from paged_kv_attention_table_amd import workloads as W
    from paged_kv_attention_table_amd.chunked import ChunkedPrefillPlan

    if args.workload == "varlen":
        w = W.config4()
        kp, vp = dev(w.k_pool, w.dtype), dev(w.v_pool, w.dtype)
        q = dev(w.q, w.dtype)
        qsl, lens, pos, tables = dev(w.query_start_loc), dev(w.seq_lens), dev(w.positions), dev(w.block_tables)
        k_new, v_new, slots = dev(w.k_new, w.dtype), dev(w.v_new, w.dtype), dev(w.slot_mapping)
        out = torch.empty((w.num_tokens, w.num_heads, w.dv), device="cuda")
        lse = torch.empty((w.num_heads, w.num_tokens), device="cuda")
        max_q = int(np.diff(w.query_start_loc).max())
        flops = varlen_flops(w)

        def attn():
            pa_varlen(kp, vp, q, out, qsl, lens, pos, tables, max_q, w.scale, causal=True,
                      sliding_window=w.sliding_window, lse=lse)

        def step():
            pa_write_kv(kp, vp, k_new, v_new, slots)
            attn()
        name, dtype = w.name, w.dtype
        cfg = {"workload": name, "prefill_seqs": 4, "decode_seqs": 12, "num_tokens": w.num_tokens,
               "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.dk,
               "sliding_window": w.sliding_window, "step": "pa_write_kv + pa_varlen"}
    else:
        cp = W.config5()
        kp, vp = dev(cp.k_pool, cp.dtype), dev(cp.v_pool, cp.dtype)
        q = dev(cp.q, cp.dtype)
        k_new, v_new, slots = dev(cp.k_new, cp.dtype), dev(cp.v_new, cp.dtype), dev(cp.slot_mapping)
        plan = ChunkedPrefillPlan(ctx_lens=cp.ctx_lens, new_lens=cp.new_lens, ctx_tables=cp.ctx_tables,
                                  new_tables=cp.new_tables, chunk=cp.chunk, block_size=cp.block_size,
                                  num_heads=cp.num_heads, head_dim_v=cp.dv, scale=cp.scale)
        out = torch.empty((cp.num_tokens, cp.num_heads, cp.dv), device="cuda")
        lse = torch.empty((cp.num_heads, cp.num_tokens), device="cuda")
        flops = chunked_flops(cp)

        def attn():
            plan.run(kp, vp, q, out, lse)

        def step():
            pa_write_kv(kp, vp, k_new, v_new, slots)
            attn()
        name, dtype = cp.name, cp.dtype
        cfg = {"workload": name, "requests": int(cp.ctx_lens.size), "num_tokens": cp.num_tokens,
               "num_heads": cp.num_heads, "head_dim_k": cp.dk, "head_dim_v": cp.dv, "chunk": cp.chunk,
               "step": "pa_write_kv + chunked pa_varlen + pa_merge_states"}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    avg_ms, med_ms = time_calls(attn, max(10, args.steps // 2))
    value = flops / (ms * 1e-3) / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    line = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": dict(cfg, flops_per_step=flops),
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "avg_ms": round(avg_ms, 5), "median_ms": round(med_ms, 5)}}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch

    from paged_kv_attention_table_amd import pa_decode, pa_write_kv
    from paged_kv_attention_table_amd import workloads as W

    if args.workload in ("varlen", "mla"):
        return run_prefill(args)
    w = W.config2() if args.workload == "decode" else W.config3()
    P = args.partition_size if args.partition_size is not None else 512
    kp, vp = dev(w.k_pool, w.dtype), dev(w.v_pool, w.dtype)
    q = dev(w.q, w.dtype)
    tables, lens = dev(w.block_tables), dev(w.seq_lens)
    k_new, v_new, slots = dev(w.k_new, w.dtype), dev(w.v_new, w.dtype), dev(w.slot_mapping)
    S, H = w.num_seqs, w.num_heads
    out = torch.empty((S, H, w.dv), device="cuda")
    pmax = max(1, -(-int(w.seq_lens.max()) // P)) if P else 0
    ws = (torch.empty((S, H, pmax), device="cuda"), torch.empty((S, H, pmax), device="cuda"),
          torch.empty((S, H, pmax, w.dv), device="cuda")) if P else (None, None, None)

    def decode():
        pa_decode(kp, vp, q, out, tables, lens, w.scale, sliding_window=w.sliding_window, partition_size=P,
                  max_logits=ws[0], exp_sums=ws[1], tmp_out=ws[2])

    def step():
        pa_write_kv(kp, vp, k_new, v_new, slots)
        decode()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    nbytes = decode_bytes(w)
    value = nbytes / (ms * 1e-3) / 1e9

    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    flush = lambda: scratch.fill_(1)
    avg_ms, med_ms = time_calls(decode, max(10, args.steps // 2), flush=flush)
    achieved = nbytes / (avg_ms * 1e-3) / 1e9

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": S, "seq_lens": [int(w.seq_lens.min()), int(w.seq_lens.max())],
                   "num_heads": H, "num_kv_heads": w.num_kv_heads, "head_dim": w.dk, "block_size": w.block_size,
                   "partition_size": P, "kv_bytes_per_step": nbytes, "step": "pa_write_kv + pa_decode"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pa_decode (per-partition kernel + reduce)", "avg_ms": round(avg_ms, 5),
                     "median_ms": round(med_ms, 5)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(w, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
