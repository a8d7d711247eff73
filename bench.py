"""Benchmark of batched paged attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload all|decode|long|decode-fp8|long-fp8|varlen|mla|varlen-fp8|mla-fp8|
                                gather|tiles]
                    [--partition-size P] [--no-cpu-baseline] [--copy-calibration] [--sweep]
                    [--ceilings]

Prints one JSON line.  With the default --workload all it covers the whole metric,
"paged-decode KV GB/s; varlen prefill TFLOP/s":

* the headline (value, ms_per_step, roofline, cpu_baseline) is the batched decode
  workload: 64 sequences, lengths uniform in [512, 4096], 32 q heads / 8 kv heads,
  head dim 128, block size 16, f16 K/V, 8 forks sharing a 256-token prefix.  One
  step = pa_write_kv of the 64 new tokens + pa_decode (unsplit: one kernel launch).
  The value is decode KV bytes per second: over sequences and kv heads, the visible
  positions times (head_dim_k + head_dim_v) * 2 bytes, divided by the wall time of a
  step;
* `secondary` holds the same fields for the mixed varlen call (4 prefill chunks of
  512 tokens + 12 decode tokens, bf16, window 1024; TFLOP/s of visible pairs), the
  MLA-style chunked prefill (8 requests, 128 heads, QK 192 / V 128, bf16; TFLOP/s)
  and the long-context split decode (8 sequences up to 131072 positions, 64 q / 8 kv
  heads, bf16, partitions of 512; GB/s), each timed over its own K steps.

Every entry's roofline divides the algorithmic bytes (or flops) by the attention
call's average duration from HIP events recorded on its stream around every call
of the timed region (`achieved`, `frac`); beside it, `achieved_flushed` /
`frac_flushed` take the median of 20 calls with a 512 MiB write between calls
(outside the events), so that every K/V byte comes from HBM.  `traffic` is the HBM
bytes per call that rocprofv3's FETCH_SIZE and WRITE_SIZE counters gave, scaled by
what the counters read for a copy of known size; it is read from profiles/ and
reported only while the kernels' source hash still matches the one recorded there.
`graph` gives the same step captured once in a HIP graph and replayed K times back
to back (host wall clock per step): the step's rate without the Python binding's
launch path between the calls, as a caller that captures its steps would see it.
`cpu_baseline` times the CPU oracle, unchanged, on a bounded sample of the same
workload on the host cores (thread count and CPU model given).

--workload X prints X's line alone (decode-fp8 / long-fp8 / varlen-fp8 / mla-fp8
are those workloads over an fp8 (E4M3) cache with per-tensor k_scale / v_scale, one
byte per K / V element, the queries in the workload's 16-bit type; gather is the MLA latent-cache gather; tiles is a diagnostic line, the prefill
tile kernel on whole tiles).  --copy-calibration appends, after
the timed region, three launches of a 1 GiB elementwise copy (torch.neg) that the
counter runs use as the known-size reference.  --sweep adds, after the timed region,
for the decode workloads each partition size in {0, 512, 1024}, the cost of device
validation, that of per-head attention sinks and that of ALiBi slopes, and for the
prefill workloads the cost of device validation, each as the median of 20 calls
with the caches flushed between calls.  --ceilings adds what plain library work
reaches on the same GPU as context for the roofline fractions: a 1 GiB device copy
(GB/s read + written) and an 8192^3 bf16 matrix product (TFLOP/s), each the median
of 10 event-timed runs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import hashlib
import re
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
VARLEN_PARTITION = 0  # split-KV partition size for the varlen workload's single-token rows
METRIC = "paged-decode KV GB/s (% HBM peak); varlen prefill TFLOP/s (% MFMA peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "decode", "long", "decode-fp8", "long-fp8", "varlen", "mla", "varlen-fp8",
                             "mla-fp8", "gather", "tiles"])
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--secondary-cpu-budget-s", type=float, default=6.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--ceilings", action="store_true")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "paged_kv_attention_table_amd", "csrc")
KERNEL_SOURCES = {"decode_mfma_kernel": ("pa_decode.h", "pa_prefill.h", "pa_common.h", "pa_misc.hip"),
                  "prefill_kernel": ("pa_prefill.h", "pa_common.h"),
                  "pa_varlen_call": ("pa_prefill.h", "pa_decode.h", "pa_varlen_fused.h", "pa_rows.h", "pa_common.h",
                                     "pa_misc.hip", "pa_api.hip"),
                  "gather_rows16_kernel": ("pa_gather.hip", "pa_common.h")}
TRAFFIC_TABLES = ("traffic.md", "traffic_prefill.md")


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_lookup(kernel, workload, partition_size):
    """HBM bytes per launch (read, write) recorded in the traffic tables under
    profiles/ for this kernel (or call), workload and partition size, or None when
    absent or when the sources changed since the counters were taken."""
    want = kernel_source_hash(kernel)
    for table in TRAFFIC_TABLES:
        path = os.path.join(ROOT, "profiles", table)
        if not os.path.exists(path):
            continue
        for line in open(path):
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) < 6 or cells[0] != kernel:
                continue
            if cells[1] == workload and cells[2] == str(partition_size) and cells[3] == want:
                try:
                    return int(cells[4]), int(cells[5])
                except ValueError:
                    return None
    return None


def copy_calibration():
    """A 1 GiB elementwise copy (read 1 GiB, write 1 GiB), three launches: the
    known-size reference for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch

    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def ceilings():
    """Measured context for the peaks: a 1 GiB copy and an 8192^3 bf16 matrix
    product (contiguous operands), median of 10 runs each."""
    import torch

    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    nb = src.numel() * 4
    for _ in range(2):
        torch.neg(src, out=dst)
    _, copy_ms = time_calls(lambda: torch.neg(src, out=dst), 10)
    del src, dst
    n = 8192
    a = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        torch.matmul(a, b, out=c)
    _, mm_ms = time_calls(lambda: torch.matmul(a, b, out=c), 10)
    torch.cuda.synchronize()
    del a, b, c
    return {"copy_gbs": round(2 * nb / (copy_ms * 1e-3) / 1e9, 1),
            "gemm_bf16_tflops": round(2 * n ** 3 / (mm_ms * 1e-3) / 1e12, 1),
            "what": "torch.neg 1 GiB copy (read + written), torch.matmul 8192^3 bf16; median of 10"}


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def flushed_median_ms(call, reps=20):
    """Median duration of call() in ms over reps calls, each preceded (outside the
    events) by a 512 MiB device write that evicts the L2 caches and the MALL."""
    import torch

    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    _, med = time_calls(call, reps, flush=lambda: scratch.fill_(1))
    del scratch
    return med


def timed_loop(steps, pre, call, lead=False):
    """Runs pre(); call() per step.  Returns (ms per step, average and median event
    duration of call() in ms), with events recorded on the current stream.

    By default ms per step is the host's wall clock and each call sits between its
    own pair of events.  lead=True is for calls shorter than the host's launch path
    (pre must do nothing): the calls are queued behind eight 512 MiB device fills
    (4 GiB of writes, about 0.7 ms) so that the host's launch overhead overlaps
    them, and one pair of events spans all of them back to back; every figure is
    then that span divided by the number of calls, the rate of back-to-back calls
    whose launches are not host-bound."""
    import torch

    torch.cuda.synchronize()
    if lead:
        filler = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        for _ in range(8):
            filler.fill_(1)
        s.record()
        for _ in range(steps):
            call()
        e.record()
        torch.cuda.synchronize()
        per = s.elapsed_time(e) / steps
        return per, per, per
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in evs:
        pre()
        s.record()
        call()
        e.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    durs = [s.elapsed_time(e) for s, e in evs]
    return wall, float(np.mean(durs)), float(np.median(durs))


def graph_step_ms(steps, step):
    """ms per step when step() (its library calls only) is captured once in a HIP graph
    and the graph is replayed `steps` times back to back: host wall clock from the
    first replay to the end of the last, and one pair of events around them, as
    (wall, events)."""
    import torch

    side = torch.cuda.Stream()  # warm-up off the capturing stream, as torch asks
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s.record()
    for _ in range(steps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = s.elapsed_time(e) / steps
    del g
    return wall, ev


def graph_entry(steps, step, work, unit_scale, unit):
    """The `graph` field of an entry: the step replayed from a captured HIP graph."""
    wall, ev = graph_step_ms(steps, step)
    return {"ms_per_step": round(wall, 5), "value": round(work / (wall * 1e-3) / unit_scale, 2), "unit": unit,
            "ms_per_step_events": round(ev, 5),
            "what": "the step captured once in a HIP graph, replayed K times; wall clock per step"}


def dev(a, dtype=None):
    import torch

    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    if dtype == "fp8_e4m3":
        return torch.from_numpy(a.view(np.uint8)).to("cuda").view(torch.float8_e4m3fn)
    return torch.from_numpy(a).to("cuda")


ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}


def decode_bytes(w):
    """Algorithmic KV bytes of one decode call: every visible position of every
    (sequence, kv head) read once, K and V."""
    eb = ELEM_BYTES[w.dtype]
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
    """The oracle (as it stands) on a bounded sample of the workload, all host cores:
    the first sequences (as many as fit the budget in one call), the call repeated
    until about budget_s seconds of host time have passed."""
    from oracle import oracle as orc_mod

    orc = orc_mod.get()
    threads = host_cores()
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    orc.write_kv(kp, vp, w.dtype, w.k_new, w.v_new, w.slot_mapping)
    S = w.num_seqs

    def call(n):
        orc.decode(kp, vp, w.dtype, w.q[:n], w.query_dtype, w.block_tables[:n], w.seq_lens[:n], w.scale,
                   threads=threads, k_scale=w.k_scale, v_scale=w.v_scale)

    t0 = time.perf_counter()
    call(min(S, 4))
    per_seq = (time.perf_counter() - t0) / min(S, 4)
    take = int(max(1, min(S, budget_s / max(per_seq, 1e-9))))
    reps = 0
    t0 = time.perf_counter()
    while True:
        call(take)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or dt + dt / reps > 1.5 * budget_s:
            break
    eb = ELEM_BYTES[w.dtype]
    nbytes = int(w.seq_lens[:take].astype(np.int64).sum()) * w.num_kv_heads * (w.dk + w.dv) * eb * reps
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "cpu": host_cpu_model(),
            "kind": "oracle",
            "sample": f"first {take} of {S} sequences, whole oracle decode call (gather + two-pass fp64) "
                      f"repeated {reps} times, {dt:.1f} s"}


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


def _timed_rows(run, per_row_flops, total_rows, budget_s, what):
    """Times run(m) (the oracle on the first m rows) on a bounded sample: a short
    calibration call, then m sized to the budget and the call repeated until about
    budget_s seconds of host time have passed.  Reports GFLOP/s of visible pairs."""
    m0 = min(total_rows, 16)
    t0 = time.perf_counter()
    run(m0)
    per = (time.perf_counter() - t0) / max(float(per_row_flops[:m0].sum()), 1.0)
    cum = np.cumsum(per_row_flops)
    m = int(np.searchsorted(cum, budget_s / max(per, 1e-18))) + 1
    m = max(m0, min(total_rows, m))
    reps, t0 = 0, time.perf_counter()
    while True:
        run(m)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or dt + dt / reps > 1.5 * budget_s:
            break
    fl = float(cum[m - 1]) * reps
    return {"value": round(fl / dt / 1e9, 4), "unit": "GFLOP/s", "cores": host_cores(), "cpu": host_cpu_model(),
            "kind": "oracle",
            "sample": f"{what}: first {m} of {total_rows} query tokens (all heads), repeated {reps} times, {dt:.1f} s"}


def cpu_baseline_varlen(w, budget_s):
    """The oracle's varlen (fp64) on the first rows of the packed mixed call."""
    from oracle import oracle as orc_mod

    orc = orc_mod.get()
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    orc.write_kv(kp, vp, w.dtype, w.k_new, w.v_new, w.slot_mapping)
    T, H = w.num_tokens, w.num_heads
    per_row = np.zeros(T, dtype=np.float64)
    for s in range(w.num_seqs):
        t0, t1 = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
        end = w.positions[t0:t1].astype(np.int64) + 1
        start = np.maximum(0, end - w.sliding_window) if w.sliding_window > 0 else np.zeros_like(end)
        per_row[t0:t1] = (end - start) * H * 2 * (w.dk + w.dv)

    def run(m):
        mask = np.zeros((T, H), dtype=np.uint8)
        mask[:m] = 1
        st, _, _ = orc.varlen(kp, vp, w.dtype, w.q, w.query_dtype, w.query_start_loc, w.seq_lens, w.positions,
                              w.block_tables, w.scale, True, w.sliding_window, row_mask=mask, threads=host_cores(),
                              k_scale=w.k_scale, v_scale=w.v_scale)
        assert st == 0

    return _timed_rows(run, per_row, T, budget_s, "oracle varlen call, causal, window")


def cpu_baseline_chunked(cp, budget_s):
    """The oracle on the chunked composition for the first request's first rows: its
    varlen (fp64) per context chunk and for the causal new tokens, the states folded
    with its merge_states in the driver's order."""
    from oracle import oracle as orc_mod

    orc = orc_mod.get()
    kp, vp = cp.k_pool.copy(), cp.v_pool.copy()
    orc.write_kv(kp, vp, cp.dtype, cp.k_new, cp.v_new, cp.slot_mapping)
    T, H = cp.num_tokens, cp.num_heads
    ctx0, n0 = int(cp.ctx_lens[0]), int(cp.new_lens[0])
    per_row = (ctx0 + np.arange(1, n0 + 1, dtype=np.float64)) * H * 2 * (cp.dk + cp.dv)
    per = cp.chunk // cp.block_size
    qsl = np.zeros(cp.ctx_lens.size + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(cp.new_lens)
    positions = np.concatenate([np.arange(n, dtype=np.int32) for n in cp.new_lens])
    nchunks = -(-int(cp.ctx_lens.max()) // cp.chunk)

    def run(m):
        mask = np.zeros((T, H), dtype=np.uint8)
        mask[:m] = 1
        state = None
        for c in range(nchunks + 1):
            if c < nchunks:
                lens = np.clip(cp.ctx_lens - c * cp.chunk, 0, cp.chunk).astype(np.int32)
                tab = np.ascontiguousarray(cp.ctx_tables[:, c * per:(c + 1) * per])
                if tab.shape[1] == 0:
                    continue
                st, o, l = orc.varlen(kp, vp, cp.dtype, cp.q, cp.query_dtype, qsl, lens, None, tab, cp.scale, False,
                                      0, row_mask=mask, threads=host_cores(), k_scale=cp.k_scale, v_scale=cp.v_scale)
            else:
                st, o, l = orc.varlen(kp, vp, cp.dtype, cp.q, cp.query_dtype, qsl, cp.new_lens.astype(np.int32),
                                      positions, cp.new_tables, cp.scale, True, 0, row_mask=mask,
                                      threads=host_cores(), k_scale=cp.k_scale, v_scale=cp.v_scale)
            assert st == 0
            o, l = o[:m].astype(np.float32), np.ascontiguousarray(l[:, :m]).astype(np.float32)
            state = (o, l) if state is None else orc.merge_states(state[0], state[1], o, l, "f32")[:2]
            state = (np.asarray(state[0], dtype=np.float32), np.asarray(state[1], dtype=np.float32))

    return _timed_rows(run, per_row, n0, budget_s, "oracle chunked composition of request 0 (context chunks "
                       "+ causal new tokens, merged)")


def cpu_baseline_gather(g, budget_s):
    """The oracle's latent-cache gather on the whole workload, repeated to the budget."""
    from oracle import oracle as orc_mod

    orc = orc_mod.get()
    T, D = int(g.cu_seq_lens[-1]), g.cache.shape[2]
    reps, t0 = 0, time.perf_counter()
    while True:
        st, _ = orc.gather_cache(g.cache, g.dtype, g.block_tables, g.cu_seq_lens, g.token_to_seq, None, g.dtype, T)
        assert st == 0
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or dt + dt / reps > 1.5 * budget_s:
            break
    return {"value": round(T * D * 2 * 2 * reps / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "cpu": host_cpu_model(),
            "kind": "oracle",
            "sample": f"the whole gather ({T} rows of {D}), one thread, repeated {reps} times, {dt:.1f} s"}


def prefill_entry(args, kind, cpu_budget_s):
    """The mixed varlen call (4 prefill chunks + 12 decode tokens) or the MLA-style
    chunked prefill, over a 16-bit cache or (kind ending in -fp8) an fp8 one: one entry
    in TFLOP/s of visible (query, key) pairs."""
    import torch

    from paged_kv_attention_table_amd import pa_varlen, pa_write_kv
    from paged_kv_attention_table_amd import workloads as W
    from paged_kv_attention_table_amd.chunked import ChunkedPrefillPlan

    fp8 = kind.endswith("-fp8")
    if kind.removesuffix("-fp8") == "varlen":
        w = W.mixed_varlen()
        if fp8:
            w = W.to_fp8(w)
        kp, vp = dev(w.k_pool, w.dtype), dev(w.v_pool, w.dtype)
        q = dev(w.q, w.query_dtype)
        qsl, lens, pos, tables = dev(w.query_start_loc), dev(w.seq_lens), dev(w.positions), dev(w.block_tables)
        k_new, v_new, slots = dev(w.k_new, w.dtype), dev(w.v_new, w.dtype), dev(w.slot_mapping)
        out = torch.empty((w.num_tokens, w.num_heads, w.dv), device="cuda")
        lse = torch.empty((w.num_heads, w.num_tokens), device="cuda")
        max_q = int(np.diff(w.query_start_loc).max())
        flops = varlen_flops(w)
        # single-token rows split over partitions (a caller workspace) unless
        # --partition-size 0
        P = VARLEN_PARTITION if args.partition_size is None else args.partition_size
        pmax = -(-int(w.seq_lens.max()) // P) if P else 0
        ws = [torch.empty(sh, device="cuda") for sh in ((w.num_seqs, w.num_heads, pmax),
                                                         (w.num_seqs, w.num_heads, pmax),
                                                         (w.num_seqs, w.num_heads, pmax, w.dv))] if P else [None] * 3

        def attn(status=None):
            pa_varlen(kp, vp, q, out, qsl, lens, pos, tables, max_q, w.scale, causal=True,
                      sliding_window=w.sliding_window, lse=lse, partition_size=P, max_logits=ws[0],
                      exp_sums=ws[1], tmp_out=ws[2], status=status, k_scale=w.k_scale, v_scale=w.v_scale)

        def write():
            pa_write_kv(kp, vp, k_new, v_new, slots)

        if P:
            kernel_label = "pa_varlen call (prefill tile kernel + split single-token rows + partition reduce)"
        else:
            kernel_label = "pa_varlen call (fused kernel: prefill tiles and single-token decode rows)"
        name, dtype = w.name, w.query_dtype
        cfg = {"workload": name, "kv_dtype": w.dtype, "prefill_seqs": 4, "decode_seqs": 12, "num_tokens": w.num_tokens,
               "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.dk,
               "sliding_window": w.sliding_window, "single_token_partition_size": P,
               "step": "pa_write_kv + pa_varlen"}
    else:
        cp = W.mla_chunked()
        if fp8:
            cp = W.chunked_to_fp8(cp)
        kp, vp = dev(cp.k_pool, cp.dtype), dev(cp.v_pool, cp.dtype)
        q = dev(cp.q, cp.query_dtype)
        k_new, v_new, slots = dev(cp.k_new, cp.dtype), dev(cp.v_new, cp.dtype), dev(cp.slot_mapping)
        plan = ChunkedPrefillPlan(ctx_lens=cp.ctx_lens, new_lens=cp.new_lens, ctx_tables=cp.ctx_tables,
                                  new_tables=cp.new_tables, chunk=cp.chunk, block_size=cp.block_size,
                                  num_heads=cp.num_heads, head_dim_v=cp.dv, scale=cp.scale)
        out = torch.empty((cp.num_tokens, cp.num_heads, cp.dv), device="cuda")
        lse = torch.empty((cp.num_heads, cp.num_tokens), device="cuda")
        flops = chunked_flops(cp)

        def attn():
            plan.run(kp, vp, q, out, lse, k_scale=cp.k_scale, v_scale=cp.v_scale)

        def write():
            pa_write_kv(kp, vp, k_new, v_new, slots)

        kernel_label = ("chunked prefill (pa_varlen_ctx_new per context chunk, merging into the state after the "
                        "first; each request's causal new tokens in its last chunk's call)")
        name, dtype = cp.name, cp.query_dtype
        cfg = {"workload": name, "kv_dtype": cp.dtype, "requests": int(cp.ctx_lens.size), "num_tokens": cp.num_tokens,
               "num_heads": cp.num_heads, "head_dim_k": cp.dk, "head_dim_v": cp.dv, "chunk": cp.chunk,
               "step": "pa_write_kv + chunked prefill (pa_varlen_ctx_new per context chunk)"}
    def step():
        write()
        attn()

    for _ in range(args.warmup):
        step()
    ms, avg_ms, med_ms = timed_loop(args.steps, write, attn)
    value = flops / (ms * 1e-3) / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    cold_ms = flushed_median_ms(attn)
    cold = flops / (cold_ms * 1e-3) / 1e12
    graph = graph_entry(args.steps, step, flops, 1e12, "TFLOP/s")
    entry = {"value": round(value, 2), "unit": "TFLOP/s", "steps": args.steps, "warmup": args.warmup,
             "ms_per_step": round(ms, 5), "dtype": dtype, "config": dict(cfg, flops_per_step=flops),
             "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                          "kernel": kernel_label, "flops_per_call": flops, "avg_ms": round(avg_ms, 5),
                          "median_ms": round(med_ms, 5), "achieved_flushed": round(cold, 2),
                          "frac_flushed": round(cold / MFMA_BF16_PEAK_TFLOPS, 4),
                          "median_ms_flushed": round(cold_ms, 5)},
             "graph": graph}
    if args.sweep and kind.removesuffix("-fp8") == "varlen":
        # context, after the timed region: the cost of device validation
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        med_status = flushed_median_ms(lambda: attn(status))
        if int(status.item()) != 0:
            raise RuntimeError(f"device validation reported status {int(status.item())}")
        entry["sweep"] = {"validation_ms": round(med_status - cold_ms, 5)}
    t = traffic_lookup("pa_varlen_call", name, P if kind.removesuffix("-fp8") == "varlen" else 0)
    if t is not None:
        entry["roofline"]["traffic"] = t[0] + t[1]
        entry["roofline"]["traffic_read"], entry["roofline"]["traffic_write"] = t
    if args.copy_calibration:
        copy_calibration()
    if cpu_budget_s > 0:
        entry["cpu_baseline"] = (cpu_baseline_varlen(w, cpu_budget_s) if kind.removesuffix("-fp8") == "varlen"
                                 else cpu_baseline_chunked(cp, cpu_budget_s))
    return entry


def run_gather(args):
    """Secondary workload: the latent-cache gather (pa_gather_cache) of every context
    row of the MLA-style requests, 576-wide bf16 rows from a permuted block pool.
    One step = one gather call; GB/s counts the rows read and written once."""
    import torch

    from paged_kv_attention_table_amd import pa_gather_cache
    from paged_kv_attention_table_amd import workloads as W

    g = W.latent_gather()
    cache = dev(g.cache, g.dtype)
    tables, cu, t2s = dev(g.block_tables), dev(g.cu_seq_lens), dev(g.token_to_seq)
    T, D = int(g.cu_seq_lens[-1]), g.cache.shape[2]
    dst = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")

    def call():
        pa_gather_cache(cache, dst, tables, cu, t2s)

    for _ in range(args.warmup):
        call()
    # a gather call is shorter than the host's launch path through Python: queue
    # the calls behind device work so that the events time the device alone
    ms, avg_ms, med_ms = timed_loop(args.steps, lambda: None, call, lead=True)
    nbytes = T * D * 2 * 2
    value = nbytes / (ms * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    line = {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": g.dtype, "data": "synthetic",
            "config": {"workload": g.name, "requests": int(g.ctx_lens.size), "rows": T, "head_dim": D,
                       "block_size": int(g.cache.shape[1]), "step": "pa_gather_cache"},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "gather_rows16_kernel", "avg_ms": round(avg_ms, 5), "median_ms": round(med_ms, 5)}}
    t = traffic_lookup("gather_rows16_kernel", g.name, 0)
    if t is not None:
        line["roofline"]["traffic"] = t[0] + t[1]
        line["roofline"]["traffic_read"], line["roofline"]["traffic_write"] = t
    if args.copy_calibration:
        copy_calibration()
    if args.ceilings:
        line["ceilings"] = ceilings()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_gather(g, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


def decode_entry(args, workload, cpu_budget_s, partition_size=None):
    """A decode workload (batched, long, or their fp8 versions): one entry in GB/s of
    visible K/V bytes.  One step = pa_write_kv of the new tokens + pa_decode."""
    import torch

    from paged_kv_attention_table_amd import pa_decode, pa_write_kv
    from paged_kv_attention_table_amd import workloads as W

    base = workload.removesuffix("-fp8")
    w = W.batched_decode() if base == "decode" else W.long_decode()
    if workload.endswith("-fp8"):
        w = W.to_fp8(w)
    if partition_size is not None:
        P = partition_size
    else:
        P = 0 if base == "decode" else 512
    kp, vp = dev(w.k_pool, w.dtype), dev(w.v_pool, w.dtype)
    q = dev(w.q, w.query_dtype)
    tables, lens = dev(w.block_tables), dev(w.seq_lens)
    k_new, v_new, slots = dev(w.k_new, w.dtype), dev(w.v_new, w.dtype), dev(w.slot_mapping)
    S, H = w.num_seqs, w.num_heads
    out = torch.empty((S, H, w.dv), device="cuda")
    max_len = int(w.seq_lens.max())

    def workspace(p):
        if not p:
            return None, None, None
        pmax = -(-max_len // p)
        return (torch.empty((S, H, pmax), device="cuda"), torch.empty((S, H, pmax), device="cuda"),
                torch.empty((S, H, pmax, w.dv), device="cuda"))

    ws = workspace(P)

    def decode(p=P, buf=ws, status=None, sinks=None, alibi=None):
        pa_decode(kp, vp, q, out, tables, lens, w.scale, sliding_window=w.sliding_window, partition_size=p,
                  max_logits=buf[0], exp_sums=buf[1], tmp_out=buf[2], status=status, sinks=sinks,
                  k_scale=w.k_scale, v_scale=w.v_scale, alibi_slopes=alibi)

    def write():
        pa_write_kv(kp, vp, k_new, v_new, slots)

    for _ in range(args.warmup):
        write()
        decode()
    ms, avg_ms, med_ms = timed_loop(args.steps, write, decode)
    nbytes = decode_bytes(w)
    value = nbytes / (ms * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    cold_ms = flushed_median_ms(decode)
    cold = nbytes / (cold_ms * 1e-3) / 1e9

    def step():
        write()
        decode()

    graph = graph_entry(args.steps, step, nbytes, 1e9, "GB/s")

    kernel = "decode_mfma_kernel"
    roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": kernel + ("" if P == 0 else " + partition reduce_kernel"),
            "bytes_per_launch": nbytes, "avg_ms": round(avg_ms, 5), "median_ms": round(med_ms, 5),
            "achieved_flushed": round(cold, 2), "frac_flushed": round(cold / HBM_PEAK_GBS, 4),
            "median_ms_flushed": round(cold_ms, 5)}
    t = traffic_lookup(kernel, w.name, P)
    if t is not None:
        roof["traffic"] = t[0] + t[1]
        roof["traffic_read"], roof["traffic_write"] = t
    entry = {"value": round(value, 2), "unit": "GB/s", "steps": args.steps, "warmup": args.warmup,
             "ms_per_step": round(ms, 5), "dtype": w.query_dtype,
             "config": {"workload": w.name, "kv_dtype": w.dtype, "num_seqs": S,
                        "seq_lens": [int(w.seq_lens.min()), max_len],
                        "num_heads": H, "num_kv_heads": w.num_kv_heads, "head_dim": w.dk,
                        "block_size": w.block_size, "partition_size": P, "kv_bytes_per_step": nbytes,
                        "step": "pa_write_kv + pa_decode"},
             "roofline": roof, "graph": graph}
    if args.sweep:
        # context, after the timed region: each partition size, and the cost of device
        # validation (status word), sinks and ALiBi; median of 20 flushed calls
        sweep = {}
        for p in (0, 512, 1024):
            buf = ws if p == P else workspace(p)
            sweep[str(p)] = round(nbytes / (flushed_median_ms(lambda: decode(p, buf)) * 1e-3) / 1e9, 1)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        med_plain = flushed_median_ms(decode)
        med_status = flushed_median_ms(lambda: decode(status=status))
        if int(status.item()) != 0:
            raise RuntimeError(f"device validation reported status {int(status.item())}")
        # attention sinks (one logit per q head) on the bench's own partition size
        sinks = torch.linspace(-2.0, 2.0, w.num_heads, device="cuda")
        med_sinks = flushed_median_ms(lambda: decode(sinks=sinks))
        # ALiBi with the geometric slopes 2^(-8 (h + 1) / H)
        slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32, device="cuda")
        med_alibi = flushed_median_ms(lambda: decode(alibi=slopes))
        entry["sweep"] = {"cold_gbs_by_partition_size": sweep, "validation_ms": round(med_status - med_plain, 5),
                          "sinks_ms": round(med_sinks - med_plain, 5), "alibi_ms": round(med_alibi - med_plain, 5)}
    if args.copy_calibration:
        copy_calibration()
    if cpu_budget_s > 0:
        entry["cpu_baseline"] = cpu_baseline_decode(w, cpu_budget_s)
    return entry


def as_line(entry, args, extra=None):
    """The contract's JSON line around one entry."""
    line = {"metric": METRIC, "value": entry["value"], "unit": entry["unit"], "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": entry["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": entry["dtype"], "data": "synthetic",
            "config": entry["config"], "roofline": entry["roofline"]}
    for k in ("graph", "sweep", "cpu_baseline"):
        if k in entry:
            line[k] = entry[k]
    if extra:
        line.update(extra)
    return line


def run_tiles(args):
    """Diagnostic workload: the prefill tile kernel on whole tiles, no masking -- 8
    sequences of 1024 queries over 5120 keys each, non-causal, H 128, Dqk 192 / Dv
    128, bf16 (the MLA workload's head shape at its first chunk's size), through one
    pa_varlen call.  Inputs are drawn on the GPU from a seeded generator; block ids
    are a seeded permutation.  It measures the kernel's own rate, not a workload of
    the metric, so it carries no CPU baseline."""
    import torch

    from paged_kv_attention_table_amd import pa_varlen

    S, qlen, klen, H, dk, dv, b = 8, 1024, 5120, 128, 192, 128, 16
    g = torch.Generator(device="cuda").manual_seed(2026)
    nb = S * klen // b + 1
    kp = torch.randn((nb, b, H, dk), device="cuda", generator=g).to(torch.bfloat16)
    vp = torch.randn((nb, b, H, dv), device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn((S * qlen, H, dk), device="cuda", generator=g).to(torch.bfloat16)
    tables = torch.randperm(nb - 1, device="cuda", generator=g)[: S * klen // b].view(S, klen // b)
    tables = tables.to(torch.int32).contiguous()
    lens = torch.full((S,), klen, dtype=torch.int32, device="cuda")
    qsl = torch.arange(0, S * qlen + 1, qlen, dtype=torch.int32, device="cuda")
    pos = torch.zeros(S * qlen, dtype=torch.int32, device="cuda")
    out = torch.empty((S * qlen, H, dv), device="cuda")
    lse = torch.empty((H, S * qlen), device="cuda")
    flops = S * H * qlen * klen * 2 * (dk + dv)

    def call():
        pa_varlen(kp, vp, q, out, qsl, lens, pos, tables, qlen, dk ** -0.5, causal=False, lse=lse)

    for _ in range(args.warmup):
        call()
    ms, avg_ms, med_ms = timed_loop(args.steps, lambda: None, call)
    achieved = flops / (avg_ms * 1e-3) / 1e12
    line = {"metric": "prefill tile kernel TFLOP/s on whole tiles (diagnostic)", "value": round(flops / (ms * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "prefill-whole-tiles", "num_seqs": S, "queries": qlen, "keys": klen, "num_heads": H,
                       "num_kv_heads": H, "head_dim_k": dk, "head_dim_v": dv, "causal": False,
                       "flops_per_step": flops, "step": "pa_varlen"},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "kernel": "prefill_kernel<BF16, 192, 128, false, false>", "avg_ms": round(avg_ms, 5),
                         "median_ms": round(med_ms, 5)}}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    import torch

    budget = 0.0 if args.no_cpu_baseline else args.cpu_budget_s
    budget2 = 0.0 if args.no_cpu_baseline else args.secondary_cpu_budget_s
    if args.workload == "gather":
        return run_gather(args)
    if args.workload == "tiles":
        return run_tiles(args)
    if args.workload in ("varlen", "mla", "varlen-fp8", "mla-fp8"):
        line = as_line(prefill_entry(args, args.workload, budget), args)
    elif args.workload != "all":
        line = as_line(decode_entry(args, args.workload, budget, args.partition_size), args)
    else:
        # the whole metric: batched decode as the headline, then the prefill half and
        # the long-context split decode, each on its own timed steps
        head = decode_entry(args, "decode", budget, args.partition_size)
        torch.cuda.empty_cache()
        secondary = []
        for kind in ("varlen", "mla"):
            e = prefill_entry(args, kind, budget2)
            secondary.append(dict({"workload": e["config"]["workload"]}, **e))
            torch.cuda.empty_cache()
        e = decode_entry(args, "long", budget2)
        secondary.append(dict({"workload": e["config"]["workload"]}, **e))
        line = as_line(head, args, {"secondary": secondary})
    if args.ceilings:
        line["ceilings"] = ceilings()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
