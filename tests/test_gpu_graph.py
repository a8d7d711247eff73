"""The entry points captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.  The
library only launches kernels on the caller's stream (no allocation, memset, copy or
synchronisation), so a captured call must replay the eager call's work exactly.
Each graph is replayed three times, with the program's own eager work (outputs
overwritten, states reset) and synchronisations between replays, and every replay is
compared bit for bit with the eager results, which the other GPU tests check against
the oracle."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import (pa_decode, pa_gather_cache, pa_merge_states, pa_varlen, pa_varlen_merge,
                                          pa_write_kv)
from paged_kv_attention_table_amd import workloads as W
from paged_kv_attention_table_amd.chunked import ChunkedPrefillPlan
from tests.gpu_util import OnDevice, bits_equal, dev, host, workload

pytestmark = pytest.mark.gpu


def overwrite(t):
    t.fill_(-7 if t.dtype == torch.int32 else float("nan"))


def replays_match_eager(run, outputs, reset=None, reps=3):
    """run() issues the calls on the current stream and writes `outputs`; reset()
    (eager, never captured) restores any state the calls read back."""
    for t in outputs:
        overwrite(t)
    if reset:
        reset()
    run()
    torch.cuda.synchronize()
    eager = [host(t.clone()) for t in outputs]
    # warm-up on a side stream before capture, as torch asks
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        if reset:
            reset()
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(reps):
        for t in outputs:
            overwrite(t)
        if reset:
            reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, want) in enumerate(zip(outputs, eager)):
            assert bits_equal(host(t), want), f"replay {rep}: output {i} differs from the eager call"
    del g
    return eager


@pytest.mark.parametrize("P", [0, 64])
def test_graph_write_and_decode(P):
    """pa_write_kv then pa_decode (unsplit, and split with its reduce) in one graph."""
    w = workload("batched-decode-small")
    d = OnDevice(w, write=False)
    S, H = w.num_seqs, w.num_heads
    out = torch.empty((S, H, w.dv), device="cuda")
    ws = (None, None, None)
    if P:
        pm = -(-int(w.seq_lens.max()) // P)
        ws = tuple(torch.empty(sh, device="cuda") for sh in ((S, H, pm), (S, H, pm), (S, H, pm, w.dv)))
    st_w = torch.empty((1,), dtype=torch.int32, device="cuda")
    st_d = torch.empty((1,), dtype=torch.int32, device="cuda")

    def run():
        pa_write_kv(d.k_pool, d.v_pool, d.k_new, d.v_new, d.slots, status=st_w)
        pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale, sliding_window=w.sliding_window,
                  partition_size=P, max_logits=ws[0], exp_sums=ws[1], tmp_out=ws[2], status=st_d)

    replays_match_eager(run, [out, st_w, st_d])
    assert int(st_w.item()) == 0 and int(st_d.item()) == 0


@pytest.mark.parametrize("fp8", [False, True])
def test_graph_mixed_varlen(fp8):
    """Prefill tiles and single-token rows of one pa_varlen call, with lse and status
    (16-bit and fp8 caches)."""
    w = workload("mixed-varlen-small")
    if fp8:
        w = W.to_fp8(w, k_scale=0.0703125, v_scale=0.04296875)
    d = OnDevice(w)
    T, H = w.num_tokens, w.num_heads
    out = torch.empty((T, H, w.dv), dtype=d.q.dtype, device="cuda")
    lse = torch.empty((H, T), device="cuda")
    st = torch.empty((1,), dtype=torch.int32, device="cuda")
    max_q = int(np.diff(w.query_start_loc).max())

    def run():
        pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions, d.tables, max_q, w.scale, causal=True,
                  sliding_window=w.sliding_window, lse=lse, status=st, k_scale=w.k_scale, v_scale=w.v_scale)

    replays_match_eager(run, [out, lse, st])
    assert int(st.item()) == 0


def test_graph_varlen_merge_state_reset():
    """pa_varlen_merge reads the state it updates, so the state is reset eagerly before
    each replay; every replay must then give the eager merge."""
    w = workload("mixed-varlen-small")
    d = OnDevice(w)
    T, H = w.num_tokens, w.num_heads
    rng = np.random.default_rng(77)
    prior_out = torch.from_numpy(rng.standard_normal((T, H, w.dv)).astype(np.float32)).cuda()
    prior_lse = torch.from_numpy((rng.standard_normal((H, T)) * 3).astype(np.float32)).cuda()
    out = torch.empty_like(prior_out)
    lse = torch.empty_like(prior_lse)
    max_q = int(np.diff(w.query_start_loc).max())

    def reset():
        out.copy_(prior_out)
        lse.copy_(prior_lse)

    def run():
        pa_varlen_merge(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions, d.tables, max_q, w.scale,
                        causal=True, sliding_window=w.sliding_window, lse=lse)

    replays_match_eager(run, [out, lse], reset=reset)


@pytest.mark.parametrize("name", ["mla-chunked-small", "mla-chunked-small-fp8"])
def test_graph_chunked_prefill(name):
    """The chunked-context driver (one pa_varlen_ctx_new call per context chunk, the
    first writing the state and the others merging into it) captured whole (16-bit
    and fp8 caches)."""
    cp = workload(name)
    k_pool, v_pool = dev(cp.k_pool, cp.dtype), dev(cp.v_pool, cp.dtype)
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_write_kv(k_pool, v_pool, dev(cp.k_new, cp.dtype), dev(cp.v_new, cp.dtype), dev(cp.slot_mapping), status=st)
    plan = ChunkedPrefillPlan(ctx_lens=cp.ctx_lens, new_lens=cp.new_lens, ctx_tables=cp.ctx_tables,
                              new_tables=cp.new_tables, chunk=cp.chunk, block_size=cp.block_size,
                              num_heads=cp.num_heads, head_dim_v=cp.dv, scale=cp.scale)
    q = dev(cp.q, cp.query_dtype)
    out = torch.empty((cp.num_tokens, cp.num_heads, cp.dv), device="cuda")
    lse = torch.empty((cp.num_heads, cp.num_tokens), device="cuda")
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    replays_match_eager(lambda: plan.run(k_pool, v_pool, q, out, lse, k_scale=cp.k_scale, v_scale=cp.v_scale),
                        [out, lse])


def test_graph_merge_states_and_gather():
    """pa_merge_states (with +inf and -inf lse rows) and the latent-cache gather."""
    rng = np.random.default_rng(78)
    T, H, D = 300, 8, 128
    po, so = (torch.from_numpy(rng.standard_normal((T, H, D)).astype(np.float32)).cuda() for _ in range(2))
    pl, sl = ((rng.standard_normal((H, T)) * 3).astype(np.float32) for _ in range(2))
    pl[:, ::11] = np.inf
    sl[:, ::7] = -np.inf
    pl[:, ::13] = -np.inf
    pl, sl = torch.from_numpy(pl).cuda(), torch.from_numpy(sl).cuda()
    out = torch.empty((T, H, D), device="cuda")
    out_lse = torch.empty((H, T), device="cuda")
    g = W.latent_gather(small=True)
    cache = dev(g.cache, "bf16")
    n = int(g.cu_seq_lens[-1])
    dst = torch.empty((n, g.cache.shape[2]), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((1,), dtype=torch.int32, device="cuda")
    tables, cu, t2s = dev(g.block_tables), dev(g.cu_seq_lens), dev(g.token_to_seq)

    def run():
        pa_merge_states(out, out_lse, po, pl, so, sl)
        pa_gather_cache(cache, dst, tables, cu, t2s, status=st)

    replays_match_eager(run, [out, out_lse, dst, st])
    assert int(st.item()) == 0
