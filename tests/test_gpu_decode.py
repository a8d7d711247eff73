"""pa_decode (unsplit and split-KV) and pa_write_kv on the GPU against the CPU oracle.

Inputs are the seeded workloads of paged_kv_attention_table_amd.workloads with
NaN-poisoned unused slots; the new token of every sequence is written through
pa_write_kv first (bit-exact against the oracle's write), then decoded."""
import math

import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_decode, pa_write_kv
from tests.gpu_util import TOL, OnDevice, assert_close, bits_equal, dev, host, threads, workload

pytestmark = pytest.mark.gpu


def run_decode(d, P, pmax=None, out_dtype=torch.float32, sliding_window=None):
    w = d.w
    S, H = w.num_seqs, w.num_heads
    out = torch.full((S, H, w.dv), float("nan"), dtype=out_dtype, device="cuda")
    ws = (None, None, None)
    if P:
        pmax = pmax or max(1, -(-int(w.seq_lens.max()) // P))
        ws = (torch.full((S, H, pmax), float("nan"), device="cuda"),
              torch.full((S, H, pmax), float("nan"), device="cuda"),
              torch.full((S, H, pmax, w.dv), float("nan"), device="cuda"))
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    win = w.sliding_window if sliding_window is None else sliding_window
    pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale, sliding_window=win, partition_size=P,
              max_logits=ws[0], exp_sums=ws[1], tmp_out=ws[2], status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out, ws


@pytest.mark.parametrize("name", ["tiny-decode", "batched-decode-small", "long-decode-small", "mixed-varlen-small"])
def test_write_kv_bit_exact(orc, name):
    w = workload(name)
    d = OnDevice(w)  # writes through pa_write_kv with a status word
    kp, vp = d.host_pools_after_write(orc)
    assert bits_equal(host(d.k_pool), kp) and bits_equal(host(d.v_pool), vp)


CASES = [("tiny-decode", 0), ("batched-decode-small", 0), ("batched-decode-small", 512), ("batched-decode-small", 32), ("batched-decode-small", 16),
         ("long-decode-small", 512), ("long-decode-small", 0), ("batched-decode", 512), ("batched-decode", 0), ("batched-decode", 1024),
         ("long-decode", 512)]


def check_decode(orc, name, P, pmax=None, window=None):
    """GPU decode (and, when split, every used partition state) against the oracle;
    partition entries past each sequence's context must stay untouched."""
    w = workload(name)
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    if pmax is None and P and P == w.partition_size and w.max_partitions:
        pmax = w.max_partitions
    win = w.sliding_window if window is None else window
    out, ws = run_decode(d, P, pmax, sliding_window=win)
    st, ref, _ = orc.decode(kp, vp, w.dtype, w.q, w.dtype, w.block_tables, w.seq_lens, w.scale,
                            sliding_window=win, threads=threads())
    assert st == 0
    tol = TOL[w.dtype]
    assert_close(host(out), ref, tol, f"{name} out")
    if P:
        pmax = ws[0].shape[-1]
        st, rml, res, rto = orc.decode(kp, vp, w.dtype, w.q, w.dtype, w.block_tables, w.seq_lens, w.scale,
                                       sliding_window=win, partition_size=P, max_partitions=pmax,
                                       threads=threads())
        assert st == 0
        ml, es, to = host(ws[0]), host(ws[1]), host(ws[2])
        used = np.zeros(ml.shape, dtype=bool)
        for s, n in enumerate(w.seq_lens):
            used[s, :, :-(-int(n) // P)] = True
        assert_close(ml, rml, tol, "max_logits", mask=used)
        rel = np.abs(es[used] - res[used]) / np.maximum(res[used], 1e-30)
        assert np.all((res[used] == 0) == (es[used] == 0)) and rel.max() <= tol, rel.max()
        assert_close(to, rto, tol, "tmp_out", mask=used)
        assert np.all(np.isnan(ml[~used])) and np.all(np.isnan(to[~used])), "partitions past the context written"


@pytest.mark.parametrize("name,P", CASES, ids=[f"{n}-P{p}" for n, p in CASES])
def test_decode_parity(orc, name, P):
    check_decode(orc, name, P)


# An oversized max_partitions gives the launcher enough (row, kv head, partition)
# items to run one wave per partition (the layout the long-context workload uses) on
# small inputs: most partitions lie past the context and must stay untouched, and
# the window empties some partitions wholly.
ONE_WAVE = [("batched-decode-small", 16, 4096, 0), ("batched-decode-small", 16, 4096, 100), ("long-decode-small", 64, 2048, 0),
           ("long-decode-small", 32, 1000, 700)]


@pytest.mark.parametrize("name,P,pmax,win", ONE_WAVE, ids=[f"{n}-P{p}-pmax{m}-w{w}" for n, p, m, w in ONE_WAVE])
def test_decode_one_wave_partitions(orc, name, P, pmax, win):
    check_decode(orc, name, P, pmax=pmax, window=win)


def test_decode_window_and_out_dtype(orc):
    """A sliding window on a split decode, and an f16 output (oracle rounded to f16)."""
    w = workload("batched-decode-small")
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    for win, P in ((100, 0), (100, 64), (1, 0), (333, 512)):
        out, _ = run_decode(d, P, sliding_window=win)
        st, ref, _ = orc.decode(kp, vp, w.dtype, w.q, w.dtype, w.block_tables, w.seq_lens, w.scale,
                                sliding_window=win, threads=threads())
        assert_close(host(out), ref, TOL[w.dtype], f"window {win} P {P}")
    out, _ = run_decode(d, 0, out_dtype=torch.float16)
    st, ref, _ = orc.decode(kp, vp, w.dtype, w.q, w.dtype, w.block_tables, w.seq_lens, w.scale, threads=threads())
    ref16 = ref.astype(np.float16).astype(np.float64)
    ulp = np.abs(np.spacing(ref.astype(np.float16))).astype(np.float64)
    err = np.abs(host(out).astype(np.float64) - ref16)
    assert np.all(err <= ulp + TOL["f16"]), err.max()


@pytest.mark.parametrize("P", [0, 512])
def test_decode_batch_invariance(P):
    """A sequence decoded alone gives the same bits as in the batch (decode page,
    section 2.5): the reduction order depends only on the sequence."""
    w = workload("batched-decode-small")
    d = OnDevice(w)
    out, _ = run_decode(d, P)
    full = host(out)
    for s in range(w.num_seqs):
        o = torch.full((1, w.num_heads, w.dv), float("nan"), device="cuda")
        ws = (None, None, None)
        if P:
            pm = -(-int(w.seq_lens.max()) // P)
            ws = tuple(torch.empty(sh, device="cuda") for sh in ((1, w.num_heads, pm), (1, w.num_heads, pm),
                                                                 (1, w.num_heads, pm, w.dv)))
        pa_decode(d.k_pool, d.v_pool, d.q[s:s + 1].contiguous(), o, d.tables[s:s + 1].contiguous(),
                  d.seq_lens[s:s + 1].contiguous(), w.scale, partition_size=P, max_logits=ws[0], exp_sums=ws[1],
                  tmp_out=ws[2])
        torch.cuda.synchronize()
        assert bits_equal(host(o)[0], full[s]), f"sequence {s}"


def test_decode_forks_read_shared_blocks():
    """Two sequences whose tables name the same blocks, with the same query, give
    the same bits."""
    w = workload("batched-decode-small")
    d = OnDevice(w)
    forks = [s for s in range(w.num_seqs) if np.array_equal(w.block_tables[s, :2], w.block_tables[0, :2])]
    tables = d.tables.clone()
    lens = d.seq_lens.clone()
    q = d.q.clone()
    tables[1] = tables[0]
    lens[1] = lens[0]
    q[1] = q[0]
    out = torch.empty((w.num_seqs, w.num_heads, w.dv), device="cuda")
    pa_decode(d.k_pool, d.v_pool, q, out, tables, lens, w.scale)
    torch.cuda.synchronize()
    assert bits_equal(host(out[0]), host(out[1]))
    assert len(forks) >= 1


def test_indexing_probe_bit_exact():
    """V holds its own slot id (exact in fp32); with a window of one position the
    output must be exactly V at the slot of position n - 1, for every row."""
    rng = np.random.default_rng(77)
    nb, b, hkv, D, H = 40, 16, 2, 64, 8
    lens = rng.integers(1, 120, size=9)
    tables = np.stack([rng.permutation(nb)[:8] for _ in lens]).astype(np.int32)
    slot_ids = np.arange(nb * b, dtype=np.float32).reshape(nb, b, 1, 1)
    v = np.broadcast_to(slot_ids * 4 + np.arange(hkv, dtype=np.float32).reshape(1, 1, hkv, 1),
                        (nb, b, hkv, D)).copy()
    v += np.arange(D, dtype=np.float32) / 128.0
    k = rng.standard_normal((nb, b, hkv, D)).astype(np.float32)
    q = rng.standard_normal((lens.size, H, D)).astype(np.float32)
    out = torch.empty((lens.size, H, D), device="cuda")
    pa_decode(dev(k), dev(v), dev(q), out, dev(tables), dev(lens.astype(np.int32)), 0.125, sliding_window=1)
    torch.cuda.synchronize()
    got = host(out)
    for s, n in enumerate(lens):
        j = n - 1
        slot = tables[s, j // b] * b + j % b
        for h in range(H):
            assert np.array_equal(got[s, h], v.reshape(-1, hkv, D)[slot, h // (H // hkv)])


def test_write_kv_status_rejects_bad_slot():
    w = workload("batched-decode-small")
    d = OnDevice(w, write=False)
    before_k, before_v = host(d.k_pool).copy(), host(d.v_pool).copy()
    for bad in (w.num_blocks * w.block_size, -1):
        slots = d.slots.clone()
        slots[3] = bad
        st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        pa_write_kv(d.k_pool, d.v_pool, d.k_new, d.v_new, slots, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 1
        assert bits_equal(host(d.k_pool), before_k) and bits_equal(host(d.v_pool), before_v)


@pytest.mark.parametrize("dtype", ["f16", "fp8_e4m3"])
def test_decode_paired_units(orc, dtype):
    """Unsplit calls of at least two rounds of the chip's CUs run two (row, kv head)
    units per workgroup (the longest with the shortest).  515 sequences x 1 kv head
    (an odd count: the middle workgroup answers one unit) against the oracle, and
    every sampled sequence bit for bit against the same sequence in a call of 8
    sequences, which runs one unit per workgroup."""
    from paged_kv_attention_table_amd import workloads as W

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = max(515, 2 * cus + 3) | 1
    rng = np.random.default_rng(4242)
    lens = rng.integers(1, 300, size=S, endpoint=True)
    w = W.make_decode("paired-units", 4242, seq_lens=lens, dtype="f16", num_heads=4, num_kv_heads=1, head_dim=128)
    if dtype == "fp8_e4m3":
        w = W.to_fp8(w)
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    out = torch.full((S, w.num_heads, w.dv), float("nan"), device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale, k_scale=w.k_scale, v_scale=w.v_scale,
              status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    full = host(out)
    st, ref, _ = orc.decode(kp, vp, w.dtype, w.q, w.query_dtype, w.block_tables, w.seq_lens, w.scale,
                            k_scale=w.k_scale, v_scale=w.v_scale, threads=threads())
    assert st == 0
    assert_close(full, ref, TOL["f16"], f"{dtype} paired out")
    for s0 in (0, 8 * (S // 16), S - 8):
        sl = slice(s0, s0 + 8)
        o = torch.full((8, w.num_heads, w.dv), float("nan"), device="cuda")
        pa_decode(d.k_pool, d.v_pool, d.q[sl].contiguous(), o, d.tables[sl].contiguous(), d.seq_lens[sl].contiguous(),
                  w.scale, k_scale=w.k_scale, v_scale=w.v_scale)
        torch.cuda.synchronize()
        assert bits_equal(host(o), full[sl]), f"sequences {s0}..{s0 + 7}"
