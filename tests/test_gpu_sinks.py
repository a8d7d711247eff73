"""Attention sinks (TensorSharp page, ForwardWithSinks) on the GPU against the CPU
oracle: pa_decode unsplit and split (the sink joins in the reduction), pa_varlen on
the tiled kernel, its single-token rows and the per-row kernel, rows that see
nothing (out = 0, lse = the sink), and sinks of -inf, below, among and far above
the scores."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_decode, pa_varlen
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, OnDevice, assert_close, host, threads, workload

pytestmark = pytest.mark.gpu


def make_sinks(H, seed):
    """Seeded float32 sink logits: N(0, 3), with -inf and a dominant +14 mixed in."""
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal(H) * 3.0).astype(np.float32)
    z[::5] = -np.inf
    z[3 % H] = 14.0
    return z


def run_decode(d, z, P):
    w = d.w
    S, H = w.num_seqs, w.num_heads
    out = torch.full((S, H, w.dv), float("nan"), device="cuda")
    ws = (None, None, None)
    if P:
        pmax = max(1, -(-int(w.seq_lens.max()) // P))
        ws = tuple(torch.full(sh, float("nan"), device="cuda") for sh in ((S, H, pmax), (S, H, pmax),
                                                                          (S, H, pmax, w.dv)))
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale, sliding_window=w.sliding_window,
              partition_size=P, max_logits=ws[0], exp_sums=ws[1], tmp_out=ws[2], status=status,
              sinks=torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out, ws


@pytest.mark.parametrize("name,P", [("tiny-decode", 0), ("tiny-decode", 16), ("batched-decode-small", 0), ("batched-decode-small", 512),
                                    ("long-decode-small", 0), ("long-decode-small", 512), ("batched-decode", 0)])
def test_decode_with_sinks(orc, name, P):
    w = workload(name)
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    z = make_sinks(w.num_heads, 41)
    out, ws = run_decode(d, z, P)
    st, ref, _ = orc.decode(kp, vp, w.dtype, w.q, w.dtype, w.block_tables, w.seq_lens, w.scale,
                            sliding_window=w.sliding_window, threads=threads(), sinks=z.astype(np.float64))
    assert st == 0
    assert_close(host(out), ref, TOL[w.dtype], f"{name} P={P} out")
    if P:  # the partition states stay sink-free
        st, rml, _, rto = orc.decode(kp, vp, w.dtype, w.q, w.dtype, w.block_tables, w.seq_lens, w.scale,
                                     sliding_window=w.sliding_window, partition_size=P,
                                     max_partitions=ws[0].shape[-1], threads=threads())
        used = np.zeros(rml.shape, dtype=bool)
        for s, n in enumerate(w.seq_lens):
            used[s, :, :-(-int(n) // P)] = True
        assert_close(host(ws[0]), rml, TOL[w.dtype], "max_logits", mask=used)
        assert_close(host(ws[2]), rto, TOL[w.dtype], "tmp_out", mask=used)


def run_varlen(d, z):
    w = d.w
    T, H = w.num_tokens, w.num_heads
    out = torch.full((T, H, w.dv), float("nan"), device="cuda")
    lse = torch.full((H, T), float("nan"), device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    max_q = int(np.diff(w.query_start_loc).max()) if w.num_seqs else 0
    pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions if w.causal else None, d.tables, max_q,
              w.scale, causal=w.causal, sliding_window=w.sliding_window, lse=lse, status=status,
              sinks=torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out, lse


VARLEN = [
    # tiled kernel (D 128, pipelined) plus single-token rows on the decode kernel
    ("mixed-varlen-small", None),
    # (dtype, H, Hkv, dk, dv, segments, causal, window, block_size)
    ("small", ("bf16", 6, 6, 192, 128, [(0, 70), (300, 21), (17, 0), (64, 64), (90, 1)], True, 0, 16)),
    ("small", ("bf16", 4, 1, 64, 64, [(300, 130), (0, 2), (77, 1)], False, 0, 16)),
    ("small", ("f32", 4, 2, 64, 64, [(0, 37), (20, 1), (5, 16), (90, 3)], True, 25, 16)),
    ("small", ("f16", 32, 8, 128, 128, [(40, 9), (3, 1), (0, 20), (700, 1)], True, 17, 16)),
]


@pytest.mark.parametrize("case", range(len(VARLEN)))
def test_varlen_with_sinks(orc, case):
    name, spec = VARLEN[case]
    if spec is None:
        w = workload(name)
    else:
        dtype, H, Hkv, dk, dv, segs, causal, window, b = spec
        w = W.make_paged(f"sinks{case}", 800 + case, dtype=dtype, block_size=b, num_heads=H, num_kv_heads=Hkv,
                         dk=dk, dv=dv, segments=segs, causal=causal, sliding_window=window)
    d = OnDevice(w)
    z = make_sinks(w.num_heads, 50 + case)
    out, lse = run_varlen(d, z)
    kp, vp = d.host_pools_after_write(orc)
    st, ref, rlse = orc.varlen(kp, vp, w.dtype, w.q, w.dtype, w.query_start_loc, w.seq_lens,
                               w.positions if w.causal else None, w.block_tables, w.scale, w.causal,
                               w.sliding_window, threads=threads(), sinks=z.astype(np.float64))
    assert st == 0
    assert_close(host(out), ref, TOL[w.dtype], "out")
    assert_close(host(lse), rlse, TOL[w.dtype], "lse")


def test_varlen_sinks_on_rows_that_see_nothing(orc):
    """Sequences with no cached position (non-causal): out = 0, lse = the sink (-inf
    where there is none)."""
    w = W.make_paged("sinks-empty", 870, dtype="bf16", block_size=16, num_heads=8, num_kv_heads=2, dk=128, dv=128,
                     segments=[(0, 5), (40, 3), (0, 1)], causal=False, sliding_window=0)
    d = OnDevice(w, write=False)
    z = make_sinks(8, 71)
    d.seq_lens.copy_(torch.tensor([0, 40, 0], dtype=torch.int32))
    out, lse = run_varlen(d, z)
    o, l = host(out), host(lse)
    rows = list(range(0, 5)) + [8]
    assert np.all(o[rows] == 0.0)
    for t in rows:
        np.testing.assert_allclose(l[:, t], z.astype(np.float64), rtol=2e-6, atol=0)
    assert np.all(np.isfinite(o[5:8]))
