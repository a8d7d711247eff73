"""ALiBi ("paged_attention_v2_pytorch.py", phase 1) on the GPU against the CPU oracle:
the MFMA decode kernel (unsplit, split over 4 waves and over one wave, fp8 pools),
the per-row kernel (fp32, head dim 64), the tiled prefill kernel and its
single-token rows (causal and not, windows, Dqk 192), sinks beside ALiBi, and the
long-context split decode at full size (positions past 10^5, slopes up to 1/2).
The bias is counted from each row's last visible position, in the oracle and in the
kernels alike, so outputs, lse and partition maxima are compared directly."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_decode, pa_varlen
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, OnDevice, assert_close, host, threads, workload

pytestmark = pytest.mark.gpu


def slopes_for(H):
    """The geometric ALiBi slopes 2^(-8 (h + 1) / H), as float32."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


def check_decode(orc, w, P, sinks=None, window=None, pmax=None):
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    S, H = w.num_seqs, w.num_heads
    slopes = slopes_for(H)
    win = w.sliding_window if window is None else window
    out = torch.full((S, H, w.dv), float("nan"), device="cuda")
    ws = (None, None, None)
    if P:
        pmax = pmax or (w.max_partitions if P == w.partition_size and w.max_partitions else
                        -(-int(w.seq_lens.max()) // P))
        ws = tuple(torch.full(sh, float("nan"), device="cuda") for sh in ((S, H, pmax), (S, H, pmax),
                                                                          (S, H, pmax, w.dv)))
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale, sliding_window=win, partition_size=P,
              max_logits=ws[0], exp_sums=ws[1], tmp_out=ws[2], status=status,
              sinks=None if sinks is None else torch.from_numpy(sinks).cuda(), k_scale=w.k_scale,
              v_scale=w.v_scale, alibi_slopes=torch.from_numpy(slopes).cuda())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    kw = dict(sliding_window=win, threads=threads(), k_scale=w.k_scale, v_scale=w.v_scale,
              alibi_slopes=slopes.astype(np.float64))
    st, ref, _ = orc.decode(kp, vp, w.dtype, w.q, w.query_dtype, w.block_tables, w.seq_lens, w.scale,
                            sinks=None if sinks is None else sinks.astype(np.float64), **kw)
    assert st == 0
    tol = TOL[w.dtype]
    assert_close(host(out), ref, tol, f"{w.name} P={P} out")
    if P:
        st, rml, res, rto = orc.decode(kp, vp, w.dtype, w.q, w.query_dtype, w.block_tables, w.seq_lens, w.scale,
                                       partition_size=P, max_partitions=pmax, **kw)
        assert st == 0
        used = np.zeros(rml.shape, dtype=bool)
        for s, n in enumerate(w.seq_lens):
            used[s, :, :-(-int(n) // P)] = True
        ml, es, to = host(ws[0]), host(ws[1]), host(ws[2])
        # a partition far before the query has a large negative maximum (-slope times
        # its distance, up to about -6e4 here); binary32 holds it to a few units in the
        # last place, so the bar is 2e-3 plus 2^-20 of the magnitude
        gm, rm = ml[used].astype(np.float64), rml[used]
        fin = np.isfinite(rm)
        assert np.array_equal(np.isneginf(gm), np.isneginf(rm))
        err = np.abs(gm[fin] - rm[fin])
        assert np.all(err <= tol + 2.0 ** -20 * np.abs(rm[fin])), (err.max(), np.abs(rm[fin]).max())
        rel = np.abs(es[used] - res[used]) / np.maximum(res[used], 1e-30)
        assert np.all((res[used] == 0) == (es[used] == 0)) and rel.max() <= tol, rel.max()
        assert_close(to, rto, tol, "tmp_out", mask=used)


DECODE = [("tiny-decode", 0), ("tiny-decode", 16), ("batched-decode-small", 0), ("batched-decode-small", 512), ("long-decode-small", 512),
          ("batched-decode", 0), ("long-decode", 512)]


@pytest.mark.parametrize("name,P", DECODE, ids=[f"{n}-P{p}" for n, p in DECODE])
def test_alibi_decode(orc, name, P):
    check_decode(orc, workload(name), P)


def test_alibi_decode_one_wave_partitions_and_window(orc):
    check_decode(orc, workload("batched-decode-small"), 16, window=100, pmax=4096)


def test_alibi_decode_with_sinks(orc):
    w = workload("batched-decode-small")
    rng = np.random.default_rng(61)
    z = (rng.standard_normal(w.num_heads) * 3).astype(np.float32)
    z[::4] = -np.inf
    for P in (0, 512):
        check_decode(orc, w, P, sinks=z)


@pytest.mark.parametrize("P", [0, 512])
def test_alibi_decode_fp8(orc, P):
    check_decode(orc, W.to_fp8(workload("batched-decode-small"), q_dtype="bf16"), P)


def test_alibi_decode_fp8_one_wave_window(orc):
    """Split fp8 decode on one-wave workgroups (an oversized partition count gives
    enough items), with a window that empties whole partitions."""
    check_decode(orc, W.to_fp8(workload("long-decode-small"), q_dtype="bf16"), 64, window=200, pmax=4096)


def run_varlen(orc, w, causal, window):
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    T, H = w.num_tokens, w.num_heads
    slopes = slopes_for(H)
    out = torch.full((T, H, w.dv), float("nan"), device="cuda")
    lse = torch.full((H, T), float("nan"), device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    max_q = int(np.diff(w.query_start_loc).max())
    pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions if causal else None, d.tables, max_q,
              w.scale, causal=causal, sliding_window=window, lse=lse, status=status,
              alibi_slopes=torch.from_numpy(slopes).cuda())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    st, ref, rlse = orc.varlen(kp, vp, w.dtype, w.q, w.dtype, w.query_start_loc, w.seq_lens,
                               w.positions if causal else None, w.block_tables, w.scale, causal, window,
                               threads=threads(), alibi_slopes=slopes.astype(np.float64))
    assert st == 0
    assert_close(host(out), ref, TOL[w.dtype], f"{w.name} causal={causal} w={window} out")
    assert_close(host(lse), rlse, TOL[w.dtype], f"{w.name} causal={causal} w={window} lse")


VARLEN = [("mixed-varlen-small", True, None), ("mixed-varlen-small", True, 0), ("mixed-varlen-small", False, 0),
          ("mixed-varlen-small", False, 50), ("mixed-varlen-shuffled", True, None)]


@pytest.mark.parametrize("name,causal,window", VARLEN, ids=[f"{n}-c{int(c)}-w{w}" for n, c, w in VARLEN])
def test_alibi_varlen(orc, name, causal, window):
    w = workload(name)
    run_varlen(orc, w, causal, w.sliding_window if window is None else window)


def test_alibi_varlen_mla_dims(orc):
    """Dqk 192 / Dv 128 prefill tiles (their ALiBi instantiation), causal, plus a
    single-token row (per-row kernel)."""
    w = W.make_paged("alibi-mla-dims", 2300, dtype="bf16", block_size=16, num_heads=16, num_kv_heads=16, dk=192,
                     dv=128, segments=[(0, 70), (300, 33), (40, 1)], causal=True)
    run_varlen(orc, w, True, 0)
