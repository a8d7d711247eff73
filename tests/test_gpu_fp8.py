"""fp8 (E4M3) KV caches and the per-tensor k_scale / v_scale on the GPU against the
CPU oracle.

The fp8 workloads are the seeded decode / varlen workloads with every K / V value
divided by its scale and rounded to E4M3 (workloads.to_fp8); the queries stay f16 /
bf16.  The oracle decodes each stored byte exactly and multiplies by the scale
("paged_attention_v2_pytorch.py", phase 1), so the GPU path -- which widens bytes
exactly to the queries' type, folds k_scale into the softmax scale and v_scale into
the normalisation -- is held to the 16-bit bar.  Also here: the scales on 16-bit and
fp32 pools through every kernel (per-row, MFMA decode, split reduce, tiled prefill)."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_decode, pa_varlen
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, OnDevice, assert_close, bits_equal, host, threads, workload

pytestmark = pytest.mark.gpu


def fp8_workload(name, q_dtype=None, k_scale=1.0 / 16, v_scale=1.0 / 32):
    return W.to_fp8(workload(name), k_scale=k_scale, v_scale=v_scale, q_dtype=q_dtype)


def run_decode(d, P, pmax=None, window=None, sinks=None, out_dtype=torch.float32, k_scale=None, v_scale=None):
    w = d.w
    S, H = w.num_seqs, w.num_heads
    out = torch.full((S, H, w.dv), float("nan"), dtype=out_dtype, device="cuda")
    ws = (None, None, None)
    if P:
        pmax = pmax or max(1, -(-int(w.seq_lens.max()) // P))
        ws = tuple(torch.full(sh, float("nan"), device="cuda") for sh in ((S, H, pmax), (S, H, pmax),
                                                                          (S, H, pmax, w.dv)))
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale,
              sliding_window=w.sliding_window if window is None else window, partition_size=P, max_logits=ws[0],
              exp_sums=ws[1], tmp_out=ws[2], status=status,
              sinks=None if sinks is None else torch.from_numpy(sinks).cuda(),
              k_scale=w.k_scale if k_scale is None else k_scale, v_scale=w.v_scale if v_scale is None else v_scale)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out, ws


def oracle_decode(orc, w, kp, vp, window=None, P=0, pmax=0, sinks=None, k_scale=None, v_scale=None):
    return orc.decode(kp, vp, w.dtype, w.q, w.query_dtype, w.block_tables, w.seq_lens, w.scale,
                      sliding_window=w.sliding_window if window is None else window, partition_size=P,
                      max_partitions=pmax, threads=threads(),
                      sinks=None if sinks is None else sinks.astype(np.float64),
                      k_scale=w.k_scale if k_scale is None else k_scale,
                      v_scale=w.v_scale if v_scale is None else v_scale)


def check_decode(orc, w, P, pmax=None, window=None, sinks=None):
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    out, ws = run_decode(d, P, pmax, window, sinks)
    st, ref, _ = oracle_decode(orc, w, kp, vp, window, sinks=sinks)
    assert st == 0
    assert_close(host(out), ref, TOL[w.dtype], f"{w.name} P={P} out")
    if P:
        pm = ws[0].shape[-1]
        st, rml, res, rto = oracle_decode(orc, w, kp, vp, window, P, pm)
        assert st == 0
        used = np.zeros(rml.shape, dtype=bool)
        for s, n in enumerate(w.seq_lens):
            used[s, :, :-(-int(n) // P)] = True
        ml, es, to = host(ws[0]), host(ws[1]), host(ws[2])
        assert_close(ml, rml, TOL[w.dtype], "max_logits", mask=used)
        rel = np.abs(es[used] - res[used]) / np.maximum(res[used], 1e-30)
        assert np.all((res[used] == 0) == (es[used] == 0)) and rel.max() <= TOL[w.dtype], rel.max()
        assert_close(to, rto, TOL[w.dtype], "tmp_out", mask=used)
        assert np.all(np.isnan(ml[~used])) and np.all(np.isnan(to[~used])), "partitions past the context written"


@pytest.mark.parametrize("name", ["batched-decode-small", "long-decode-small"])
def test_fp8_write_kv_bit_exact(orc, name):
    w = fp8_workload(name)
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    assert bits_equal(host(d.k_pool), kp) and bits_equal(host(d.v_pool), vp)


# (workload, partition size, queries' type): unsplit (8 waves per workgroup), split
# with 4 waves per partition, and split with one wave per partition (long_decode: 8 x 8 x
# 256 items); both query types.
CASES = [("batched-decode-small", 0, "bf16"), ("batched-decode-small", 0, "f16"), ("batched-decode-small", 512, "bf16"),
         ("batched-decode-small", 16, "f16"), ("long-decode-small", 512, "bf16"), ("long-decode-small", 0, "f16"),
         ("batched-decode", 0, "f16"), ("batched-decode", 512, "bf16"), ("long-decode", 512, "bf16")]


@pytest.mark.parametrize("name,P,qd", CASES, ids=[f"{n}-P{p}-{q}" for n, p, q in CASES])
def test_fp8_decode_parity(orc, name, P, qd):
    w = fp8_workload(name, q_dtype=qd)
    check_decode(orc, w, P, pmax=w.max_partitions if P and P == w.partition_size and w.max_partitions else None)


def test_fp8_decode_one_wave_partitions(orc):
    """An oversized max_partitions on a small batch: one wave per partition, most
    partitions past the context (untouched), a window that empties some."""
    w = fp8_workload("batched-decode-small")
    check_decode(orc, w, 16, pmax=4096, window=100)


# Group sizes 1 / 8 / 16, block sizes 16 / 32 / 128, ragged lengths around the
# 16-position tiles (1, 15, 16, 17, ...), windows, and sinks.
SHAPES = [(8, 8, 16, 0, False), (16, 2, 32, 0, True), (32, 2, 128, 37, True), (16, 1, 16, 5, False),
          (64, 8, 64, 0, True), (16, 4, 16, 37, True), (48, 6, 32, 300, False)]


@pytest.mark.parametrize("H,Hkv,b,window,with_sinks", SHAPES,
                         ids=[f"H{h}-Hkv{k}-b{b}-w{w}-{'sinks' if z else 'nosinks'}" for h, k, b, w, z in SHAPES])
def test_fp8_decode_shapes(orc, H, Hkv, b, window, with_sinks):
    lens = [1, 15, 16, 17, 33, 100, 257, 1000, 1500]
    base = W.make_decode(f"fp8-shapes-H{H}-Hkv{Hkv}-b{b}", 2100 + H + b, seq_lens=lens, dtype="bf16", num_heads=H,
                         num_kv_heads=Hkv, head_dim=128, block_size=b, sliding_window=window)
    w = W.to_fp8(base, k_scale=0.0703125, v_scale=0.04296875)
    z = None
    if with_sinks:
        rng = np.random.default_rng(H * 7 + b)
        z = (rng.standard_normal(H) * 3).astype(np.float32)
        z[::3] = -np.inf
    for P in (0, max(64, b)):
        check_decode(orc, w, P, sinks=z)


def test_fp8_decode_out_in_query_type(orc):
    """Output in the queries' 16-bit type (the oracle's result rounded to it)."""
    for qd, tt, bits in (("bf16", torch.bfloat16, 8), ("f16", torch.float16, 11)):
        w = fp8_workload("batched-decode-small", q_dtype=qd)
        d = OnDevice(w)
        kp, vp = d.host_pools_after_write(orc)
        out, _ = run_decode(d, 0, out_dtype=tt)
        st, ref, _ = oracle_decode(orc, w, kp, vp)
        assert st == 0
        rt = torch.from_numpy(ref).to(tt).double().numpy()
        err = np.abs(out.double().cpu().numpy() - rt)
        ulp = np.abs(rt) * 2.0 ** (1 - bits)  # one unit in the last place of the 16-bit type, or more
        assert np.all(err <= ulp + TOL["fp8_e4m3"]), err.max()


def test_fp8_varlen_single_tokens(orc):
    """pa_varlen over an fp8 pool with one query token per sequence: causal tokens at
    positions before the end of their sequence, a window, the lse, and a sequence
    with no tokens."""
    segments = [(40, 1), (700, 1), (0, 1), (129, 0), (2000, 1), (15, 1)]
    base = W.make_paged("fp8-varlen-singles", 2200, dtype="bf16", block_size=16, num_heads=32, num_kv_heads=8,
                        dk=128, dv=128, segments=segments, causal=True, sliding_window=300)
    w = W.to_fp8(base, k_scale=0.05, v_scale=0.125)
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    # query positions moved back from the newest token (still inside each sequence)
    pos = w.positions.copy()
    pos[1] -= 200
    pos[3] -= 1000
    dpos = torch.from_numpy(pos).cuda()
    for causal in (True, False):
        out = torch.full((w.num_tokens, w.num_heads, w.dv), float("nan"), device="cuda")
        lse = torch.full((w.num_heads, w.num_tokens), float("nan"), device="cuda")
        status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, dpos if causal else None, d.tables, 1, w.scale,
                  causal=causal, sliding_window=w.sliding_window, lse=lse, status=status, k_scale=w.k_scale,
                  v_scale=w.v_scale)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        st, ref, rlse = orc.varlen(kp, vp, w.dtype, w.q, w.query_dtype, w.query_start_loc, w.seq_lens,
                                   pos if causal else None, w.block_tables, w.scale, causal, w.sliding_window,
                                   threads=threads(), k_scale=w.k_scale, v_scale=w.v_scale)
        assert st == 0
        assert_close(host(out), ref, TOL["fp8_e4m3"], f"causal={causal} out")
        assert_close(host(lse), rlse, TOL["fp8_e4m3"], f"causal={causal} lse")


# k_scale / v_scale on pools that are not fp8: (workload, entry point, partition size).
# tiny_decode is fp32 with head dim 64 (per-row kernel); batched-decode-small f16 (MFMA decode and
# the split reduce); mixed-varlen-small bf16 varlen (tiled prefill plus single-token rows).
SCALED = [("tiny-decode", "decode", 0), ("tiny-decode", "decode", 16), ("batched-decode-small", "decode", 0),
          ("batched-decode-small", "decode", 512), ("mixed-varlen-small", "varlen", 0)]


@pytest.mark.parametrize("name,call,P", SCALED, ids=[f"{n}-{c}-P{p}" for n, c, p in SCALED])
def test_scales_on_unquantized_pools(orc, name, call, P):
    ks, vs = 0.4375, 2.5
    w = workload(name)
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    tol = TOL[w.dtype] * vs
    if call == "decode":
        out, _ = run_decode(d, P, k_scale=ks, v_scale=vs)
        st, ref, _ = oracle_decode(orc, w, kp, vp, k_scale=ks, v_scale=vs)
        assert st == 0
        assert_close(host(out), ref, tol, f"{name} P={P}")
        return
    out = torch.full((w.num_tokens, w.num_heads, w.dv), float("nan"), device="cuda")
    lse = torch.full((w.num_heads, w.num_tokens), float("nan"), device="cuda")
    max_q = int(np.diff(w.query_start_loc).max())
    pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions, d.tables, max_q, w.scale, causal=True,
              sliding_window=w.sliding_window, lse=lse, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    st, ref, rlse = orc.varlen(kp, vp, w.dtype, w.q, w.dtype, w.query_start_loc, w.seq_lens, w.positions,
                               w.block_tables, w.scale, True, w.sliding_window, threads=threads(), k_scale=ks,
                               v_scale=vs)
    assert st == 0
    assert_close(host(out), ref, tol, f"{name} out")
    assert_close(host(lse), rlse, TOL[w.dtype], f"{name} lse")
