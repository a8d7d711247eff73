"""A seeded sweep of the varlen prefill path on the GPU against the CPU oracle: each
case draws one combination of the tiled kernel's options and checks every output
row and lse of a pa_varlen (or pa_varlen_merge) call.

Drawn per case: the pool type (f16, bf16, or fp8 E4M3 with f16 / bf16 queries and
random per-tensor scales), the head dims the tiled kernel takes for it, the kv
head count and head-group size (1 to 32 q heads per kv head), the block size (16 to
128), causal or not, a sliding window or none, attention sinks, ALiBi slopes, a
merge into a prior state, and 1 to 6 sequences of context 0..700 and 0..150 query
tokens (single tokens, empty sequences and ragged tails included).  A second sweep
draws pa_varlen_ctx_new calls (the two-segment kernel): contexts 0..600 and new
tokens 0..200 per sequence, 16-bit or fp8 pools, written or merged into a prior
state.  Sizes stay small so the oracle answers each case in well under a second."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_varlen, pa_varlen_merge
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, OnDevice, assert_close, dev, host, threads
from tests.test_gpu_ctx_new import CtxNewCase
from tests.test_gpu_fp8_prefill import Fp8CtxNewCase
from tests.test_gpu_varlen_merge import prior_state

pytestmark = pytest.mark.gpu

NCASES = 120


def draw(seed):
    rng = np.random.default_rng(40_000 + seed)
    kind = ["f16", "bf16", "fp8"][seed % 3]
    dims = [(128, 128), (192, 128)] + ([(64, 64)] if kind != "fp8" else [])
    dk, dv = dims[int(rng.integers(len(dims)))]
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 32]))
    while hkv * G > 64:
        hkv //= 2
    b = int(rng.choice([16, 32, 64, 128]))
    causal = bool(rng.integers(2))
    window = int(rng.choice([0, 0, 1, 33, 200]))
    nseq = int(rng.integers(1, 7))
    segs = []
    for _ in range(nseq):
        c = int(rng.choice([0, int(rng.integers(1, 700))]))
        n = int(rng.choice([0, 1, int(rng.integers(2, 150))]))
        segs.append((c, n))
    if sum(n for _, n in segs) == 0:
        segs[0] = (segs[0][0], 17)
    return dict(kind=kind, dk=dk, dv=dv, hkv=hkv, G=G, b=b, causal=causal, window=window, segs=segs,
                sinks=bool(rng.integers(2)), alibi=bool(rng.integers(3) == 0), merge=bool(rng.integers(3) == 0),
                qd=str(rng.choice(["f16", "bf16"])), ks=float(rng.choice([0.0625, 0.0703125, 0.125])),
                vs=float(rng.choice([0.03125, 0.04296875, 0.25])), seed=seed)


@pytest.mark.parametrize("seed", range(NCASES))
def test_prefill_sweep(orc, seed):
    c = draw(seed)
    base_dtype = c["qd"] if c["kind"] == "fp8" else c["kind"]
    H = c["hkv"] * c["G"]
    w = W.make_paged(f"sweep{seed}", 41_000 + seed, dtype=base_dtype, block_size=c["b"], num_heads=H,
                     num_kv_heads=c["hkv"], dk=c["dk"], dv=c["dv"], segments=c["segs"], causal=c["causal"],
                     sliding_window=c["window"])
    if c["kind"] == "fp8":
        w = W.to_fp8(w, k_scale=c["ks"], v_scale=c["vs"])
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    T = w.num_tokens
    rng = np.random.default_rng(42_000 + seed)
    sinks = rng.standard_normal(H) * 2 if c["sinks"] else None
    alibi = np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]) if c["alibi"] else None
    tens = lambda a: None if a is None else torch.from_numpy(np.asarray(a, np.float32)).cuda()  # noqa: E731
    max_q = int(np.diff(w.query_start_loc).max())
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pos = d.positions if c["causal"] else None
    if c["merge"]:
        po, pl = prior_state(43_000 + seed, T, H, w.dv)
        out = torch.from_numpy(po.copy()).cuda()
        lse = torch.from_numpy(pl.copy()).cuda()
        pa_varlen_merge(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, pos, d.tables, max_q, w.scale,
                        causal=c["causal"], sliding_window=c["window"], lse=lse, status=status, sinks=tens(sinks),
                        alibi_slopes=tens(alibi), k_scale=w.k_scale, v_scale=w.v_scale)
    else:
        out = torch.full((T, H, w.dv), float("nan"), device="cuda")
        lse = torch.full((H, T), float("nan"), device="cuda")
        pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, pos, d.tables, max_q, w.scale,
                  causal=c["causal"], sliding_window=c["window"], lse=lse, status=status, sinks=tens(sinks),
                  alibi_slopes=tens(alibi), k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, c
    f64 = lambda a: None if a is None else np.asarray(a, np.float64)  # noqa: E731
    st, ref, rlse = orc.varlen(kp, vp, w.dtype, w.q, w.query_dtype, w.query_start_loc, w.seq_lens,
                               w.positions if c["causal"] else None, w.block_tables, w.scale, c["causal"],
                               c["window"], threads=threads(), sinks=f64(sinks), alibi_slopes=f64(alibi),
                               k_scale=w.k_scale, v_scale=w.v_scale)
    assert st == 0
    if c["merge"]:
        ref, rlse = orc.merge_states(po, pl, ref.astype(np.float32), rlse.astype(np.float32), "f32")
    tol = TOL[w.dtype] * max(1.0, w.v_scale)
    assert_close(host(out), ref, tol, f"case {c} out")
    assert_close(host(lse), rlse, TOL[w.dtype], f"case {c} lse")


NCTX = 48


@pytest.mark.parametrize("seed", range(NCTX))
def test_ctx_new_sweep(orc, seed):
    rng = np.random.default_rng(44_000 + seed)
    kind = ["f16", "bf16", "fp8"][seed % 3]
    dk, dv = [(128, 128), (192, 128), (64, 64)][int(rng.integers(3 if kind != "fp8" else 2))]
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    b = int(rng.choice([16, 32, 64]))
    nseq = int(rng.integers(1, 6))
    ctx = [int(rng.choice([0, int(rng.integers(1, 600))])) for _ in range(nseq)]
    new = [int(rng.choice([0, 1, int(rng.integers(2, 200))])) for _ in range(nseq)]
    merge = bool(rng.integers(2))
    if kind == "fp8":
        qd = str(rng.choice(["f16", "bf16"]))
        cs = Fp8CtxNewCase(45_000 + seed, ctx, new, G * hkv, hkv, dk, dv, qd, b=b)
    else:
        cs = CtxNewCase(45_000 + seed, ctx, new, G * hkv, hkv, dk, dv, kind, b=b)
    att, alse = cs.expected(orc)
    H = G * hkv
    if merge:
        po, pl = prior_state(46_000 + seed, cs.T, H, dv)
        out, lse = dev(po.copy()), dev(pl.copy())
        ref, rlse = orc.merge_states(po, pl, att.astype(np.float32), alse.astype(np.float32), "f32")
    else:
        out = torch.full((cs.T, H, dv), float("nan"), device="cuda")
        lse = torch.full((H, cs.T), float("nan"), device="cuda")
        ref, rlse = att, alse
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    cs.run(out, lse, merge=merge, status=st)
    assert int(st.item()) == 0
    what = f"{kind} dims {dk}/{dv} Hkv {hkv} G {G} b {b} ctx {ctx} new {new} merge {merge}"
    assert_close(host(out), ref, TOL["bf16"], what + " out")
    assert_close(host(lse), rlse, TOL["bf16"], what + " lse")
