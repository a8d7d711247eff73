"""Prefill over fp8 (E4M3) caches on the GPU against the CPU oracle: pa_varlen,
pa_varlen_merge and pa_varlen_ctx_new with queries of several tokens, which run on
the tiled MFMA kernel with K widened to the queries' type and V to f16 as the tiles
are staged (single-token sequences of the MFMA decode kernel's shapes go to the fp8
decode kernel; of other shapes, to the tiled kernel too).

The workloads are the seeded varlen workloads with every K / V value divided by its
scale and rounded to E4M3 (workloads.to_fp8); the oracle decodes each stored byte
exactly and multiplies by the scale ("paged_attention_v2_pytorch.py", phase 1), so
the widening is exact and the 16-bit bar holds."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_varlen, pa_varlen_ctx_new
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, OnDevice, assert_close, dev, host, threads, workload
from tests.test_gpu_ctx_new import CtxNewCase
from tests.test_gpu_varlen_merge import check as merge_check

pytestmark = pytest.mark.gpu

KS, VS = 0.0703125, 0.04296875  # per-tensor scales: stored values span most of E4M3's range


def run_and_check(orc, w, causal=True, window=None, sinks=None, alibi=None):
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    window = w.sliding_window if window is None else window
    T, H = w.num_tokens, w.num_heads
    out = torch.full((T, H, w.dv), float("nan"), device="cuda")
    lse = torch.full((H, T), float("nan"), device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    tens = lambda a: None if a is None else torch.from_numpy(np.asarray(a, np.float32)).cuda()  # noqa: E731
    max_q = int(np.diff(w.query_start_loc).max())
    pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions if causal else None, d.tables, max_q,
              w.scale, causal=causal, sliding_window=window, lse=lse, status=status, sinks=tens(sinks),
              alibi_slopes=tens(alibi), k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    f64 = lambda a: None if a is None else np.asarray(a, np.float64)  # noqa: E731
    st, ref, rlse = orc.varlen(kp, vp, w.dtype, w.q, w.query_dtype, w.query_start_loc, w.seq_lens,
                               w.positions if causal else None, w.block_tables, w.scale, causal, window,
                               threads=threads(), sinks=f64(sinks), alibi_slopes=f64(alibi), k_scale=w.k_scale,
                               v_scale=w.v_scale)
    assert st == 0
    assert_close(host(out), ref, TOL["fp8_e4m3"], f"{w.name} out")
    assert_close(host(lse), rlse, TOL["fp8_e4m3"], f"{w.name} lse")


# (16-bit dtype the values are drawn in, queries' type, H, Hkv, dk, dv, segments
# (context, new tokens), causal, window, block size)
CASES = [
    # singles on the fp8 decode kernel beside tiles; ragged tails, an empty context
    ("bf16", "bf16", 32, 8, 128, 128, [(3000, 1), (100, 40), (0, 1), (50, 70), (2047, 1), (700, 300)], True, 0, 16),
    ("f16", "f16", 16, 4, 128, 128, [(3, 50), (140, 1), (0, 129), (33, 17), (500, 64)], True, 200, 32),
    # f16 queries over values drawn in bf16; a head group of 3; blocks of 64
    ("bf16", "f16", 6, 2, 128, 128, [(7, 100), (0, 1), (250, 45)], True, 0, 64),
    # MLA head dims: single tokens go through the tiled kernel as well
    ("bf16", "bf16", 8, 8, 192, 128, [(0, 70), (300, 21), (17, 1), (64, 64), (1000, 1)], True, 0, 16),
    ("f16", "f16", 16, 1, 192, 128, [(1709, 40), (0, 33)], False, 0, 16),
    # 32 q heads per kv head: beyond the decode kernel, everything on the tiled one
    ("bf16", "bf16", 32, 1, 128, 128, [(50, 1), (20, 9), (0, 1)], True, 0, 16),
    # blocks of 128 positions (a 32-key tile inside one block)
    ("f16", "bf16", 16, 2, 192, 128, [(900, 77), (0, 200), (130, 1)], True, 300, 128),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fp8_varlen_prefill(orc, case):
    dtype, qd, H, Hkv, dk, dv, segs, causal, window, b = CASES[case]
    base = W.make_paged(f"fp8-prefill{case}", 3100 + case, dtype=dtype, block_size=b, num_heads=H, num_kv_heads=Hkv,
                        dk=dk, dv=dv, segments=segs, causal=causal, sliding_window=window)
    run_and_check(orc, W.to_fp8(base, k_scale=KS, v_scale=VS, q_dtype=qd), causal=causal)


def test_fp8_prefill_empty_sequences_and_loose_bound(orc):
    """A sequence with no query tokens between others, a context-free single token,
    and max_query_len above the longest sequence (the grid then holds tiles past
    every sequence's end, which exit)."""
    base = W.make_paged("fp8-prefill-empty", 3500, dtype="bf16", block_size=16, num_heads=8, num_kv_heads=2, dk=128,
                        dv=128, segments=[(40, 70), (129, 0), (0, 1), (300, 45), (7, 0)], causal=True,
                        sliding_window=0)
    w = W.to_fp8(base, k_scale=KS, v_scale=VS)
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    out = torch.full((w.num_tokens, w.num_heads, w.dv), float("nan"), device="cuda")
    lse = torch.full((w.num_heads, w.num_tokens), float("nan"), device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions, d.tables, 400, w.scale, causal=True,
              lse=lse, status=status, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    st, ref, rlse = orc.varlen(kp, vp, w.dtype, w.q, w.query_dtype, w.query_start_loc, w.seq_lens, w.positions,
                               w.block_tables, w.scale, True, 0, threads=threads(), k_scale=w.k_scale,
                               v_scale=w.v_scale)
    assert st == 0
    assert_close(host(out), ref, TOL["fp8_e4m3"], "out")
    assert_close(host(lse), rlse, TOL["fp8_e4m3"], "lse")


@pytest.mark.parametrize("qd", ["bf16", "f16"])
def test_fp8_prefill_out_in_query_type(orc, qd):
    """Outputs in the queries' 16-bit type: the oracle's result rounded to that type,
    within one unit in its last place plus the bound."""
    from tests.gpu_util import TORCH

    w = W.to_fp8(workload("mixed-varlen-small"), k_scale=KS, v_scale=VS, q_dtype=qd)
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    out = torch.full((w.num_tokens, w.num_heads, w.dv), float("nan"), dtype=TORCH[qd], device="cuda")
    max_q = int(np.diff(w.query_start_loc).max())
    pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions, d.tables, max_q, w.scale, causal=True,
              sliding_window=w.sliding_window, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    st, ref, _ = orc.varlen(kp, vp, w.dtype, w.q, w.query_dtype, w.query_start_loc, w.seq_lens, w.positions,
                            w.block_tables, w.scale, True, w.sliding_window, threads=threads(), k_scale=w.k_scale,
                            v_scale=w.v_scale)
    assert st == 0
    rt = torch.from_numpy(ref).to(TORCH[qd]).double().numpy()
    err = np.abs(out.double().cpu().numpy() - rt)
    ulp = np.abs(rt) * 2.0 ** (1 - (8 if qd == "bf16" else 11))
    assert np.all(err <= ulp + TOL["fp8_e4m3"]), err.max()


@pytest.mark.parametrize("name", ["mixed-varlen-small", "mixed-varlen-shuffled"])
def test_fp8_mixed_varlen_workloads(orc, name):
    run_and_check(orc, W.to_fp8(workload(name), k_scale=KS, v_scale=VS))


def test_fp8_prefill_sinks_and_alibi(orc):
    base = W.make_paged("fp8-prefill-sinks", 3200, dtype="bf16", block_size=16, num_heads=16, num_kv_heads=4, dk=128,
                        dv=128, segments=[(400, 90), (0, 33), (77, 1), (1500, 17)], causal=True, sliding_window=0)
    w = W.to_fp8(base, k_scale=KS, v_scale=VS)
    rng = np.random.default_rng(3201)
    z = rng.standard_normal(w.num_heads) * 2
    z[::3] = -np.inf
    slopes = np.array([2.0 ** (-8.0 * (h + 1) / w.num_heads) for h in range(w.num_heads)])
    run_and_check(orc, w, sinks=z)
    run_and_check(orc, w, alibi=slopes)
    run_and_check(orc, w, sinks=z, alibi=slopes, window=129)


@pytest.mark.parametrize("dk", [128, 192])
def test_fp8_prefill_merged_into_a_state(orc, dk):
    base = W.make_paged(f"fp8-prefill-merge{dk}", 3300 + dk, dtype="bf16", block_size=16, num_heads=8,
                        num_kv_heads=2 if dk == 128 else 8, dk=dk, dv=128,
                        segments=[(300, 45), (0, 1), (64, 64), (900, 1), (5, 130)], causal=True, sliding_window=0)
    w = W.to_fp8(base, k_scale=KS, v_scale=VS)
    merge_check(orc, w)
    merge_check(orc, w, causal=False, window=0)


class Fp8CtxNewCase(CtxNewCase):
    """A CtxNewCase whose pools are rounded to E4M3 after division by the scales."""

    def __init__(self, seed, ctx, new, H, Hkv, dk, dv, q_dtype, b=16):
        super().__init__(seed, ctx, new, H, Hkv, dk, dv, q_dtype, b=b)
        self.q_dtype = q_dtype
        self.k_pool = W.quantize_e4m3(W.widen_storage(self.k_pool, q_dtype), KS)
        self.v_pool = W.quantize_e4m3(W.widen_storage(self.v_pool, q_dtype), VS)
        self.dtype = "fp8_e4m3"

    def run(self, out, lse, merge, status=None):
        pa_varlen_ctx_new(dev(self.k_pool, "fp8_e4m3"), dev(self.v_pool, "fp8_e4m3"), dev(self.q, self.q_dtype), out,
                          lse, dev(self.qsl), dev(np.array(self.ctx, np.int32)), dev(self.ctx_tables),
                          dev(np.array(self.new, np.int32)), dev(self.positions), dev(self.new_tables),
                          max(self.q_counts), self.scale, merge=merge, status=status, k_scale=KS, v_scale=VS)
        torch.cuda.synchronize()

    def expected(self, orc):
        out = np.zeros((self.T, self.H, self.dv))
        lse = np.zeros((self.H, self.T))
        q64 = orc.decode_elems(self.q, self.q_dtype)
        G = self.H // self.Hkv
        for r in range(len(self.ctx)):
            c, n = self.ctx[r], self.new[r]
            g = lambda pool, tab, m: orc.gather(pool, "fp8_e4m3", self.b, tab, m)  # noqa: E731
            K = KS * np.concatenate([g(self.k_pool, self.ctx_tables[r], c), g(self.k_pool, self.new_tables[r], n)])
            V = VS * np.concatenate([g(self.v_pool, self.ctx_tables[r], c), g(self.v_pool, self.new_tables[r], n)])
            t0, t1 = int(self.qsl[r]), int(self.qsl[r + 1])
            hi = c + np.arange(1, n + 1) if n > 0 else np.array([c])
            for h in range(self.H):
                o, l = orc.attend_gathered(q64[t0:t1, h], K[:, h // G], V[:, h // G], np.zeros(t1 - t0, np.int64), hi,
                                           self.scale)
                out[t0:t1, h] = o
                lse[h, t0:t1] = l
        return out, lse


CTX = [
    # (queries' type, H, Hkv, dk, dv, ctx, new)
    ("bf16", 8, 8, 192, 128, [0, 32, 1709, 100], [40, 130, 1, 77]),
    ("f16", 8, 2, 128, 128, [300, 0, 64, 17, 5], [129, 33, 0, 200, 1]),
]


@pytest.mark.parametrize("case", range(len(CTX)))
@pytest.mark.parametrize("merge", [False, True])
def test_fp8_ctx_new(orc, case, merge):
    qd, H, Hkv, dk, dv, ctx, new = CTX[case]
    cs = Fp8CtxNewCase(3400 + case, ctx, new, H, Hkv, dk, dv, qd)
    att, alse = cs.expected(orc)
    if merge:
        po, pl, _, _, _ = W.merge_case(3450 + case, cs.T, H, dv, special_fraction=0.1)
        out, lse = dev(po.copy()), dev(pl.copy())
        ref, rlse = orc.merge_states(po, pl, att.astype(np.float32), alse.astype(np.float32), "f32")
    else:
        out = torch.full((cs.T, H, dv), float("nan"), device="cuda")
        lse = torch.full((H, cs.T), float("nan"), device="cuda")
        ref, rlse = att, alse
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    cs.run(out, lse, merge=merge, status=st)
    assert int(st.item()) == 0
    assert_close(host(out), ref, TOL["fp8_e4m3"], "out")
    assert_close(host(lse), rlse, TOL["fp8_e4m3"], "lse")
