"""pa_varlen_ctx_new (a context segment and the new tokens in one softmax) on the
GPU against the CPU oracle.

The expected result is the definition ("cpu_mla_prefill.cpp": MlaPrefillAttention
over the context and the new tokens, merged by MergeAttnStates): token i of a
sequence sees every context position and new positions 0..i, both gathered
explicitly through their tables; the oracle's two-pass core answers each row, and
with merge its MergeAttnStates folds the result into a prior state.  Contexts of
length 0, of whole tiles and of ragged lengths, sequences without new tokens (their
positions are never read), GQA and the MLA head dims are covered."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_varlen_ctx_new
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, assert_close, dev, host, threads

pytestmark = pytest.mark.gpu


class CtxNewCase:
    """Contexts and new tokens of several sequences in one permuted block pool, each
    segment starting on a block boundary of its own table; unused slots hold NaN."""

    def __init__(self, seed, ctx, new, H, Hkv, dk, dv, dtype, b=16):
        rng = np.random.default_rng(seed)
        self.ctx, self.new = list(ctx), list(new)
        self.H, self.Hkv, self.dk, self.dv, self.dtype, self.b = H, Hkv, dk, dv, dtype, b
        cb = [-(-c // b) for c in ctx]
        nbk = [-(-n // b) for n in new]
        nb = sum(cb) + sum(nbk) + 1
        ids = rng.permutation(nb)
        self.ctx_tables = np.full((len(ctx), max(1, max(cb))), ids[-1], np.int32)
        self.new_tables = np.full((len(ctx), max(1, max(nbk))), ids[-1], np.int32)
        cur = 0
        for r in range(len(ctx)):
            self.ctx_tables[r, :cb[r]] = ids[cur:cur + cb[r]]
            cur += cb[r]
            self.new_tables[r, :nbk[r]] = ids[cur:cur + nbk[r]]
            cur += nbk[r]
        nan = W.nan_value(dtype)
        self.k_pool = np.full((nb, b, Hkv, dk), nan, dtype=W.STORAGE[dtype])
        self.v_pool = np.full((nb, b, Hkv, dv), nan, dtype=W.STORAGE[dtype])
        for r in range(len(ctx)):
            for tab, n in ((self.ctx_tables[r], ctx[r]), (self.new_tables[r], new[r])):
                for j in range(n):
                    self.k_pool[tab[j // b], j % b] = W._round_to(rng.standard_normal((Hkv, dk)).astype(np.float32),
                                                                  dtype)
                    self.v_pool[tab[j // b], j % b] = W._round_to(rng.standard_normal((Hkv, dv)).astype(np.float32),
                                                                  dtype)
        # sequences without new tokens still own query rows (one here): they see the
        # context alone
        self.q_counts = [n if n > 0 else 1 for n in new]
        self.qsl = np.concatenate([[0], np.cumsum(self.q_counts)]).astype(np.int32)
        T = int(self.qsl[-1])
        self.positions = np.concatenate(
            [np.arange(n, dtype=np.int32) if n > 0 else np.full(1, 12345, np.int32) for n in new])
        self.q = W._round_to(rng.standard_normal((T, H, dk)).astype(np.float32), dtype)
        self.scale = 1.0 / np.sqrt(dk)
        self.T = T

    def run(self, out, lse, merge, status=None):
        d = self.dtype
        pa_varlen_ctx_new(dev(self.k_pool, d), dev(self.v_pool, d), dev(self.q, d), out, lse, dev(self.qsl),
                          dev(np.array(self.ctx, np.int32)), dev(self.ctx_tables), dev(np.array(self.new, np.int32)),
                          dev(self.positions), dev(self.new_tables), max(self.q_counts), self.scale, merge=merge,
                          status=status)
        torch.cuda.synchronize()

    def expected(self, orc):
        """(out [T, H, dv], lse [H, T]) by the definition, float64."""
        out = np.zeros((self.T, self.H, self.dv))
        lse = np.zeros((self.H, self.T))
        q64 = orc.decode_elems(self.q, self.dtype)
        G = self.H // self.Hkv
        for r in range(len(self.ctx)):
            c, n = self.ctx[r], self.new[r]
            K = np.concatenate([orc.gather(self.k_pool, self.dtype, self.b, self.ctx_tables[r], c),
                                orc.gather(self.k_pool, self.dtype, self.b, self.new_tables[r], n)])
            V = np.concatenate([orc.gather(self.v_pool, self.dtype, self.b, self.ctx_tables[r], c),
                                orc.gather(self.v_pool, self.dtype, self.b, self.new_tables[r], n)])
            t0, t1 = int(self.qsl[r]), int(self.qsl[r + 1])
            hi = c + np.arange(1, n + 1) if n > 0 else np.array([c])
            for h in range(self.H):
                o, l = orc.attend_gathered(q64[t0:t1, h], K[:, h // G], V[:, h // G], np.zeros(t1 - t0, np.int64), hi,
                                           self.scale)
                out[t0:t1, h] = o
                lse[h, t0:t1] = l
        return out, lse


CASES = [
    # (dtype, H, Hkv, dk, dv, ctx, new)
    ("bf16", 8, 8, 192, 128, [0, 32, 1709, 100], [40, 130, 1, 77]),
    ("f16", 8, 2, 128, 128, [300, 0, 64, 17, 5], [129, 33, 0, 200, 1]),
    ("bf16", 4, 1, 64, 64, [47, 500], [300, 0]),
    ("f16", 32, 8, 128, 128, [1000, 2049], [64, 15]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_ctx_new_matches_definition(orc, case):
    dtype, H, Hkv, dk, dv, ctx, new = CASES[case]
    cs = CtxNewCase(900 + case, ctx, new, H, Hkv, dk, dv, dtype)
    out = torch.full((cs.T, H, dv), float("nan"), device="cuda")
    lse = torch.full((H, cs.T), float("nan"), device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    cs.run(out, lse, merge=False, status=st)
    assert int(st.item()) == 0
    ref, rlse = cs.expected(orc)
    assert_close(host(out), ref, TOL[dtype], "out")
    assert_close(host(lse), rlse, TOL[dtype], "lse")


@pytest.mark.parametrize("case", [0, 1])
def test_ctx_new_merged_into_a_state(orc, case):
    """merge=True folds the result into a prior state with MergeAttnStates' rules,
    including prior rows of lse +inf and -inf."""
    dtype, H, Hkv, dk, dv, ctx, new = CASES[case]
    cs = CtxNewCase(950 + case, ctx, new, H, Hkv, dk, dv, dtype)
    po, pl, _, _, special = W.merge_case(77 + case, cs.T, H, dv, special_fraction=0.1)
    out, lse = dev(po.copy()), dev(pl.copy())
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    cs.run(out, lse, merge=True, status=st)
    assert int(st.item()) == 0
    att, alse = cs.expected(orc)
    ref, rlse = orc.merge_states(po, pl, att.astype(np.float32), alse.astype(np.float32), "f32")
    assert_close(host(out), ref, TOL[dtype], "merged out")
    assert_close(host(lse), rlse, TOL[dtype], "merged lse")


def test_ctx_new_rejects_bad_content():
    """Device checks: a new position outside [0, new_len), a new-table id outside
    the pool; the output stays untouched.  A sequence without new tokens may hold
    any position (never read)."""
    cs = CtxNewCase(990, [100, 50], [20, 0], 4, 2, 128, 128, "f16")
    for what in ("position", "new id"):
        pos, tabs = cs.positions.copy(), cs.new_tables.copy()
        if what == "position":
            cs.positions[3] = 20
        else:
            cs.new_tables[0, 0] = cs.k_pool.shape[0]
        out = torch.full((cs.T, 4, 128), float("nan"), device="cuda")
        lse = torch.full((4, cs.T), float("nan"), device="cuda")
        st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        cs.run(out, lse, merge=False, status=st)
        assert int(st.item()) == 1, what
        assert np.all(np.isnan(host(out))) and np.all(np.isnan(host(lse))), what
        cs.positions, cs.new_tables = pos, tabs
