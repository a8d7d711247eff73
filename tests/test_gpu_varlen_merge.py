"""pa_varlen_merge (varlen attention merged into an existing state) on the GPU against
the CPU oracle's varlen followed by its merge ("cpu_mla_prefill.cpp":
MlaPrefillAttention, then MergeAttnStates with this call as the suffix).  The prior
state has rows whose lse is +inf or -inf, and some rows of the call see nothing, so
every edge rule of the merge is exercised on each kernel that can carry it: the
tiled prefill kernel, the per-row kernel, and the MFMA decode kernel's single-token
rows (16-bit and fp8 caches)."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_varlen_merge
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, OnDevice, assert_close, host, threads, workload

pytestmark = pytest.mark.gpu


def prior_state(seed, T, H, D):
    """A seeded state: N(0, 1) outputs; lse N(0, 3), 8 % of rows +inf and 8 % -inf."""
    rng = np.random.default_rng(seed)
    out = rng.standard_normal((T, H, D)).astype(np.float32)
    lse = (rng.standard_normal((H, T)) * 3).astype(np.float32)
    u = rng.random((H, T))
    lse[u < 0.08] = np.inf
    lse[(u >= 0.08) & (u < 0.16)] = -np.inf
    return out, lse


def check(orc, w, causal=True, window=None, sinks=None, alibi=None, seed=91):
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    window = w.sliding_window if window is None else window
    T, H = w.num_tokens, w.num_heads
    po, pl = prior_state(seed, T, H, w.dv)
    out = torch.from_numpy(po.copy()).cuda()
    lse = torch.from_numpy(pl.copy()).cuda()
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    tens = lambda a: None if a is None else torch.from_numpy(np.asarray(a, np.float32)).cuda()  # noqa: E731
    max_q = int(np.diff(w.query_start_loc).max())
    pa_varlen_merge(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions if causal else None, d.tables, max_q,
                    w.scale, causal=causal, sliding_window=window, lse=lse, status=status, sinks=tens(sinks),
                    alibi_slopes=tens(alibi), k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    f64 = lambda a: None if a is None else np.asarray(a, np.float64)  # noqa: E731
    st, so, sl = orc.varlen(kp, vp, w.dtype, w.q, w.query_dtype, w.query_start_loc, w.seq_lens,
                            w.positions if causal else None, w.block_tables, w.scale, causal, window, threads=threads(),
                            sinks=f64(sinks), alibi_slopes=f64(alibi), k_scale=w.k_scale, v_scale=w.v_scale)
    assert st == 0
    ref, rlse = orc.merge_states(po, pl, so.astype(np.float32), sl.astype(np.float32), "f32")
    assert_close(host(out), ref, TOL[w.dtype], f"{w.name} out")
    assert_close(host(lse), rlse, TOL[w.dtype], f"{w.name} lse")


@pytest.mark.parametrize("name,causal,window", [("mixed-varlen-small", True, None), ("mixed-varlen-small", False, 0),
                                                ("mixed-varlen-small", True, 7), ("mixed-varlen-shuffled", True, None)])
def test_merge_tiles_and_single_rows(orc, name, causal, window):
    check(orc, workload(name), causal=causal, window=window)


def test_merge_with_sinks_and_alibi(orc):
    w = workload("mixed-varlen-small")
    rng = np.random.default_rng(93)
    z = rng.standard_normal(w.num_heads) * 2
    z[::3] = -np.inf
    slopes = np.array([2.0 ** (-8.0 * (h + 1) / w.num_heads) for h in range(w.num_heads)])
    check(orc, w, sinks=z, alibi=slopes)


def test_merge_row_kernel_and_empty_rows(orc):
    """Block size 8 (every token on the per-row kernel), and a sequence with no
    context read non-causally: its rows see nothing, so the prior state passes
    through (or becomes -inf where it was +inf / -inf)."""
    w = W.make_paged("merge-rows-path", 2600, dtype="bf16", block_size=8, num_heads=8, num_kv_heads=4, dk=64, dv=64,
                     segments=[(30, 20), (700, 1), (0, 3), (90, 7)], causal=True, sliding_window=0)
    w.seq_lens[2] = 0  # nothing cached for sequence 2 (read non-causally below)
    check(orc, w, causal=False)


def test_merge_single_token_rows_fp8(orc):
    segments = [(40, 1), (700, 1), (0, 1), (129, 0), (3000, 1)]
    base = W.make_paged("merge-singles", 2700, dtype="bf16", block_size=16, num_heads=32, num_kv_heads=8, dk=128,
                        dv=128, segments=segments, causal=True, sliding_window=0)
    check(orc, base)
    check(orc, W.to_fp8(base))
