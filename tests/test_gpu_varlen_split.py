"""pa_varlen with split single-token rows (partition_size > 0) on the GPU against the
CPU oracle's unsplit varlen: the tiled prefill kernel plus split single-token rows
(16-bit and fp8 caches), the per-row kernel for every other token plus split
single-token rows (a shape the tiled kernel does not take), single-token calls only
(16-bit and fp8 caches), causal and not, windows, sinks and ALiBi, and the device
check of the partition count.  Outputs and lse of every token are compared."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_varlen
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, OnDevice, assert_close, host, threads, workload

pytestmark = pytest.mark.gpu


def run(orc, w, P, causal=None, window=None, sinks=None, alibi=None, pmax=None, expect_status=0):
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    causal = w.causal if causal is None else causal
    window = w.sliding_window if window is None else window
    T, H, S = w.num_tokens, w.num_heads, w.num_seqs
    out = torch.full((T, H, w.dv), float("nan"), device="cuda")
    lse = torch.full((H, T), float("nan"), device="cuda")
    pmax = pmax or max(1, -(-int(w.seq_lens.max()) // P))
    ws = tuple(torch.full(sh, float("nan"), device="cuda") for sh in ((S, H, pmax), (S, H, pmax), (S, H, pmax, w.dv)))
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    max_q = int(np.diff(w.query_start_loc).max())
    tens = lambda a: None if a is None else torch.from_numpy(np.asarray(a, np.float32)).cuda()  # noqa: E731
    pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions if causal else None, d.tables, max_q,
              w.scale, causal=causal, sliding_window=window, lse=lse, status=status, sinks=tens(sinks),
              alibi_slopes=tens(alibi), k_scale=w.k_scale, v_scale=w.v_scale, partition_size=P, max_logits=ws[0],
              exp_sums=ws[1], tmp_out=ws[2])
    torch.cuda.synchronize()
    assert int(status.item()) == expect_status
    if expect_status:
        assert torch.isnan(out).all(), "a refused call wrote its output"
        return
    f64 = lambda a: None if a is None else np.asarray(a, np.float64)  # noqa: E731
    st, ref, rlse = orc.varlen(kp, vp, w.dtype, w.q, w.query_dtype, w.query_start_loc, w.seq_lens,
                               w.positions if causal else None, w.block_tables, w.scale, causal, window,
                               threads=threads(), sinks=f64(sinks), alibi_slopes=f64(alibi), k_scale=w.k_scale,
                               v_scale=w.v_scale)
    assert st == 0
    assert_close(host(out), ref, TOL[w.dtype], f"{w.name} P={P} out")
    assert_close(host(lse), rlse, TOL[w.dtype], f"{w.name} P={P} lse")


@pytest.mark.parametrize("name,P", [("mixed-varlen-small", 16), ("mixed-varlen-small", 128), ("mixed-varlen-shuffled", 64),
                                    ("mixed-varlen", 256)])
def test_split_singles_beside_prefill_tiles(orc, name, P):
    run(orc, workload(name), P)


@pytest.mark.parametrize("name,P", [("mixed-varlen-small", 64), ("mixed-varlen", 256)])
def test_split_singles_beside_fp8_prefill_tiles(orc, name, P):
    """fp8 cache: the tiled kernel's launch, then the split rows on the fp8 decode
    kernel and the reduce."""
    run(orc, W.to_fp8(workload(name), k_scale=0.0703125, v_scale=0.04296875), P)


@pytest.mark.parametrize("causal,window", [(False, 0), (False, 100), (True, 0)])
def test_split_singles_masks(orc, causal, window):
    run(orc, workload("mixed-varlen-small"), 32, causal=causal, window=window)


def test_split_singles_with_sinks_and_alibi(orc):
    w = workload("mixed-varlen-small")
    rng = np.random.default_rng(71)
    z = rng.standard_normal(w.num_heads) * 3
    z[::5] = -np.inf
    slopes = np.array([2.0 ** (-8.0 * (h + 1) / w.num_heads) for h in range(w.num_heads)])
    run(orc, w, 64, sinks=z, alibi=slopes)


def test_split_singles_beside_row_kernel(orc):
    """Block size 8: the tiled kernel does not take it, so multi-token sequences go
    through the per-row kernel (which then leaves the single-token ones out)."""
    w = W.make_paged("split-rows-path", 2400, dtype="bf16", block_size=8, num_heads=8, num_kv_heads=4, dk=64, dv=64,
                     segments=[(30, 20), (700, 1), (0, 1), (90, 7), (1500, 1), (12, 0)], causal=True,
                     sliding_window=400)
    run(orc, w, 64)


def test_split_single_token_calls(orc):
    """Every sequence holds at most one token (16-bit and fp8 caches)."""
    segments = [(40, 1), (700, 1), (0, 1), (129, 0), (3000, 1), (15, 1)]
    base = W.make_paged("split-singles-only", 2500, dtype="bf16", block_size=16, num_heads=32, num_kv_heads=8,
                        dk=128, dv=128, segments=segments, causal=True, sliding_window=0)
    run(orc, base, 128)
    run(orc, W.to_fp8(base), 256)


def test_split_partition_count_checked(orc):
    """A workspace with too few partitions for a single-token sequence is refused on
    the device, and nothing is written."""
    w = workload("mixed-varlen-small")
    run(orc, w, 16, pmax=2, expect_status=1)
