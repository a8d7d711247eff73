"""pa_decode_noalloc (split-KV decode whose partition states live in the library's
static device buffer) against pa_decode with caller workspaces, through the C ABI.

Two calls in a row share the buffer: the long-context split decode at full size
(8 sequences up to 131072 positions, 64 q heads, P = 512; its states take 65 MiB
of the 96), then a smaller batch with other partition sizes, whose states overwrite
part of the first call's.  Each output must equal pa_decode's bit for bit (the same
kernels on the same states), and the smaller one also the oracle within the bound."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import PaError, binding, pa_decode, pa_decode_noalloc
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, OnDevice, assert_close, bits_equal, host, threads, workload

pytestmark = pytest.mark.gpu


def with_workspaces(d, P, sliding_window=0, sinks=None):
    w = d.w
    S, H = w.num_seqs, w.num_heads
    pmax = -(-(d.tables.shape[1] * w.block_size) // P)
    ws = [torch.full(sh, float("nan"), device="cuda") for sh in ((S, H, pmax), (S, H, pmax), (S, H, pmax, w.dv))]
    out = torch.full((S, H, w.dv), float("nan"), device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale, sliding_window=sliding_window,
              partition_size=P, max_logits=ws[0], exp_sums=ws[1], tmp_out=ws[2], status=st, sinks=sinks,
              k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return host(out)


def static(d, P, sliding_window=0, sinks=None):
    w = d.w
    out = torch.full((w.num_seqs, w.num_heads, w.dv), float("nan"), device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode_noalloc(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale, sliding_window=sliding_window,
                      partition_size=P, status=st, sinks=sinks, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return host(out)


def test_noalloc_matches_pa_decode_on_two_calls(orc):
    big = OnDevice(workload("long-decode"))
    got = static(big, 512)
    assert bits_equal(got, with_workspaces(big, 512)), "long split decode, P 512"

    small = OnDevice(workload("batched-decode-small"))
    sinks = torch.linspace(-1.0, 2.0, small.w.num_heads, device="cuda")
    for P, win in ((64, 0), (32, 100)):
        got = static(small, P, sliding_window=win, sinks=sinks)
        assert bits_equal(got, with_workspaces(small, P, sliding_window=win, sinks=sinks)), f"P {P} window {win}"
        w = small.w
        kp, vp = small.host_pools_after_write(orc)
        st, ref, _ = orc.decode(kp, vp, w.dtype, w.q, w.dtype, w.block_tables, w.seq_lens, w.scale,
                                sliding_window=win, sinks=host(sinks).astype(np.float64), threads=threads())
        assert st == 0
        assert_close(got, ref, TOL[w.dtype], f"P {P} window {win} vs oracle")


def test_noalloc_fp8_two_calls():
    """fp8 caches: the long split decode (kv-head pairs) at full size, then a smaller
    batch, both bit for bit as pa_decode with caller workspaces."""
    big = OnDevice(W.to_fp8(workload("long-decode")))
    assert bits_equal(static(big, 512), with_workspaces(big, 512)), "fp8 long split decode, P 512"
    small = OnDevice(W.to_fp8(workload("batched-decode-small"), k_scale=0.0703125, v_scale=0.04296875))
    assert bits_equal(static(small, 64, sliding_window=100), with_workspaces(small, 64, sliding_window=100)), \
        "fp8 batch, P 64, window 100"


def test_noalloc_refuses_what_does_not_fit():
    d = OnDevice(workload("batched-decode-small"))
    w = d.w
    out = torch.full((w.num_seqs, w.num_heads, w.dv), float("nan"), device="cuda")
    wide = torch.zeros((w.num_seqs, 8192 * 64 // w.block_size), dtype=torch.int32, device="cuda")
    with pytest.raises(PaError) as e:
        pa_decode_noalloc(d.k_pool, d.v_pool, d.q, out, wide, d.seq_lens, w.scale, partition_size=64)
    assert e.value.status == binding.PA_ESCRATCH
    torch.cuda.synchronize()
    assert np.all(np.isnan(host(out))), "a refused call wrote its output"
