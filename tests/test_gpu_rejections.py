"""Device-resident content errors ("Paged attention for decode in C", section 2.6 and
its bad-tables test): with a status word the call stores PA_EINVAL and writes no
output.  Every case is forced from the host through the inputs; all kernels still
run to completion (they test the status word and return)."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_decode, pa_varlen
from tests.gpu_util import OnDevice, host, workload

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def decode_status(d, tables=None, lens=None, P=0, pmax=None):
    w = d.w
    out = torch.full((w.num_seqs, w.num_heads, w.dv), SENTINEL, device="cuda")
    ws = (None, None, None)
    if P:
        ws = tuple(torch.full(sh, SENTINEL, device="cuda") for sh in
                   ((w.num_seqs, w.num_heads, pmax), (w.num_seqs, w.num_heads, pmax),
                    (w.num_seqs, w.num_heads, pmax, w.dv)))
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables if tables is None else tables,
              d.seq_lens if lens is None else lens, w.scale, partition_size=P, max_logits=ws[0], exp_sums=ws[1],
              tmp_out=ws[2], status=st)
    torch.cuda.synchronize()
    untouched = bool(torch.all(out == SENTINEL)) and all(bool(torch.all(x == SENTINEL)) for x in ws if x is not None)
    return int(st.item()), untouched


def test_decode_rejections():
    d = OnDevice(workload("batched-decode-small"))
    w = d.w
    assert decode_status(d)[0] == 0
    cases = []
    lens = d.seq_lens.clone(); lens[2] = 0; cases.append(("empty context", None, lens))
    lens = d.seq_lens.clone(); lens[0] = w.max_blocks * w.block_size + 1; cases.append(("table too short", None, lens))
    t = d.tables.clone(); t[1, 0] = w.num_blocks; cases.append(("id past the pool", t, None))
    t = d.tables.clone(); t[3, 1] = -1; cases.append(("negative id", t, None))
    for what, tables, lens in cases:
        st, untouched = decode_status(d, tables, lens)
        assert st == 1 and untouched, what
    # max_partitions too small for the longest sequence
    pm = -(-int(w.seq_lens.max()) // 64) - 1
    st, untouched = decode_status(d, P=64, pmax=pm)
    assert st == 1 and untouched


def varlen_status(d, qsl=None, pos=None, lens=None, max_q=None):
    w = d.w
    out = torch.full((w.num_tokens, w.num_heads, w.dv), SENTINEL, device="cuda")
    lse = torch.full((w.num_heads, w.num_tokens), SENTINEL, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    max_q = int(np.diff(w.query_start_loc).max()) if max_q is None else max_q
    pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl if qsl is None else qsl, d.seq_lens if lens is None else lens,
              d.positions if pos is None else pos, d.tables, max_q, w.scale, causal=True,
              sliding_window=w.sliding_window, lse=lse, status=st)
    torch.cuda.synchronize()
    return int(st.item()), bool(torch.all(out == SENTINEL)) and bool(torch.all(lse == SENTINEL))


def test_varlen_rejections():
    d = OnDevice(workload("mixed-varlen-small"))
    w = d.w
    assert varlen_status(d)[0] == 0
    p = d.positions.clone(); p[5] = int(w.seq_lens[0]); assert varlen_status(d, pos=p) == (1, True)
    p = d.positions.clone(); p[0] = -3; assert varlen_status(d, pos=p) == (1, True)
    q = d.qsl.clone(); q[2] = q[1] - 1; assert varlen_status(d, qsl=q) == (1, True)
    q = d.qsl.clone(); q[-1] = q[-1] - 1; assert varlen_status(d, qsl=q) == (1, True)
    q = d.qsl.clone(); q[0] = 1; assert varlen_status(d, qsl=q) == (1, True)
    l = d.seq_lens.clone(); l[1] = -1; assert varlen_status(d, lens=l) == (1, True)
    assert varlen_status(d, max_q=int(np.diff(w.query_start_loc).max()) - 1) == (1, True)
