"""pa_decode across the supported shape space on the GPU against the CPU oracle: head
dims 32 / 64 / 128 / 256, 1 to 16 q heads per kv head, block sizes 8 to 128,
f32 / f16 / bf16 caches, unsplit and split, with and without a sliding window, and
lengths on either side of block and tile boundaries (1, b - 1, b, b + 1, ...).  The
MFMA decode kernel takes head dim 128 with power-of-two blocks of at least 16 in
f16 / bf16; the per-row kernel takes the rest."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_decode
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, OnDevice, assert_close, host, threads

pytestmark = pytest.mark.gpu

# dtype, H, Hkv, D, block, lengths, window, partition size
SHAPES = [
    ("f16", 32, 2, 128, 32, [1, 16, 17, 31, 32, 33, 700, 1500], 0, 0),
    ("f16", 32, 2, 128, 32, [1, 16, 17, 31, 32, 33, 700, 1500], 0, 64),
    ("bf16", 8, 8, 128, 128, [1, 127, 128, 129, 900, 2000], 0, 256),
    ("bf16", 8, 8, 128, 128, [1, 127, 128, 129, 900, 2000], 300, 0),
    ("f16", 16, 1, 128, 16, [2000, 4000, 15], 0, 0),
    ("f16", 16, 1, 128, 64, [2000, 4000, 15], 129, 128),
    ("f32", 8, 4, 256, 16, [5, 300, 1000], 0, 0),
    ("f32", 8, 4, 256, 16, [5, 300, 1000], 50, 128),
    ("bf16", 16, 2, 256, 32, [33, 1000], 0, 64),
    ("f16", 16, 4, 32, 8, [3, 8, 9, 400], 0, 0),
    ("f16", 16, 4, 32, 8, [3, 8, 9, 400], 0, 16),
    ("bf16", 64, 8, 64, 64, [64, 65, 640, 3000], 0, 0),
    ("bf16", 64, 8, 64, 64, [64, 65, 640, 3000], 1000, 512),
    ("f32", 48, 3, 64, 16, [1, 2, 47, 1024], 7, 0),
]


@pytest.mark.parametrize("case", range(len(SHAPES)),
                         ids=[f"{s[0]}-H{s[1]}-Hkv{s[2]}-D{s[3]}-b{s[4]}-w{s[6]}-P{s[7]}" for s in SHAPES])
def test_decode_shapes(orc, case):
    dtype, H, Hkv, D, b, lens, window, P = SHAPES[case]
    w = W.make_decode(f"decode-shape{case}", 900 + case, seq_lens=lens, dtype=dtype, num_heads=H, num_kv_heads=Hkv,
                      head_dim=D, block_size=b, sliding_window=window)
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    S = w.num_seqs
    out = torch.full((S, H, D), float("nan"), device="cuda")
    ws = (None, None, None)
    if P:
        pm = -(-max(lens) // P)
        ws = tuple(torch.full(sh, float("nan"), device="cuda") for sh in ((S, H, pm), (S, H, pm), (S, H, pm, D)))
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale, sliding_window=window, partition_size=P,
              max_logits=ws[0], exp_sums=ws[1], tmp_out=ws[2], status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    st, ref, _ = orc.decode(kp, vp, w.dtype, w.q, w.dtype, w.block_tables, w.seq_lens, w.scale,
                            sliding_window=window, threads=threads())
    assert st == 0
    assert_close(host(out), ref, TOL[dtype], f"case {case}")
    if P:
        st, rml, _, rto = orc.decode(kp, vp, w.dtype, w.q, w.dtype, w.block_tables, w.seq_lens, w.scale,
                                     sliding_window=window, partition_size=P, max_partitions=ws[0].shape[-1],
                                     threads=threads())
        assert st == 0
        used = np.zeros(ws[0].shape, dtype=bool)
        for s, n in enumerate(lens):
            used[s, :, :-(-int(n) // P)] = True
        assert_close(host(ws[0]), rml, TOL[dtype], "max_logits", mask=used)
        assert_close(host(ws[2]), rto, TOL[dtype], "tmp_out", mask=used)
