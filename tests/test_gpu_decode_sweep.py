"""A seeded sweep of pa_decode on the GPU against the CPU oracle: each case draws one
combination of the decode options and checks every output row.

Drawn per case: the pool type (f32, f16, bf16, or fp8 E4M3 with f16 / bf16 queries and
random per-tensor scales), the head dim the kernels take for it (32 / 64 / 128 / 256;
fp8: 128), the kv head count and head-group size (1 to 16 q heads per kv head), the
block size (8 to 128, 48 included; fp8 and the MFMA kernel: powers of two of at
least 16), 1 to 12 sequences of 1..3000 positions with block and tile boundaries
over-represented, a sliding window or none, unsplit or split with a drawn partition
size (the split states compared too), attention sinks and ALiBi slopes."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_decode
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, OnDevice, assert_close, host, threads

pytestmark = pytest.mark.gpu

NCASES = 96


def draw(seed):
    rng = np.random.default_rng(50_000 + seed)
    kind = ["f32", "f16", "bf16", "fp8"][seed % 4]
    D = 128 if kind == "fp8" else int(rng.choice([32, 64, 128, 128, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    if D == 256 and G > 8:
        G = 8  # the row kernel's limit at head dim 256
    b = int(rng.choice([16, 32, 64, 128])) if kind == "fp8" else int(rng.choice([8, 16, 32, 48, 64, 128]))
    S = int(rng.integers(1, 13))
    lens = []
    for _ in range(S):
        r = rng.random()
        if r < 0.35:
            lens.append(int(max(1, b * int(rng.integers(1, 20)) + int(rng.choice([-1, 0, 1])))))
        else:
            lens.append(int(rng.integers(1, 3000)))
    window = int(rng.choice([0, 0, 1, 17, 300]))
    P = int(rng.choice([0, 0, b * int(rng.integers(1, 9)), 512]))
    if P and P % b:
        P = b * (P // b + 1)
    return dict(kind=kind, D=D, hkv=hkv, G=G, b=b, lens=lens, window=window, P=P, sinks=bool(rng.integers(2)),
                alibi=bool(rng.integers(3) == 0), qd=str(rng.choice(["f16", "bf16"])),
                ks=float(rng.choice([0.0625, 0.0703125, 0.125])), vs=float(rng.choice([0.03125, 0.04296875, 0.25])))


@pytest.mark.parametrize("seed", range(NCASES))
def test_decode_sweep(orc, seed):
    c = draw(seed)
    base = c["qd"] if c["kind"] == "fp8" else c["kind"]
    H, D, P = c["hkv"] * c["G"], c["D"], c["P"]
    w = W.make_decode(f"decode-sweep{seed}", 51_000 + seed, seq_lens=c["lens"], dtype=base, num_heads=H,
                      num_kv_heads=c["hkv"], head_dim=D, block_size=c["b"], sliding_window=c["window"])
    if c["kind"] == "fp8":
        w = W.to_fp8(w, k_scale=c["ks"], v_scale=c["vs"])
    d = OnDevice(w)
    kp, vp = d.host_pools_after_write(orc)
    S = w.num_seqs
    rng = np.random.default_rng(52_000 + seed)
    sinks = rng.standard_normal(H) * 2 if c["sinks"] else None
    alibi = np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], np.float32) if c["alibi"] else None
    tens = lambda a: None if a is None else torch.from_numpy(np.asarray(a, np.float32)).cuda()  # noqa: E731
    f64 = lambda a: None if a is None else np.asarray(a, np.float64)  # noqa: E731
    out = torch.full((S, H, D), float("nan"), device="cuda")
    ws = (None, None, None)
    pm = 0
    if P:
        pm = -(-max(c["lens"]) // P)
        ws = tuple(torch.full(sh, float("nan"), device="cuda") for sh in ((S, H, pm), (S, H, pm), (S, H, pm, D)))
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale, sliding_window=c["window"],
              partition_size=P, max_logits=ws[0], exp_sums=ws[1], tmp_out=ws[2], status=status, sinks=tens(sinks),
              alibi_slopes=tens(alibi), k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, c
    kw = dict(sliding_window=c["window"], threads=threads(), sinks=f64(sinks), alibi_slopes=f64(alibi),
              k_scale=w.k_scale, v_scale=w.v_scale)
    st, ref, _ = orc.decode(kp, vp, w.dtype, w.q, w.query_dtype, w.block_tables, w.seq_lens, w.scale, **kw)
    assert st == 0
    tol = TOL[w.dtype]
    assert_close(host(out), ref, tol, f"case {c}")
    if P:
        st, rml, res, rto = orc.decode(kp, vp, w.dtype, w.q, w.query_dtype, w.block_tables, w.seq_lens, w.scale,
                                     partition_size=P, max_partitions=pm, **kw)
        assert st == 0
        used = np.zeros((S, H, pm), dtype=bool)
        for s, n in enumerate(c["lens"]):
            used[s, :, :-(-int(n) // P)] = True
        ml, es = host(ws[0]), host(ws[1])
        # with ALiBi a partition far before the query has a maximum near -slope * distance
        # (about -1000 here), where fp32 rounds the bias product to ~6e-5: allow 4 ulps of it
        g, r = ml[used], rml[used]
        ninf = np.isneginf(r)  # partitions wholly outside the window
        assert np.array_equal(np.isneginf(g), ninf), c
        err = np.abs(g[~ninf] - r[~ninf])
        assert np.all(err <= tol + 2.0 ** -21 * np.abs(r[~ninf])), (c, err.max())
        rel = np.abs(es[used] - res[used]) / np.maximum(res[used], 1e-30)
        assert np.all((res[used] == 0) == (es[used] == 0)) and rel.max() <= tol, (c, rel.max())
        assert_close(host(ws[2]), rto, tol, f"case {c} tmp_out", mask=used)
