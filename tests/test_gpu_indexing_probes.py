"""Bit-exact table / slot indexing through the hot-path kernels ("Paged attention for
decode in C", section 2.1 and the section 3 worked example: position j of a
sequence lives at slot j mod b of block table[j / b]).

Every V row holds an encoding of where it lives: dims 0-3 the base-16 digits of its
slot id (block * b + offset), dim 4 its kv head, the other dims (d mod 8) / 8.  All
of these are exact in f16, bf16 and fp8 E4M3, and the digits tell every row of the
pool apart.  With a window of one position each query sees exactly one key, so
every output row is that key's V row: the (slot, kv head) read back from the
rounded digits must equal the one the table names, exactly, for every row and head,
and the values must agree to a few binary32 ulps (the kernels normalise by a
reciprocal of the softmax sum, which may leave the last bit or two).  Covered: the
MFMA decode kernel (unsplit, multi-wave split, one-wave split; 16-bit and fp8
caches, the latter also on kv-head pairs), the tiled prefill kernel (several query
tokens per sequence, causal, head dims 128, 192 / 128 and 64; 16-bit and fp8 caches)
and the single-token rows of a mixed varlen call.  K is random and unused blocks hold NaN, so a wrong
slot shows as a wrong index or a NaN."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_decode, pa_varlen
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def encoded_values(nb, b, hkv, dv):
    slot = np.arange(nb * b, dtype=np.int64).reshape(nb, b, 1, 1)
    v = np.broadcast_to((np.arange(dv) % 8 / 8.0).reshape(1, 1, 1, dv), (nb, b, hkv, dv)).copy()
    for k in range(4):
        v[..., k] = np.broadcast_to((slot[..., 0] >> (4 * k)) & 15, (nb, b, hkv))
    v[..., 4] = np.arange(hkv).reshape(1, 1, hkv)
    return v.astype(np.float32)


def decode_index(row):
    """(slot, kv head) from an output row."""
    digits = np.rint(row[:4]).astype(np.int64)
    return int(sum(int(x) << (4 * k) for k, x in enumerate(digits))), int(np.rint(row[4]))


def to_storage(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return {"f16": t.half(), "bf16": t.bfloat16(), "fp8": t.to(torch.float8_e4m3fn)}[dtype].cuda()


def make_pools(rng, nb, b, hkv, dk, dv, dtype, used_blocks):
    k = rng.standard_normal((nb, b, hkv, dk)).astype(np.float32)
    v = encoded_values(nb, b, hkv, dv)
    unused = np.setdiff1d(np.arange(nb), used_blocks)
    k[unused] = np.nan
    v[unused] = np.nan
    return to_storage(k, dtype), to_storage(v, dtype), v


def check_rows(got, v, tables, b, pos_of_row, seq_of_row, G):
    """got [rows, H, dv] float32; every (row, head) equals the V row of its slot."""
    rows, H, dv = got.shape
    flat = v.reshape(-1, v.shape[2], dv)
    for r in range(rows):
        s, j = seq_of_row[r], pos_of_row[r]
        slot = int(tables[s, j // b]) * b + j % b
        for h in range(H):
            g = h // G
            assert decode_index(got[r, h]) == (slot, g), (r, h, slot, g, got[r, h, :5])
            err = np.abs(got[r, h] - flat[slot, g])
            assert np.all(err <= 2.0 ** -21 * np.maximum(1.0, np.abs(flat[slot, g]))), (r, h, err.max())


@pytest.mark.parametrize("dtype,P,pmax", [("f16", 0, None), ("bf16", 0, None), ("f16", 64, None),
                                          ("bf16", 16, 1024), ("fp8", 0, None), ("fp8", 128, None),
                                          ("fp8", 16, 1024)])
def test_decode_index_probe(dtype, P, pmax):
    rng = np.random.default_rng(91)
    b, hkv, D, H = 16, 8, 128, 32
    lens = rng.integers(1, 1500, size=21)
    lens[:3] = [1, 16, 17]
    need = -(-lens // b)
    nb = int(need.sum()) + 9  # slot ids stay below 16^4
    assert nb * b < 16 ** 4
    perm = rng.permutation(nb)
    tables = np.full((lens.size, int(need.max())), perm[-1], dtype=np.int32)
    cur = 0
    for s, k in enumerate(need):
        tables[s, :k] = perm[cur:cur + k]
        cur += k
    assert cur < nb
    kp, vp, v = make_pools(rng, nb, b, hkv, D, D, dtype, perm[:cur])
    qd = torch.float16 if dtype in ("f16", "fp8") else torch.bfloat16
    q = torch.from_numpy(rng.standard_normal((lens.size, H, D)).astype(np.float32)).to(qd).cuda()
    out = torch.full((lens.size, H, D), float("nan"), device="cuda")
    ws = (None, None, None)
    if P:
        pm = pmax or -(-int(lens.max()) // P)
        ws = tuple(torch.full(sh, float("nan"), device="cuda") for sh in ((lens.size, H, pm), (lens.size, H, pm),
                                                                        (lens.size, H, pm, D)))
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode(kp, vp, q, out, dev(tables), dev(lens.astype(np.int32)), 0.088, sliding_window=1, partition_size=P,
              max_logits=ws[0], exp_sums=ws[1], tmp_out=ws[2], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    check_rows(host(out), v, tables, b, lens - 1, np.arange(lens.size), H // hkv)


@pytest.mark.parametrize("dtype,H,hkv,dk,dv", [("f16", 32, 8, 128, 128), ("bf16", 32, 8, 128, 128),
                                               ("bf16", 16, 16, 192, 128), ("f16", 8, 2, 64, 64),
                                               ("fp8", 32, 8, 128, 128), ("fp8", 16, 16, 192, 128)])
def test_varlen_index_probe(dtype, H, hkv, dk, dv):
    """Prefill chunks (tiled kernel) and single tokens (decode kernel, or the tiled
    kernel where the decode kernel does not take the shape) in one call; fp8 caches
    with bf16 queries."""
    rng = np.random.default_rng(92)
    b = 16
    segments = [(0, 70), (333, 1), (45, 130), (1000, 1), (17, 33), (0, 1), (260, 64)]
    lens = np.array([c + n for c, n in segments])
    need = -(-lens // b)
    nb = int(need.sum()) + 5
    perm = rng.permutation(nb)
    tables = np.full((lens.size, int(need.max())), perm[-1], dtype=np.int32)
    cur = 0
    for s, k in enumerate(need):
        tables[s, :k] = perm[cur:cur + k]
        cur += k
    kp, vp, v = make_pools(rng, nb, b, hkv, dk, dv, dtype, perm[:cur])
    qsl = np.concatenate([[0], np.cumsum([n for _, n in segments])]).astype(np.int32)
    positions = np.concatenate([np.arange(c, c + n) for c, n in segments]).astype(np.int32)
    seq_of = np.concatenate([np.full(n, s) for s, (_, n) in enumerate(segments)])
    T = int(qsl[-1])
    qd = torch.float16 if dtype == "f16" else torch.bfloat16
    q = torch.from_numpy(rng.standard_normal((T, H, dk)).astype(np.float32)).to(qd).cuda()
    out = torch.full((T, H, dv), float("nan"), device="cuda")
    lse = torch.full((H, T), float("nan"), device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_varlen(kp, vp, q, out, dev(qsl), dev(lens.astype(np.int32)), dev(positions), dev(tables),
              int(np.diff(qsl).max()), 1.0 / np.sqrt(dk), causal=True, sliding_window=1, lse=lse, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    check_rows(host(out), v, tables, b, positions, seq_of, H // hkv)
