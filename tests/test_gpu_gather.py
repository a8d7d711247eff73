"""pa_gather_cache (the latent-cache gather of "cpu_mla_prefill.cpp",
GatherMlaCache) on the GPU against the CPU oracle, bit for bit: same-dtype copies
(16-byte path), conversions between f32 / f16 / bf16 (element path), windows given
by seq_starts, rows past a sequence's end left untouched, a strided output, and the
device check of the indices."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import PaError, pa_gather_cache
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu

STORE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def rand_storage(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32) * 4.0
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_dev(a, dtype):
    t = dev(a, dtype)
    return t if dtype != "bf16" else t.view(torch.bfloat16)


def same_bits(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.uint16 and b.dtype == np.uint16:
        an = ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
        bn = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    else:
        an, bn = np.isnan(a), np.isnan(b)
    ua = a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)
    ub = b.view(ua.dtype)
    return np.array_equal(an, bn) and np.array_equal(ua[~an], ub[~bn])


def build(rng, nseq, lens_range, b, D, dtype, spare=5):
    lens = rng.integers(*lens_range, size=nseq, endpoint=True)
    need = [(int(n) + b - 1) // b for n in lens]
    max_blocks = max(1, max(need))
    nb = sum(need) + spare
    ids = rng.permutation(nb)
    tables = np.full((nseq, max_blocks), ids[-1], np.int32)
    cur = 0
    for s, k in enumerate(need):
        tables[s, :k] = ids[cur:cur + k]
        cur += k
    cache = rand_storage(rng, (nb, b, D), dtype)
    return lens, tables, cache


CASES = [  # (cache dtype, dst dtype, head_dim, block_size)
    ("bf16", "bf16", 576, 16), ("f32", "f32", 64, 8), ("bf16", "f32", 576, 16), ("f32", "bf16", 96, 16),
    ("f16", "f16", 36, 4), ("f16", "bf16", 40, 16), ("bf16", "f16", 128, 32), ("f32", "f16", 24, 16),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_gather_bit_exact(orc, case):
    sd, dd, D, b = CASES[case]
    rng = np.random.default_rng(900 + case)
    lens, tables, cache = build(rng, 6, (1, 300), b, D, sd)
    # each sequence contributes a window [start, start + take) of its positions,
    # plus rows past the last sequence's end that must keep the sentinel
    starts = np.array([rng.integers(0, n) for n in lens], np.int32)
    take = np.array([rng.integers(1, n - st + 1) for n, st in zip(lens, starts)], np.int32)
    cu = np.concatenate([[0], np.cumsum(take)]).astype(np.int32)
    T = int(cu[-1]) + 3
    t2s = np.concatenate([np.repeat(np.arange(6), take), [5, 5, 5]]).astype(np.int32)
    sentinel = rand_storage(rng, (T, D), dd)
    st, ref = orc.gather_cache(cache, sd, tables, cu, t2s, starts, dd, T, dst=sentinel.copy())
    assert st == 0
    dst = to_dev(sentinel, dd)
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_gather_cache(to_dev(cache, sd), dst, dev(tables), dev(cu), dev(t2s), seq_starts=dev(starts), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert same_bits(host(dst), ref)


def test_gather_mla_chunks_into_strided_rows(orc):
    """Context chunks of 4096 positions of 8 requests (lengths up to 16384, latent
    rows of 576 bf16), each chunk gathered into the left part of wider rows."""
    rng = np.random.default_rng(950)
    lens, tables, cache = build(rng, 8, (0, 16384), 16, 576, "bf16")
    for c in range(int(lens.max() + 4095) // 4096):
        take = np.clip(lens - 4096 * c, 0, 4096).astype(np.int32)
        starts = np.full(8, 4096 * c, np.int32)
        cu = np.concatenate([[0], np.cumsum(take)]).astype(np.int32)
        T = int(cu[-1])
        if T == 0:
            continue
        t2s = np.repeat(np.arange(8), take).astype(np.int32)
        st, ref = orc.gather_cache(cache, "bf16", tables, cu, t2s, starts, "bf16", T)
        assert st == 0
        wide = torch.zeros((T, 640), dtype=torch.bfloat16, device="cuda")
        pa_gather_cache(to_dev(cache, "bf16"), wide[:, :576], dev(tables), dev(cu), dev(t2s), seq_starts=dev(starts))
        torch.cuda.synchronize()
        got = host(wide)
        assert same_bits(got[:, :576], ref) and np.all(got[:, 576:] == 0)


def test_gather_refuses_bad_indices_before_writing():
    rng = np.random.default_rng(960)
    lens, tables, cache = build(rng, 3, (20, 40), 16, 64, "f16")
    cu = np.array([0, 5, 10, 15], np.int32)
    t2s = np.repeat(np.arange(3), 5).astype(np.int32)
    bad = t2s.copy()
    bad[7] = 3  # no such sequence
    dst = torch.full((15, 64), 3.0, dtype=torch.float16, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_gather_cache(to_dev(cache, "f16"), dst, dev(tables), dev(cu), dev(bad), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1 and bool((dst == 3.0).all())
    with pytest.raises(ValueError):
        pa_gather_cache(to_dev(cache, "f16"), dst[:, :60], dev(tables), dev(cu), dev(t2s))
    with pytest.raises(PaError):  # output rows that overlap
        pa_gather_cache(to_dev(cache, "f16"), torch.empty(15, 64, dtype=torch.float16, device="cuda")
                        .as_strided((15, 64), (32, 1)), dev(tables), dev(cu), dev(t2s))
