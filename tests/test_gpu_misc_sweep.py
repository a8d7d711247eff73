"""Seeded sweeps of the three smaller entry points on the GPU against the CPU oracle.

pa_write_kv: pool type (f32, f16, bf16, fp8 E4M3), kv heads, head dims (equal and
192 / 128), block sizes 1 to 64 (not only powers of two), 1 to 400 tokens into
distinct random slots; the new rows hold random bit patterns (NaN payloads
included), and both pools must equal the oracle's byte for byte.

pa_merge_states: element type (f32, f16, bf16), 1 to 300 tokens, 1 to 32 heads,
head dims 1 to 256 (odd ones take the element path), a seeded share of rows with
+inf / -inf lse on either side, with and without a prefill_tokens_with_context
limit: edge and pass-through rows must be exact copies, blended rows within
rounding of the oracle (1e-5 for f32; for 16-bit types one ulp, plus the fp32
blend's error where its two terms nearly cancel).

pa_gather_cache: cache and destination types (f32, f16, bf16 each way), head dims
1 to 600, block sizes 1 to 64, windows given by seq_starts or not, rows past the
last sequence that must keep their contents, destination rows strided or not:
bit for bit."""
import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_gather_cache, pa_merge_states, pa_write_kv
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import assert_close, dev, host
from tests.test_gpu_gather import build, rand_storage, same_bits, to_dev

pytestmark = pytest.mark.gpu

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8_e4m3": np.uint8}
BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8_e4m3": np.uint8}

NWRITE = 32


def random_bits(rng, shape, dtype):
    """Random bit patterns of the storage type (NaN and inf encodings included)."""
    ut = BITS[dtype]
    return rng.integers(0, np.iinfo(ut).max, size=shape, dtype=ut, endpoint=True).view(STORAGE[dtype])


@pytest.mark.parametrize("seed", range(NWRITE))
def test_write_kv_sweep(orc, seed):
    rng = np.random.default_rng(60_000 + seed)
    dtype = ["f32", "f16", "bf16", "fp8_e4m3"][seed % 4]
    hkv = int(rng.choice([1, 2, 4, 8]))
    dk, dv = [(32, 32), (64, 64), (128, 128), (192, 128), (256, 256)][int(rng.integers(5))]
    b = int(rng.choice([1, 3, 8, 16, 48, 64]))
    nb = int(rng.integers(1, 2048 // b + 2))
    T = int(rng.integers(1, min(400, nb * b) + 1))
    slots = rng.permutation(nb * b)[:T].astype(np.int32)
    kp, vp = random_bits(rng, (nb, b, hkv, dk), dtype), random_bits(rng, (nb, b, hkv, dv), dtype)
    kn, vn = random_bits(rng, (T, hkv, dk), dtype), random_bits(rng, (T, hkv, dv), dtype)
    k_pool, v_pool = dev(kp, dtype), dev(vp, dtype)
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_write_kv(k_pool, v_pool, dev(kn, dtype), dev(vn, dtype), dev(slots), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    rk, rv = kp.copy(), vp.copy()
    assert orc.write_kv(rk, rv, dtype, kn, vn, slots) == 0
    what = f"{dtype} Hkv {hkv} dims {dk}/{dv} b {b} blocks {nb} tokens {T}"
    assert host(k_pool).tobytes() == rk.tobytes(), what + ": K pool"
    assert host(v_pool).tobytes() == rv.tobytes(), what + ": V pool"


NMERGE = 30


@pytest.mark.parametrize("seed", range(NMERGE))
def test_merge_states_sweep(orc, seed):
    rng = np.random.default_rng(61_000 + seed)
    dtype = ["f32", "bf16", "f16"][seed % 3]
    T = int(rng.integers(1, 301))
    H = int(rng.choice([1, 2, 8, 32]))
    D = int(rng.choice([1, 3, 37, 64, 128, 256]))
    po, pl, so, sl, special = W.merge_case(62_000 + seed, T, H, D, special_fraction=float(rng.choice([0.0, 0.05, 0.3])))
    ptwc = int(rng.choice([-1, int(rng.integers(0, T + 1))]))
    if dtype != "f32":
        po, so = W._round_to(po, dtype), W._round_to(so, dtype)
    out = torch.full((T, H, D), float("nan"), device="cuda", dtype={"f32": torch.float32, "f16": torch.float16,
                                                                    "bf16": torch.bfloat16}[dtype])
    out_lse = torch.full((H, T), float("nan"), device="cuda")
    pa_merge_states(out, out_lse, dev(po, dtype), dev(pl), dev(so, dtype), dev(sl), prefill_tokens_with_context=ptwc)
    torch.cuda.synchronize()
    ref, rlse = orc.merge_states(po, pl, so, sl, dtype, ptwc)
    got = host(out)
    if dtype == "bf16":
        got = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.asarray(got, np.float64)
    glse = host(out_lse).astype(np.float64)
    exact = special.T.copy()  # [T, H]
    if ptwc >= 0:
        exact[ptwc:] = True
    what = f"{dtype} T {T} H {H} D {D} limit {ptwc}"
    assert np.array_equal(got[exact], ref[exact]), what + ": edge / pass-through rows must be exact copies"
    assert np.array_equal(glse.T[exact], rlse.T[exact]), what + ": edge / pass-through lse"
    regular = ~exact
    assert_close(glse.T[regular], rlse.T[regular], 1e-5, what + ": merged lse")
    if dtype == "f32":
        assert_close(got[regular], ref[regular], 1e-5, what + ": merged out")
    else:
        # one rounding to the 16-bit type (one ulp of slack), after the blend x wp + y ws
        # in fp32, whose error is a few fp32 ulps of the operands (weights <= 1): where
        # they nearly cancel, that error is large next to the result itself
        ulp = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -10
        tiny = 2.0 ** -133 if dtype == "bf16" else 2.0 ** -24  # spacing at the bottom of the range
        wide = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()  # noqa: E731
                          if dtype == "bf16" else a.astype(np.float64))
        mag = (np.abs(wide(po)) + np.abs(wide(so)))[regular]
        err = np.abs(got[regular] - ref[regular])
        bound = np.maximum(ulp * np.abs(ref[regular]), tiny) + 2.0 ** -22 * mag
        assert np.all(err <= bound), (what, float((err - bound).max()))


NGATHER = 24


@pytest.mark.parametrize("seed", range(NGATHER))
def test_gather_cache_sweep(orc, seed):
    rng = np.random.default_rng(63_000 + seed)
    types = ["f32", "f16", "bf16"]
    sd, dd = types[seed % 3], types[(seed // 3) % 3]
    D = int(rng.choice([1, 2, 7, 24, 64, 96, 128, 576, 600]))
    b = int(rng.choice([1, 5, 16, 32, 64]))
    nseq = int(rng.integers(1, 7))
    lens, tables, cache = build(rng, nseq, (1, 400), b, D, sd)
    use_starts = bool(rng.integers(2))
    if use_starts:
        starts = np.array([rng.integers(0, n) for n in lens], np.int32)
    else:
        starts = np.zeros(nseq, np.int32)
    take = np.array([rng.integers(1, n - st + 1) for n, st in zip(lens, starts)], np.int32)
    cu = np.concatenate([[0], np.cumsum(take)]).astype(np.int32)
    extra = int(rng.integers(0, 4))  # rows past the last sequence's end: left as they are
    T = int(cu[-1]) + extra
    t2s = np.concatenate([np.repeat(np.arange(nseq), take), [nseq - 1] * extra]).astype(np.int32)
    sentinel = rand_storage(rng, (T, D), dd)
    st, ref = orc.gather_cache(cache, sd, tables, cu, t2s, starts if use_starts else None, dd, T,
                               dst=sentinel.copy())
    assert st == 0
    pad = int(rng.choice([0, 0, 3, 16]))  # destination rows pad extra elements beyond D
    wide = to_dev(rand_storage(rng, (T, D + pad), dd), dd)
    wide[:, :D] = to_dev(sentinel, dd)
    pad_before = host(wide[:, D:].contiguous())
    dst = wide[:, :D]
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_gather_cache(to_dev(cache, sd), dst, dev(tables), dev(cu), dev(t2s),
                    seq_starts=dev(starts) if use_starts else None, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    what = f"{sd}->{dd} D {D} b {b} seqs {nseq} starts {use_starts} pad {pad}"
    assert same_bits(host(dst.contiguous()), ref), what
    assert host(wide[:, D:].contiguous()).tobytes() == pad_before.tobytes(), what + ": elements past the rows"
