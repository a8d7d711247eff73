"""Pins of the CPU oracle against facts fixed outside it.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with what the pages or the mathematics fix:

* the worked example of "Paged attention for decode in C", section 3 (golden file);
* torch's scaled_dot_product_attention and logsumexp in float64 on the logical,
  unpaged cache with the GQA heads repeated -- the dense path of the
  "ar_modules_attention.py" page -- for decode, prefill chunks, windows, GQA and
  unequal QK / V head dims;
* numpy's float16 and torch's bfloat16 conversions for every 16-bit pattern;
* closed forms and invariants: one visible key returns its value exactly, q = 0
  averages the visible values, partitions reduce to the unsplit result, merging the
  two halves of a context gives the whole, block permutations and batching change
  no bit;
* the rejection rules of the decode page's section 2.6 and the merge edge rules of
  the "cpu_mla_prefill.cpp" page (MergeAttnStates);
* attention sinks as defined by ForwardWithSinks ("ManagedPagedAttention.cs"): a
  sink equals one more visible position with a zero value (checked against the
  sink-free path on a pool that holds such a position), plus closed forms;
* the latent-cache gather (GatherMlaCache) returns the logical rows a cache was
  scattered from, and its rounding to binary16 / bfloat16 gives numpy's and torch's
  bits;
* fp8 (E4M3) caches: every pattern decodes as torch's float8_e4m3fn, with the
  format's landmarks; a pool with k_scale / v_scale attends like SDPA over the cache
  torch dequantizes ("paged_attention_v2_pytorch.py", phase 1), and the scales obey
  their closed forms;
* ALiBi: outputs equal the v2 page's slope * position form computed by torch; the
  lse is the page's minus slope * (end - 1), the position the bias is counted from
  here; a one-position window returns the value and score exactly.

The same functions run against deliberately broken builds of the oracle in
test_oracle_mutants.py, which checks that each planted mistake fails at least one.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

EINVAL, ESHAPE = 1, 2


# --------------------------------------------------------------------------------
# Test-side helpers: logical caches, a test-side pool writer, dense references.
# --------------------------------------------------------------------------------

def stored(values_f64, dtype):
    """Round float values to storage (f32 / f16 / bf16 / fp8 e4m3 bits) with library
    routines."""
    a = np.asarray(values_f64, dtype=np.float32)
    if dtype == "f32":
        return a.copy()
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "fp8_e4m3":
        return torch.from_numpy(a.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return torch.from_numpy(a.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def widen(a, dtype):
    """Storage -> float64 with numpy / torch (independent of the oracle's decoders)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double().numpy()
    if dtype == "fp8_e4m3":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    return np.asarray(a).astype(np.float64)


def nan_storage(dtype):
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0),
            "fp8_e4m3": np.uint8(0x7F)}[dtype]


class Case:
    """A batch of sequences with logical caches, scattered into a pool by the test."""

    def __init__(self, rng, lengths, H, Hkv, dk, dv, dtype, b, spare_blocks=3, shared=None):
        self.lengths = list(lengths)
        self.H, self.Hkv, self.dk, self.dv, self.dtype, self.b = H, Hkv, dk, dv, dtype, b
        need = [(n + b - 1) // b for n in lengths]
        self.max_blocks = max(1, max(need))
        fresh = sum(need) - (shared[1] * (len(shared[0]) - 1) if shared else 0)
        self.num_blocks = fresh + spare_blocks
        ids = rng.permutation(self.num_blocks)
        self.tables = np.full((len(lengths), self.max_blocks), ids[-1], dtype=np.int32)
        cur = 0
        prefix = None
        for s, k in enumerate(need):
            start = 0
            if shared and s in shared[0] and prefix is not None:
                self.tables[s, :shared[1]] = prefix
                start = shared[1]
            self.tables[s, start:k] = ids[cur:cur + k - start]
            cur += k - start
            if shared and s in shared[0] and prefix is None:
                prefix = self.tables[s, :shared[1]].copy()
        self.K = [stored(rng.standard_normal((n, Hkv, dk)), dtype) for n in lengths]
        self.V = [stored(rng.standard_normal((n, Hkv, dv)), dtype) for n in lengths]
        if shared:
            first = shared[0][0]
            P = shared[1] * b
            for s in shared[0]:
                self.K[s][:P] = self.K[first][:P]
                self.V[s][:P] = self.V[first][:P]
        nan = nan_storage(dtype)
        self.k_pool = np.full((self.num_blocks, b, Hkv, dk), nan, dtype=self.K[0].dtype if lengths else np.float32)
        self.v_pool = np.full((self.num_blocks, b, Hkv, dv), nan, dtype=self.k_pool.dtype)
        for s, n in enumerate(lengths):
            for j in range(n):
                self.k_pool[self.tables[s, j // b], j % b] = self.K[s][j]
                self.v_pool[self.tables[s, j // b], j % b] = self.V[s][j]


def dense_reference(q_rows, K, V, lo, hi, scale, group):
    """torch SDPA (float64, CPU) on the logical cache with GQA heads repeated and a
    boolean visibility mask; lse from torch.logsumexp of the masked scores.
    q_rows [R, H, dk]; K [n, Hkv, dk]; V [n, Hkv, dv]; lo/hi [R] visible ranges.
    Rows with nothing visible are returned as NaN (SDPA leaves them undefined)."""
    R, H, dk = q_rows.shape
    n = K.shape[0]
    q = torch.from_numpy(np.ascontiguousarray(q_rows, dtype=np.float64)).permute(1, 0, 2).unsqueeze(0)
    k = torch.from_numpy(np.ascontiguousarray(K, dtype=np.float64)).repeat_interleave(group, dim=1)
    v = torch.from_numpy(np.ascontiguousarray(V, dtype=np.float64)).repeat_interleave(group, dim=1)
    k = k.permute(1, 0, 2).unsqueeze(0).contiguous()
    v = v.permute(1, 0, 2).unsqueeze(0).contiguous()
    j = torch.arange(n)
    mask = (j[None, :] >= torch.as_tensor(lo)[:, None]) & (j[None, :] < torch.as_tensor(hi)[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask[None, None], scale=scale)
    scores = (q @ k.transpose(-1, -2)) * scale
    scores = scores.masked_fill(~mask[None, None], float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    out = out[0].permute(1, 0, 2).numpy().copy()  # [R, H, dv]
    lse = lse[0].numpy().copy()  # [H, R]
    empty = (torch.as_tensor(hi) <= torch.as_tensor(lo)).numpy()
    out[empty] = np.nan
    return out, lse


def _varlen_segments(rng, case, segments, causal, window):
    """q and positions for (context, new) segments over case.lengths."""
    qsl = np.zeros(len(segments) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum([nq for _, nq in segments])
    T = int(qsl[-1])
    positions = np.concatenate([np.arange(c, c + nq) for c, nq in segments]).astype(np.int32) if T else \
        np.zeros(0, np.int32)
    q = stored(rng.standard_normal((T, case.H, case.dk)), case.dtype)
    return q, qsl, positions


def _ranges(positions, n, causal, window):
    end = positions + 1 if causal else np.full_like(positions, n)
    start = np.maximum(0, end - window) if window > 0 else np.zeros_like(end)
    return start, end


# --------------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------------

def _hand_pool():
    g = json.load(open(os.path.join(GOLDEN, "decode_hand_example.json")))
    b, D = g["block_size"], g["head_dim"]
    kp = np.full((g["num_blocks"], b, 1, D), np.nan, dtype=np.float32)
    vp = np.full_like(kp, np.nan)
    for j in range(g["seq_len"]):
        kp[g["table"][j // b], j % b, 0] = g["k"][j]
        vp[g["table"][j // b], j % b, 0] = g["v"][j]
    return g, kp, vp


def pin_hand_example(orc):
    """Section 3 of the decode page: o = [3, 4]; l and a as printed (7 decimals)."""
    g, kp, vp = _hand_pool()
    q = np.array([[g["q"]]], dtype=np.float32)
    bt = np.array([g["table"]], dtype=np.int32)
    st, out, lse = orc.decode(kp, vp, "f32", q, "f32", bt, [g["seq_len"]], g["scale"])
    assert st == 0, st
    np.testing.assert_allclose(out[0, 0], g["expect"]["out"], rtol=0, atol=1e-12)
    l_total = math.exp(lse[0, 0] - g["expect"]["running_after_block"][-1]["m"])
    tol = 0.5 * 10 ** -g["printed_decimals"] + 1e-12
    assert abs(l_total - g["expect"]["l"]) <= tol, l_total
    np.testing.assert_allclose(out[0, 0] * l_total, g["expect"]["a"], rtol=0, atol=tol * 10)
    # the same through varlen: one token at position 2, causal
    st, out2, lse2 = orc.varlen(kp, vp, "f32", q, "f32", [0, 1], [g["seq_len"]], [2], bt, g["scale"], True, 0)
    assert st == 0 and np.array_equal(out2, out) and np.array_equal(lse2, lse)


def pin_hand_example_per_block(orc):
    """Partitions of one block each reproduce the page's per-block running update:
    block 1 alone is the difference between the printed running values."""
    g, kp, vp = _hand_pool()
    q = np.array([[g["q"]]], dtype=np.float32)
    bt = np.array([g["table"]], dtype=np.int32)
    st, ml, es, to = orc.decode(kp, vp, "f32", q, "f32", bt, [g["seq_len"]], g["scale"],
                                partition_size=g["block_size"], max_partitions=2)
    assert st == 0, st
    run = g["expect"]["running_after_block"]
    tol = 0.5 * 10 ** -g["printed_decimals"] + 1e-12
    l0, a0 = run[0]["l"], np.array(run[0]["a"])
    l1, a1 = run[1]["l"] - run[0]["l"], np.array(run[1]["a"]) - np.array(run[0]["a"])
    assert ml[0, 0, 0] == run[0]["m"] and ml[0, 0, 1] == run[1]["m"], ml
    assert abs(es[0, 0, 0] - l0) <= tol and abs(es[0, 0, 1] - l1) <= 2 * tol, es
    np.testing.assert_allclose(to[0, 0, 0] * es[0, 0, 0], a0, atol=10 * tol, rtol=0)
    np.testing.assert_allclose(to[0, 0, 1] * es[0, 0, 1], a1, atol=10 * tol, rtol=0)
    red = orc.reduce_partitions(ml, es, to, [g["seq_len"]], g["block_size"])
    np.testing.assert_allclose(red[0, 0], g["expect"]["out"], atol=1e-12, rtol=0)


def pin_hand_example_written_through_slots(orc):
    """The worked example's cache written through the slot mapping gives the same."""
    g, kp_ref, vp_ref = _hand_pool()
    b = g["block_size"]
    kp = np.full_like(kp_ref, np.nan)
    vp = np.full_like(vp_ref, np.nan)
    slots = np.array([g["table"][j // b] * b + j % b for j in range(g["seq_len"])], dtype=np.int32)
    k_new = np.array(g["k"], dtype=np.float32)[:, None, :]
    v_new = np.array(g["v"], dtype=np.float32)[:, None, :]
    assert orc.write_kv(kp, vp, "f32", k_new, v_new, slots) == 0
    assert np.array_equal(kp, kp_ref, equal_nan=True) and np.array_equal(vp, vp_ref, equal_nan=True)
    q = np.array([[g["q"]]], dtype=np.float32)
    st, out, _ = orc.decode(kp, vp, "f32", q, "f32", np.array([g["table"]], np.int32), [g["seq_len"]], 1.0)
    assert st == 0
    np.testing.assert_allclose(out[0, 0], g["expect"]["out"], atol=1e-12, rtol=0)


def pin_decode_matches_dense(orc):
    """Decode page's differential test: GQA 6:2, D = 32, lengths 1 / 37 / 70 in
    shuffled blocks, window 0 and 20, against SDPA on the gathered logical cache."""
    rng = np.random.default_rng(7)
    for dtype in ("f32", "f16", "bf16"):
        case = Case(rng, [1, 37, 70], H=6, Hkv=2, dk=32, dv=32, dtype=dtype, b=16)
        q = stored(rng.standard_normal((3, 6, 32)), dtype)
        for window in (0, 20):
            st, out, lse = orc.decode(case.k_pool, case.v_pool, dtype, q, dtype, case.tables, case.lengths,
                                      0.17, sliding_window=window)
            assert st == 0, st
            for s, n in enumerate(case.lengths):
                pos = np.array([n - 1])
                lo, hi = _ranges(pos, n, True, window)
                ref, rlse = dense_reference(widen(q[s:s + 1], dtype), widen(case.K[s], dtype),
                                            widen(case.V[s], dtype), lo, hi, 0.17, 3)
                np.testing.assert_allclose(out[s], ref[0], atol=1e-12, rtol=1e-12)
                np.testing.assert_allclose(lse[:, s], rlse[:, 0], atol=1e-12, rtol=1e-12)


def pin_varlen_matches_dense(orc):
    """Prefill chunks mixed with decode tokens, causal and not, windows, GQA 4:1, 2:1
    and 1:1, QK dim 48 with V dim 32, against SDPA + logsumexp per sequence."""
    rng = np.random.default_rng(11)
    for (H, Hkv, dk, dv, dtype) in ((8, 2, 48, 32, "bf16"), (4, 2, 32, 32, "f16"), (3, 3, 16, 24, "f32")):
        segments = [(0, 9), (5, 1), (30, 12), (50, 1), (0, 1), (17, 0)]
        lengths = [c + nq for c, nq in segments]
        case = Case(rng, lengths, H=H, Hkv=Hkv, dk=dk, dv=dv, dtype=dtype, b=4)
        for causal, window in ((True, 0), (True, 7), (False, 0), (False, 10)):
            q, qsl, positions = _varlen_segments(rng, case, segments, causal, window)
            st, out, lse = orc.varlen(case.k_pool, case.v_pool, dtype, q, dtype, qsl, lengths,
                                      positions if causal else None, case.tables, 0.3, causal, window)
            assert st == 0, st
            for s, n in enumerate(lengths):
                t0, t1 = qsl[s], qsl[s + 1]
                if t1 == t0:
                    continue
                lo, hi = _ranges(positions[t0:t1], n, causal, window)
                ref, rlse = dense_reference(widen(q[t0:t1], dtype), widen(case.K[s], dtype),
                                            widen(case.V[s], dtype), lo, hi, 0.3, H // Hkv)
                np.testing.assert_allclose(out[t0:t1], ref, atol=1e-12, rtol=1e-12)
                np.testing.assert_allclose(lse[:, t0:t1], rlse, atol=1e-12, rtol=1e-12)


def pin_empty_rows(orc):
    """A sequence of length 0 read non-causally gives zero outputs and lse = -inf."""
    rng = np.random.default_rng(3)
    case = Case(rng, [0, 5], H=2, Hkv=1, dk=8, dv=8, dtype="f32", b=4)
    q = stored(rng.standard_normal((3, 2, 8)), "f32")
    st, out, lse = orc.varlen(case.k_pool, case.v_pool, "f32", q, "f32", [0, 2, 3], [0, 5], None, case.tables,
                              1.0, False, 0)
    assert st == 0
    assert np.all(out[:2] == 0.0) and np.all(np.isneginf(lse[:, :2])), (out[:2], lse)
    assert np.all(np.isfinite(out[2])) and np.all(np.isfinite(lse[:, 2]))


def pin_decoders(orc):
    """Every f16 and bf16 bit pattern decodes as numpy / torch decode it."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.decode_elems(bits.view(np.float16), "f16")
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(got, ref, equal_nan=True)
    got = orc.decode_elems(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(got, ref, equal_nan=True)


def pin_permutation_invariance(orc):
    """Brute force over every physical block order of tiny caches: the result is
    bitwise the same for all orders and equals the dense reference."""
    rng = np.random.default_rng(5)
    for b, n in ((1, 5), (2, 7), (4, 13)):
        nblk = (n + b - 1) // b
        K = rng.standard_normal((n, 1, 4)).astype(np.float32)
        V = rng.standard_normal((n, 1, 4)).astype(np.float32)
        q = rng.standard_normal((1, 1, 4)).astype(np.float32)
        for window in range(0, n + 1):
            first = None
            for perm in itertools.permutations(range(nblk)):
                kp = np.full((nblk, b, 1, 4), np.nan, np.float32)
                vp = np.full_like(kp, np.nan)
                for j in range(n):
                    kp[perm[j // b], j % b] = K[j]
                    vp[perm[j // b], j % b] = V[j]
                st, out, lse = orc.decode(kp, vp, "f32", q, "f32", np.array([perm], np.int32), [n], 0.5,
                                          sliding_window=window)
                assert st == 0
                if first is None:
                    first = (out.copy(), lse.copy())
                    lo, hi = _ranges(np.array([n - 1]), n, True, window)
                    ref, rlse = dense_reference(q.astype(np.float64), K.astype(np.float64), V.astype(np.float64),
                                                lo, hi, 0.5, 1)
                    np.testing.assert_allclose(out[0], ref[0], atol=1e-13, rtol=0)
                    np.testing.assert_allclose(lse[:, 0], rlse[:, 0], atol=1e-13, rtol=0)
                else:
                    assert np.array_equal(out, first[0]) and np.array_equal(lse, first[1])


def pin_closed_forms(orc):
    """One visible key returns its value exactly and lse = its score; q = 0 returns
    the mean of the visible values."""
    rng = np.random.default_rng(9)
    case = Case(rng, [23, 40], H=4, Hkv=2, dk=16, dv=16, dtype="f32", b=4)
    q = stored(rng.standard_normal((2, 4, 16)), "f32")
    st, out, lse = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.25,
                              sliding_window=1)
    assert st == 0
    for s, n in enumerate(case.lengths):
        for h in range(4):
            g = h // 2
            assert np.array_equal(out[s, h], case.V[s][n - 1, g].astype(np.float64))
            score = 0.25 * float(np.dot(q[s, h].astype(np.float64), case.K[s][n - 1, g].astype(np.float64)))
            assert abs(lse[h, s] - score) <= 1e-14 * max(1.0, abs(score))
    qz = np.zeros_like(q)
    st, out, lse = orc.decode(case.k_pool, case.v_pool, "f32", qz, "f32", case.tables, case.lengths, 0.25,
                              sliding_window=9)
    for s, n in enumerate(case.lengths):
        for h in range(4):
            mean = case.V[s][n - 9:n, h // 2].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(out[s, h], mean, atol=1e-14, rtol=0)
            assert abs(lse[h, s] - math.log(9)) < 1e-14


def pin_partitions_reduce_to_unsplit(orc):
    """Split-KV states (normalised partial outputs) reduce to the unsplit result, for
    several partition sizes and windows; a partition covering the whole context equals
    the unsplit output bit for bit; partitions outside the window are (-inf, 0, 0)."""
    rng = np.random.default_rng(13)
    case = Case(rng, [1, 15, 16, 17, 90, 133], H=4, Hkv=1, dk=16, dv=8, dtype="bf16", b=4)
    q = stored(rng.standard_normal((6, 4, 16)), "bf16")
    for window in (0, 5, 37):
        st, out, lse = orc.decode(case.k_pool, case.v_pool, "bf16", q, "bf16", case.tables, case.lengths, 0.4,
                                  sliding_window=window)
        assert st == 0
        for P in (4, 8, 32, 136):
            pmax = -(-max(case.lengths) // P)
            st, ml, es, to = orc.decode(case.k_pool, case.v_pool, "bf16", q, "bf16", case.tables, case.lengths,
                                        0.4, sliding_window=window, partition_size=P, max_partitions=pmax)
            assert st == 0
            red = orc.reduce_partitions(ml, es, to, case.lengths, P)
            np.testing.assert_allclose(red, out, atol=1e-13, rtol=0)
            for s, n in enumerate(case.lengths):
                start = max(0, n - window) if window > 0 else 0
                for p in range(-(-n // P)):
                    if (p + 1) * P <= start:
                        assert np.all(np.isneginf(ml[s, :, p])) and np.all(es[s, :, p] == 0)
                        assert np.all(to[s, :, p] == 0)
                if P >= n:
                    assert np.array_equal(to[s, :, 0], out[s])


def pin_merge_halves_equal_whole(orc):
    """Attention over a context equals the merge of attention over its two halves
    (both read non-causally), in out and lse."""
    rng = np.random.default_rng(17)
    n = 57
    case = Case(rng, [n, 30, n - 30], H=2, Hkv=2, dk=8, dv=8, dtype="f32", b=4)
    # sequences 1 and 2 hold positions [0, 30) and [30, 57) of sequence 0
    for j in range(n):
        src = case.k_pool[case.tables[0, j // 4], j % 4]
        vsrc = case.v_pool[case.tables[0, j // 4], j % 4]
        s, jj = (1, j) if j < 30 else (2, j - 30)
        case.k_pool[case.tables[s, jj // 4], jj % 4] = src
        case.v_pool[case.tables[s, jj // 4], jj % 4] = vsrc
    q = stored(rng.standard_normal((5, 2, 8)), "f32")
    whole = orc.varlen(case.k_pool, case.v_pool, "f32", q, "f32", [0, 5], [n], None, case.tables[:1], 0.5, False, 0)
    a = orc.varlen(case.k_pool, case.v_pool, "f32", q, "f32", [0, 5], [30], None, case.tables[1:2], 0.5, False, 0)
    bb = orc.varlen(case.k_pool, case.v_pool, "f32", q, "f32", [0, 5], [n - 30], None, case.tables[2:3], 0.5, False,
                    0)
    merged, mlse = orc.merge_states(a[1].astype(np.float32), a[2].astype(np.float32), bb[1].astype(np.float32),
                                    bb[2].astype(np.float32))
    np.testing.assert_allclose(merged, whole[1], atol=1e-6, rtol=0)  # inputs rounded to fp32
    np.testing.assert_allclose(mlse, whole[2], atol=1e-6, rtol=0)
    # merging with an empty (-inf) state returns the other state exactly
    empty_lse = np.full((2, 5), -np.inf, np.float32)
    x_out, x_lse = a[1].astype(np.float32), a[2].astype(np.float32)
    m2, l2 = orc.merge_states(x_out, x_lse, np.zeros_like(x_out), empty_lse)
    assert np.array_equal(m2, x_out.astype(np.float64)) and np.array_equal(l2, x_lse.astype(np.float64))
    m3, l3 = orc.merge_states(np.zeros_like(x_out), empty_lse, x_out, x_lse)
    assert np.array_equal(m3, x_out.astype(np.float64)) and np.array_equal(l3, x_lse.astype(np.float64))


def pin_merge_edge_rules(orc):
    """MergeAttnStates edge rules: +-inf lse counts as -inf; both -inf copies the
    prefix with lse -inf; one side -inf returns the other side unchanged; tokens at or
    past prefill_tokens_with_context copy the suffix."""
    rng = np.random.default_rng(19)
    T, H, D = 6, 5, 8
    po = rng.standard_normal((T, H, D)).astype(np.float32)
    so = rng.standard_normal((T, H, D)).astype(np.float32)
    pl = rng.standard_normal((H, T)).astype(np.float32)
    sl = rng.standard_normal((H, T)).astype(np.float32)
    inf = np.float32(np.inf)
    pl[0, 0], sl[0, 0] = inf, 1.5        # prefix +inf -> suffix wins
    pl[1, 0], sl[1, 0] = 0.25, inf       # suffix +inf -> prefix wins
    pl[2, 0], sl[2, 0] = -inf, -inf      # both -inf -> prefix copy, lse -inf
    pl[3, 0], sl[3, 0] = inf, -inf       # +inf and -inf -> both -inf
    pl[4, 0], sl[4, 0] = inf, inf        # both +inf -> both -inf
    out, olse = orc.merge_states(po, pl, so, sl, "f32", prefill_tokens_with_context=4)
    f = lambda a: a.astype(np.float64)
    assert np.array_equal(out[0, 0], f(so[0, 0])) and olse[0, 0] == np.float64(np.float32(1.5))
    assert np.array_equal(out[0, 1], f(po[0, 1])) and olse[1, 0] == np.float64(np.float32(0.25))
    for h in (2, 3, 4):
        assert np.array_equal(out[0, h], f(po[0, h])) and np.isneginf(olse[h, 0])
    # pass-through rows
    assert np.array_equal(out[4:], f(so[4:])) and np.array_equal(olse[:, 4:], f(sl[:, 4:]))
    # regular rows are convex blends: between the two inputs elementwise
    lo = np.minimum(po[1:4], so[1:4]) - 1e-6
    hi = np.maximum(po[1:4], so[1:4]) + 1e-6
    assert np.all(out[1:4] >= lo) and np.all(out[1:4] <= hi)
    assert np.all(olse[:, 1:4] >= np.maximum(pl[:, 1:4], sl[:, 1:4]) - 1e-12)
    assert np.all(olse[:, 1:4] <= np.maximum(pl[:, 1:4], sl[:, 1:4]) + math.log(2) + 1e-12)


def pin_invariance(orc):
    """Forks and batching (decode page, section 2.5 and its shared-blocks test): 16
    sequences, the first two blocks shared by all; each sequence alone gives the same
    bits as in the batch; one thread gives the same bits as eight; two sequences with
    the same table and query give the same row."""
    rng = np.random.default_rng(21)
    lengths = list(rng.integers(33, 90, size=16))
    case = Case(rng, lengths, H=4, Hkv=2, dk=16, dv=16, dtype="f16", b=16, shared=(list(range(16)), 2))
    q = stored(rng.standard_normal((16, 4, 16)), "f16")
    q[5] = q[3]
    tables = case.tables.copy()
    tables[5] = tables[3]
    lens = np.array(lengths, np.int32)
    lens[5] = lens[3]
    st, out, lse = orc.decode(case.k_pool, case.v_pool, "f16", q, "f16", tables, lens, 0.25, threads=8)
    assert st == 0
    st1, out1, lse1 = orc.decode(case.k_pool, case.v_pool, "f16", q, "f16", tables, lens, 0.25, threads=1)
    assert np.array_equal(out, out1) and np.array_equal(lse, lse1)
    assert np.array_equal(out[5], out[3])
    for s in range(16):
        st, o1, l1 = orc.decode(case.k_pool, case.v_pool, "f16", q[s:s + 1], "f16", tables[s:s + 1], lens[s:s + 1],
                                0.25, threads=1)
        assert np.array_equal(o1[0], out[s]) and np.array_equal(l1[:, 0], lse[:, s])
    # the shared prefix gathers to the same bits for every fork
    g0 = orc.gather(case.k_pool, "f16", 16, tables[0], 32)
    for s in range(1, 16):
        assert np.array_equal(orc.gather(case.k_pool, "f16", 16, tables[s], 32), g0)


def pin_write_kv_round_trip(orc):
    """Scatter through the slot mapping, then gather through the table: identity, bit
    for bit; a repeated slot keeps the last token written."""
    rng = np.random.default_rng(23)
    for dtype in ("f32", "f16", "bf16"):
        b, Hkv, dk, dv, n = 4, 3, 8, 12, 29
        nb = 10
        table = rng.permutation(nb)[:8].astype(np.int32)
        k_new = stored(rng.standard_normal((n, Hkv, dk)), dtype)
        v_new = stored(rng.standard_normal((n, Hkv, dv)), dtype)
        slots = np.array([table[j // b] * b + j % b for j in range(n)], dtype=np.int32)
        kp = np.zeros((nb, b, Hkv, dk), dtype=k_new.dtype)
        vp = np.zeros((nb, b, Hkv, dv), dtype=k_new.dtype)
        assert orc.write_kv(kp, vp, dtype, k_new, v_new, slots) == 0
        assert np.array_equal(orc.gather(kp, dtype, b, table, n), widen(k_new, dtype))
        assert np.array_equal(orc.gather(vp, dtype, b, table, n), widen(v_new, dtype))
        dup = slots.copy()
        dup[7] = dup[3]
        assert orc.write_kv(kp, vp, dtype, k_new, v_new, dup) == 0
        assert np.array_equal(kp.reshape(-1, Hkv, dk)[dup[3]], k_new[7])


def pin_rejections(orc):
    """Decode page, section 2.6 and its bad-tables test, plus the varlen and write
    readings: each bad input is rejected and the outputs keep their sentinel."""
    rng = np.random.default_rng(29)
    case = Case(rng, [5, 9], H=4, Hkv=2, dk=8, dv=8, dtype="f32", b=4, spare_blocks=0)
    q = stored(rng.standard_normal((2, 4, 8)), "f32")
    good_t, good_l = case.tables.copy(), np.array(case.lengths, np.int32)

    def dec(tables=good_t, lens=good_l, H=4, **kw):
        qq = q if H == 4 else stored(rng.standard_normal((2, H, 8)), "f32")
        sentinel = np.full((2, H, 8), 7.0)
        r = orc.decode(case.k_pool, case.v_pool, "f32", qq, "f32", tables, lens, 1.0, out=sentinel, **kw)
        return r[0], sentinel

    st, _ = dec()
    assert st == 0
    bad = good_l.copy(); bad[0] = 0                      # empty context
    st, o = dec(lens=bad); assert st == EINVAL and np.all(o == 7.0), st
    for s in (0, 1):                                     # needs 4 blocks, a row holds 3
        bad = good_l.copy(); bad[s] = 13                 # (row 0 is followed by valid ids)
        st, o = dec(lens=bad); assert st == EINVAL and np.all(o == 7.0), st
    t = good_t.copy(); t[1, 1] = case.num_blocks + 5     # id past the pool
    st, o = dec(tables=t); assert st == EINVAL and np.all(o == 7.0), st
    t = good_t.copy(); t[0, 0] = -1                      # negative id
    st, o = dec(tables=t); assert st == EINVAL and np.all(o == 7.0), st
    st, o = dec(H=3); assert st == ESHAPE and np.all(o == 7.0), st      # H % Hkv != 0
    st, _ = dec(partition_size=6, max_partitions=4); assert st == EINVAL, st   # not a multiple of b
    st, _ = dec(partition_size=4, max_partitions=2); assert st == EINVAL, st   # 9 tokens need 3
    # varlen: positions and query_start_loc
    qv = stored(rng.standard_normal((4, 4, 8)), "f32")

    def var(qsl, pos, lens=good_l, causal=True):
        sentinel = np.full((4, 4, 8), 7.0)
        r = orc.varlen(case.k_pool, case.v_pool, "f32", qv, "f32", qsl, lens, pos, good_t, 1.0, causal, 0,
                       out=sentinel)
        return r[0], sentinel

    st, _ = var([0, 2, 4], [3, 4, 7, 8]); assert st == 0
    st, o = var([0, 2, 4], [3, 5, 7, 8]); assert st == EINVAL and np.all(o == 7.0)   # pos >= n
    st, o = var([0, 2, 4], [3, -1, 7, 8]); assert st == EINVAL and np.all(o == 7.0)  # pos < 0
    st, o = var([0, 3, 2], [3, 4, 7, 8]); assert st == EINVAL and np.all(o == 7.0)   # decreasing
    st, o = var([0, 2, 3], [3, 4, 7, 8]); assert st == EINVAL and np.all(o == 7.0)   # last != T
    st, o = var([1, 2, 4], [3, 4, 7, 8]); assert st == EINVAL and np.all(o == 7.0)   # first != 0
    # write_kv: a slot outside the pool leaves the pool untouched
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    kn = np.ones((2, 2, 8), np.float32)
    n_slots = case.num_blocks * 4
    for bad_slot in (n_slots, -1):
        assert orc.write_kv(kp, vp, "f32", kn, kn, np.array([0, bad_slot], np.int32)) == EINVAL
        assert np.array_equal(kp, case.k_pool, equal_nan=True) and np.array_equal(vp, case.v_pool, equal_nan=True)


def _sink_position_case(rng, n_list, H, scale, target):
    """One sequence per entry of n_list, with position 0 of each holding, per head h,
    a key whose score against that sequence's query is target + h / 2 and a zero
    value.  Returns (case, q, z) with z[s, h] the exact score of that key."""
    lengths = [n + 1 for n in n_list]
    case = Case(rng, lengths, H=H, Hkv=H, dk=16, dv=16, dtype="f32", b=4)
    q = stored(rng.standard_normal((len(lengths), H, 16)), "f32")
    z = np.empty((len(lengths), H))
    for s in range(len(lengths)):
        for h in range(H):
            qh = q[s, h].astype(np.float64)
            k0 = ((target + 0.5 * h) / (scale * float(qh @ qh)) * qh).astype(np.float32)
            case.k_pool[case.tables[s, 0], 0, h] = k0
            case.v_pool[case.tables[s, 0], 0, h] = 0.0
            z[s, h] = scale * float(qh @ k0.astype(np.float64))
    return case, q, z


def pin_sink_is_a_zero_value_position(orc):
    """An attention sink ("ManagedPagedAttention.cs", ForwardWithSinks) acts as one
    more visible position whose score is the sink logit and whose value is zero:
    decode with sink z_h over positions 1 .. n - 1 equals decode without sinks over
    positions 0 .. n - 1 of the same pool, position 0 holding a key that scores z_h
    and a zero value.  Checked unsplit, split (partitions and reduction) and through
    the varlen entry, for sinks below, among and above the scores."""
    rng = np.random.default_rng(21)
    H, scale = 3, 0.25
    for target in (-6.0, 0.4, 9.0):
        case, q, z = _sink_position_case(rng, (1, 6, 13, 30), H, scale, target)
        for s, n in enumerate(case.lengths):
            one = case.tables[s:s + 1]
            ref_st, ref, rlse = orc.decode(case.k_pool, case.v_pool, "f32", q[s:s + 1], "f32", one, [n], scale)
            st, out, lse = orc.decode(case.k_pool, case.v_pool, "f32", q[s:s + 1], "f32", one, [n], scale,
                                      sliding_window=n - 1, sinks=z[s])
            assert ref_st == 0 and st == 0
            np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse, rlse, atol=1e-12, rtol=0)
            P = 8
            pm = (n + P - 1) // P
            st, ml, es, to = orc.decode(case.k_pool, case.v_pool, "f32", q[s:s + 1], "f32", one, [n], scale,
                                        sliding_window=n - 1, partition_size=P, max_partitions=pm, sinks=z[s])
            assert st == 0
            plain = orc.decode(case.k_pool, case.v_pool, "f32", q[s:s + 1], "f32", one, [n], scale,
                               sliding_window=n - 1, partition_size=P, max_partitions=pm)
            for x, y in zip((ml, es, to), plain[1:]):  # the states leave the sink to the reduction
                assert np.array_equal(x, y, equal_nan=True)
            red = orc.reduce_partitions(ml, es, to, [n], P, sinks=z[s])
            np.testing.assert_allclose(red, ref, atol=1e-12, rtol=0)
            st, vout, vlse = orc.varlen(case.k_pool, case.v_pool, "f32", q[s:s + 1], "f32", [0, 1], [n], [n - 1],
                                        one, scale, True, n - 1, sinks=z[s])
            assert st == 0
            np.testing.assert_allclose(vout, ref, atol=1e-12, rtol=0)
            np.testing.assert_allclose(vlse, rlse, atol=1e-12, rtol=0)


def pin_sink_closed_forms(orc):
    """A sink equal to the only visible score halves that key's value (lse = score +
    ln 2); with nothing visible a sink gives a zero output and lse = the sink; sinks
    of -inf change no bit of the sink-free result."""
    rng = np.random.default_rng(22)
    case = Case(rng, [9, 17], H=4, Hkv=2, dk=16, dv=16, dtype="f32", b=4)
    q = stored(rng.standard_normal((2, 4, 16)), "f32")
    for s, n in enumerate(case.lengths):
        z = np.array([0.25 * float(q[s, h].astype(np.float64) @ case.K[s][n - 1, h // 2].astype(np.float64))
                      for h in range(4)])
        st, out, lse = orc.decode(case.k_pool, case.v_pool, "f32", q[s:s + 1], "f32", case.tables[s:s + 1], [n],
                                  0.25, sliding_window=1, sinks=z)
        assert st == 0
        for h in range(4):
            np.testing.assert_allclose(out[0, h], 0.5 * case.V[s][n - 1, h // 2].astype(np.float64), atol=1e-14,
                                       rtol=0)
            assert abs(lse[h, 0] - (z[h] + math.log(2.0))) < 1e-13
    z = np.array([1.5, -2.0, 0.0, 7.25])
    qv = stored(rng.standard_normal((3, 4, 16)), "f32")
    st, out, lse = orc.varlen(case.k_pool, case.v_pool, "f32", qv, "f32", [0, 2, 3], [0, 17], None, case.tables,
                              0.25, False, 0, sinks=z)
    assert st == 0
    assert np.all(out[:2] == 0.0) and np.array_equal(lse[:, 0], z) and np.array_equal(lse[:, 1], z)
    none = np.full(4, -np.inf)
    for kw in ({}, {"sliding_window": 5}):
        a = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.25, **kw)
        b = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.25, sinks=none, **kw)
        assert a[0] == b[0] == 0 and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


def _same_bits(a, b):
    """Bitwise equality of two storage arrays of one type (float32, float16, or bf16
    as uint16), any NaN equal to any NaN."""
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    if a.dtype == np.uint16:  # bf16 bits
        an = ((a & 0x7F80) == 0x7F80) & ((a & 0x007F) != 0)
        bn = ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
        ua, ub = a, b
    else:
        an, bn = np.isnan(a), np.isnan(b)
        ua = a.view(np.uint32 if a.dtype == np.float32 else np.uint16)
        ub = b.view(ua.dtype)
    return np.array_equal(an, bn) and np.array_equal(ua[~an], ub[~bn])


def pin_encoders(orc):
    """Rounding to binary16 and bfloat16 (nearest, ties to even) gives the bits
    numpy's float16 and torch's bfloat16 conversions give: every bf16 and f16 value,
    binary32 edge values and a million random binary32 bit patterns."""
    rng = np.random.default_rng(31)
    pats = [np.arange(1 << 16, dtype=np.uint32) << 16,  # every bf16 value as binary32
            np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float32).view(np.uint32),
            rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32),
            np.array([0x477FEFFF, 0x477FF000, 0x477FF001, 0x387FC000, 0x33000000, 0x33000001, 0x7F7FFFFF,
                      0x7F7F8000, 0x7F7F7FFF, 0x80000000, 0x00000001], dtype=np.uint32)]
    f32 = np.concatenate(pats).view(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        vals = f32.astype(np.float64)
        f16 = f32.astype(np.float16)
    assert _same_bits(orc.encode_elems(vals, "f16"), f16)
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert _same_bits(orc.encode_elems(vals, "bf16"), ref)
    assert _same_bits(orc.encode_elems(vals, "f32"), f32)


def _gather_case(rng, lengths, D, dtype, b):
    """A Case with one kv head (its pool is a [blocks, b, D] latent cache)."""
    case = Case(rng, lengths, H=1, Hkv=1, dk=D, dv=D, dtype=dtype, b=b)
    return case, case.k_pool.reshape(case.num_blocks, b, D)


def pin_gather_returns_logical_rows(orc):
    """GatherMlaCache ("cpu_mla_prefill.cpp") on a cache scattered from logical
    per-sequence rows returns those rows: whole sequences, windows starting at
    seq_starts, rows past a sequence's end left untouched, and a conversion to
    another dtype equal to the library conversion of the logical rows."""
    rng = np.random.default_rng(33)
    for dtype, b in (("bf16", 16), ("f32", 4), ("f16", 8)):
        case, cache = _gather_case(rng, [37, 5, 60, 16], 24, dtype, b)
        logical = [k.reshape(len(k), 24) for k in case.K]
        # whole sequences, packed
        lens = np.array(case.lengths)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        t2s = np.repeat(np.arange(len(lens)), lens).astype(np.int32)
        st, out = orc.gather_cache(cache, dtype, case.tables, cu, t2s, None, dtype, int(cu[-1]))
        assert st == 0 and _same_bits(out, np.concatenate(logical))
        # windows: sequence s contributes take[s] rows from starts[s]; two spare rows
        # past the last sequence's end must stay untouched
        starts = np.array([3, 0, 41, 15], dtype=np.int32)
        take = np.array([20, 5, 19, 1], dtype=np.int32)
        cu = np.concatenate([[0], np.cumsum(take)]).astype(np.int32)
        T = int(cu[-1]) + 2
        t2s = np.concatenate([np.repeat(np.arange(4), take), [3, 3]]).astype(np.int32)
        sentinel = stored(np.full((T, 24), 7.0), dtype)
        st, out = orc.gather_cache(cache, dtype, case.tables, cu, t2s, starts, dtype, T, dst=sentinel.copy())
        want = np.concatenate([logical[s][starts[s]:starts[s] + take[s]] for s in range(4)])
        assert st == 0 and _same_bits(out[:-2], want)
        assert _same_bits(out[-2:], sentinel[-2:])
        # to another dtype
        other = {"bf16": "f32", "f32": "bf16", "f16": "bf16"}[dtype]
        st, out = orc.gather_cache(cache, dtype, case.tables, cu, t2s, starts, other, T)
        w64 = widen(want, dtype)
        assert st == 0 and _same_bits(out[:-2], stored(w64, other))


def pin_gather_rejections(orc):
    """A sequence index outside [0, num_seqs), a negative position, a block index past
    the table row or a block id outside the cache is refused before any write."""
    rng = np.random.default_rng(34)
    case, cache = _gather_case(rng, [10, 7], 8, "f32", 4)
    cu = np.array([0, 10, 17], np.int32)
    t2s = np.repeat(np.arange(2), [10, 7]).astype(np.int32)
    st, _ = orc.gather_cache(cache, "f32", case.tables, cu, t2s, None, "f32", 17)
    assert st == 0
    bad_t2s = t2s.copy()
    bad_t2s[4] = 2
    bad_tab = case.tables.copy()
    bad_tab[1, 0] = case.num_blocks
    cases = [dict(t2s=bad_t2s), dict(starts=np.array([0, -1], np.int32)),
             dict(starts=np.array([0, 4 * case.max_blocks], np.int32)), dict(tables=bad_tab)]
    for kw in cases:
        dst = np.full((17, 8), 5.0, np.float32)
        st, out = orc.gather_cache(cache, "f32", kw.get("tables", case.tables), cu, kw.get("t2s", t2s),
                                   kw.get("starts"), "f32", 17, dst=dst)
        assert st == EINVAL and np.all(out == 5.0), kw


# --------------------------------------------------------------------------------
# fp8 caches and the per-tensor K / V scales
# --------------------------------------------------------------------------------

def pin_e4m3_decoder(orc):
    """Every fp8 pattern decodes as torch's float8_e4m3fn decodes it, and the format's
    landmarks hold: 448 is the largest finite value, 2^-9 the smallest subnormal,
    2^-6 the smallest normal, 0x38 is 1, the sign bit negates, 0x7F / 0xFF are NaN
    and nothing is infinite; the positive patterns 0x00..0x7E increase."""
    bits = np.arange(256, dtype=np.uint8)
    got = orc.decode_elems(bits, "fp8_e4m3")
    ref = torch.from_numpy(bits.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(got, ref, equal_nan=True)
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x07] == 7 * 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert got[0x38] == 1.0 and got[0xB8] == -1.0 and got[0x39] == 1.125
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and not np.isinf(got).any()
    assert np.count_nonzero(np.isnan(got)) == 2
    assert np.all(np.diff(got[:0x7F]) > 0)
    assert np.array_equal(got[0x80:0xFF], -got[:0x7F]) and math.copysign(1.0, got[0x80]) == -1.0


def _fp8_case(rng, lengths, H, Hkv, D, b):
    """An fp8 case whose stored values span the subnormals up to about 40 (the logical
    values are those times the scales)."""
    case = Case(rng, lengths, H=H, Hkv=Hkv, dk=D, dv=D, dtype="f32", b=b)
    k8 = [stored(8.0 * widen(k, "f32"), "fp8_e4m3") for k in case.K]
    v8 = [stored(8.0 * widen(v, "f32"), "fp8_e4m3") for v in case.V]
    kp = np.full(case.k_pool.shape, 0x7F, np.uint8)
    vp = np.full(case.v_pool.shape, 0x7F, np.uint8)
    for s, n in enumerate(lengths):
        for j in range(n):
            kp[case.tables[s, j // b], j % b] = k8[s][j]
            vp[case.tables[s, j // b], j % b] = v8[s][j]
    return case, k8, v8, kp, vp


def pin_fp8_pool_is_the_dequantized_cache(orc):
    """"paged_attention_v2_pytorch.py", phase 1: an fp8 pool with k_scale / v_scale
    attends like SDPA over the cache torch dequantizes (stored value times scale),
    for decode (unsplit and through partitions), windows and varlen chunks."""
    rng = np.random.default_rng(41)
    ks, vs = 0.1171875, 0.0732421875
    case, k8, v8, kp, vp = _fp8_case(rng, [1, 29, 70], H=8, Hkv=2, D=32, b=8)
    assert np.any((k8[2] & 0x78) == 0) and np.any((k8[2] & 0x7F) >= 0x50)  # subnormals and large codes
    q = stored(rng.standard_normal((3, 8, 32)), "bf16")
    for window in (0, 13):
        st, out, lse = orc.decode(kp, vp, "fp8_e4m3", q, "bf16", case.tables, case.lengths, 0.2,
                                  sliding_window=window, k_scale=ks, v_scale=vs)
        assert st == 0, st
        st, ml, es, to = orc.decode(kp, vp, "fp8_e4m3", q, "bf16", case.tables, case.lengths, 0.2,
                                    sliding_window=window, partition_size=16, max_partitions=5,
                                    k_scale=ks, v_scale=vs)
        assert st == 0, st
        red = orc.reduce_partitions(ml, es, to, case.lengths, 16)
        for s, n in enumerate(case.lengths):
            lo, hi = _ranges(np.array([n - 1]), n, True, window)
            ref, rlse = dense_reference(widen(q[s:s + 1], "bf16"), widen(k8[s], "fp8_e4m3") * ks,
                                        widen(v8[s], "fp8_e4m3") * vs, lo, hi, 0.2, 4)
            np.testing.assert_allclose(out[s], ref[0], atol=1e-12, rtol=1e-12)
            np.testing.assert_allclose(lse[:, s], rlse[:, 0], atol=1e-12, rtol=1e-12)
            np.testing.assert_allclose(red[s], ref[0], atol=1e-12, rtol=1e-12)
    segments = [(0, 1), (20, 9), (69, 1)]
    qv = stored(rng.standard_normal((11, 8, 32)), "f16")
    qsl = np.array([0, 1, 10, 11], np.int32)
    positions = np.concatenate([np.arange(c, c + k) for c, k in segments]).astype(np.int32)
    st, out, lse = orc.varlen(kp, vp, "fp8_e4m3", qv, "f16", qsl, case.lengths, positions, case.tables, 0.3,
                              True, 0, k_scale=ks, v_scale=vs)
    assert st == 0, st
    for s, n in enumerate(case.lengths):
        t0, t1 = qsl[s], qsl[s + 1]
        lo, hi = _ranges(positions[t0:t1], n, True, 0)
        ref, rlse = dense_reference(widen(qv[t0:t1], "f16"), widen(k8[s], "fp8_e4m3") * ks,
                                    widen(v8[s], "fp8_e4m3") * vs, lo, hi, 0.3, 4)
        np.testing.assert_allclose(out[t0:t1], ref, atol=1e-12, rtol=1e-12)
        np.testing.assert_allclose(lse[:, t0:t1], rlse, atol=1e-12, rtol=1e-12)


def pin_scale_closed_forms(orc):
    """On any pool, k_scale = c scores like a softmax scale multiplied by c, and
    v_scale = c multiplies every output by c and leaves the lse alone; scales that are
    zero, negative or not finite are rejected."""
    rng = np.random.default_rng(43)
    case = Case(rng, [9, 33], H=4, Hkv=2, dk=16, dv=16, dtype="f32", b=4)
    q = stored(rng.standard_normal((2, 4, 16)), "f32")
    st, base, blse = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.25)
    assert st == 0
    st, out, lse = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.125,
                              k_scale=2.0)
    assert st == 0 and np.array_equal(out, base) and np.array_equal(lse, blse)
    st, out, lse = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.25,
                              v_scale=0.375)
    assert st == 0 and np.array_equal(lse, blse)
    np.testing.assert_allclose(out, 0.375 * base, rtol=1e-13, atol=1e-15)
    for bad in (0.0, -1.0, math.inf, math.nan):
        for kw in ({"k_scale": bad}, {"v_scale": bad}):
            st, *_ = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.25, **kw)
            assert st == EINVAL, (kw, st)
            st, *_ = orc.varlen(case.k_pool, case.v_pool, "f32", q, "f32", [0, 1, 2], case.lengths, [8, 32],
                                case.tables, 0.25, True, 0, **kw)
            assert st == EINVAL, (kw, st)


# --------------------------------------------------------------------------------
# ALiBi ("paged_attention_v2_pytorch.py", phase 1)
# --------------------------------------------------------------------------------

def alibi_slopes(H):
    """The geometric slopes 2^(-8 (h + 1) / H) (the page takes slopes as given)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)])


def page_alibi_reference(q_rows, K, V, lo, hi, scale, group, slopes):
    """The page's form with torch in float64: scores scale * q.k + slope_h * j (j the
    key's absolute position), masked to [lo, hi), softmax over keys; lse by
    torch.logsumexp.  Returns out [R, H, dv], lse [H, R]."""
    q = torch.from_numpy(np.ascontiguousarray(q_rows, dtype=np.float64))  # [R, H, dk]
    k = torch.from_numpy(np.ascontiguousarray(K, dtype=np.float64)).repeat_interleave(group, dim=1)
    v = torch.from_numpy(np.ascontiguousarray(V, dtype=np.float64)).repeat_interleave(group, dim=1)
    n = K.shape[0]
    j = torch.arange(n, dtype=torch.float64)
    scores = torch.einsum("rhd,nhd->rhn", q, k) * scale + torch.from_numpy(slopes)[None, :, None] * j[None, None, :]
    vis = (j[None, :] >= torch.as_tensor(lo)[:, None]) & (j[None, :] < torch.as_tensor(hi)[:, None])
    scores = scores.masked_fill(~vis[:, None, :], float("-inf"))
    out = torch.einsum("rhn,nhd->rhd", torch.softmax(scores, dim=-1), v)
    return out.numpy(), torch.logsumexp(scores, dim=-1).numpy().T


def pin_alibi_matches_the_pages_bias(orc):
    """Decode (unsplit and split), varlen causal and not, windows, GQA 4:1: every
    output equals the page's form; lse equals the page's minus slope * (end - 1)."""
    rng = np.random.default_rng(47)
    H, Hkv = 8, 2
    slopes = alibi_slopes(H)
    case = Case(rng, [1, 40, 150], H=H, Hkv=Hkv, dk=16, dv=24, dtype="f32", b=8)
    q = stored(rng.standard_normal((3, H, 16)), "f32")
    for window in (0, 30):
        st, out, lse = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.3,
                                  sliding_window=window, alibi_slopes=slopes)
        assert st == 0
        st, ml, es, to = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.3,
                                    sliding_window=window, partition_size=16, max_partitions=10,
                                    alibi_slopes=slopes)
        assert st == 0
        red = orc.reduce_partitions(ml, es, to, case.lengths, 16)
        for s_, n in enumerate(case.lengths):
            lo, hi = _ranges(np.array([n - 1]), n, True, window)
            ref, rlse = page_alibi_reference(widen(q[s_:s_ + 1], "f32"), widen(case.K[s_], "f32"),
                                             widen(case.V[s_], "f32"), lo, hi, 0.3, H // Hkv, slopes)
            np.testing.assert_allclose(out[s_], ref[0], atol=1e-12, rtol=1e-12)
            np.testing.assert_allclose(red[s_], ref[0], atol=1e-12, rtol=1e-12)
            np.testing.assert_allclose(lse[:, s_], rlse[:, 0] - slopes * (n - 1), atol=1e-11, rtol=1e-12)
    segments = [(0, 7), (30, 1), (100, 12)]
    lengths = [c + k for c, k in segments]
    case = Case(rng, lengths, H=H, Hkv=Hkv, dk=16, dv=16, dtype="f32", b=4)
    for causal, window in ((True, 0), (True, 9), (False, 0), (False, 20)):
        qv, qsl, positions = _varlen_segments(rng, case, segments, causal, window)
        st, out, lse = orc.varlen(case.k_pool, case.v_pool, "f32", qv, "f32", qsl, lengths,
                                  positions if causal else None, case.tables, 0.25, causal, window,
                                  alibi_slopes=slopes)
        assert st == 0
        for s_, n in enumerate(lengths):
            t0, t1 = qsl[s_], qsl[s_ + 1]
            lo, hi = _ranges(positions[t0:t1], n, causal, window)
            ref, rlse = page_alibi_reference(widen(qv[t0:t1], "f32"), widen(case.K[s_], "f32"),
                                             widen(case.V[s_], "f32"), lo, hi, 0.25, H // Hkv, slopes)
            np.testing.assert_allclose(out[t0:t1], ref, atol=1e-12, rtol=1e-12)
            np.testing.assert_allclose(lse[:, t0:t1], rlse - slopes[:, None] * (hi - 1)[None, :], atol=1e-11,
                                       rtol=1e-12)


def pin_alibi_closed_forms(orc):
    """A window of one position sees only the row's last position, whose ALiBi term
    is zero: out = v exactly and lse = scale * q.k exactly, whatever the slopes.
    Zero slopes change no bit."""
    rng = np.random.default_rng(53)
    case = Case(rng, [23, 40], H=4, Hkv=2, dk=16, dv=16, dtype="f32", b=4)
    q = stored(rng.standard_normal((2, 4, 16)), "f32")
    slopes = np.array([0.5, 1.5, 0.03125, 3.0])
    st, out, lse = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.25,
                              sliding_window=1, alibi_slopes=slopes)
    assert st == 0
    for s_, n in enumerate(case.lengths):
        for h in range(4):
            assert np.array_equal(out[s_, h], case.V[s_][n - 1, h // 2].astype(np.float64))
            score = 0.25 * float(np.dot(q[s_, h].astype(np.float64), case.K[s_][n - 1, h // 2].astype(np.float64)))
            assert abs(lse[h, s_] - score) <= 1e-14 * max(1.0, abs(score)), (lse[h, s_], score)
    st, base, blse = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.25)
    st, out, lse = orc.decode(case.k_pool, case.v_pool, "f32", q, "f32", case.tables, case.lengths, 0.25,
                              alibi_slopes=np.zeros(4))
    assert np.array_equal(out, base) and np.array_equal(lse, blse)


def pin_attend_gathered_matches_dense(orc):
    """The two-pass core on caller-gathered arrays ("cpu_mla_prefill.cpp",
    MlaPrefillAttention: QK head dim 192, V head dim 128, contiguous K / V) against
    torch SDPA + logsumexp in float64, with every row on its own visible range --
    full, prefix, suffix, interior, one key -- and an empty row (out 0, lse -inf).
    The same rows computed by the paged varlen path over a pool holding those keys
    give the same bits (both are the one definition)."""
    rng = np.random.default_rng(31)
    n, dk, dv = 53, 192, 128
    K = rng.standard_normal((n, dk))
    V = rng.standard_normal((n, dv))
    lo = np.array([0, 0, 17, 5, 52, 30, 9, 12], dtype=np.int64)
    hi = np.array([n, 20, n, 44, 53, 31, 9, 40], dtype=np.int64)
    rows = lo.size
    q = rng.standard_normal((rows, dk))
    scale = 1.0 / math.sqrt(dk)
    out, lse = orc.attend_gathered(q, K, V, lo, hi, scale)
    ref, rlse = dense_reference(q[:, None, :], K[:, None, :], V[:, None, :], lo, hi, scale, 1)
    live = hi > lo
    np.testing.assert_allclose(out[live], ref[live, 0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse[live], rlse[0, live], atol=1e-12, rtol=0)
    assert np.all(out[~live] == 0.0) and np.all(np.isneginf(lse[~live])), (out[~live], lse[~live])
    # one visible key: its value exactly, lse = its score
    one = np.flatnonzero(hi - lo == 1)
    for r in one:
        assert np.array_equal(out[r], V[lo[r]]), r
        assert abs(lse[r] - scale * float(np.dot(q[r], K[lo[r]]))) <= 1e-13
    # the same rows through the paged varlen path: one sequence per row, non-causal,
    # each sequence's cache = keys [0, hi) of this one (window = hi - lo)
    for r in range(rows):
        if hi[r] == lo[r]:
            continue
        kp = stored(K[None, :, None, :], "f32")
        vp = stored(V[None, :, None, :], "f32")
        kk, vv = kp[0, :, 0].astype(np.float64), vp[0, :, 0].astype(np.float64)
        qq = stored(q[r:r + 1, None, :], "f32")
        o1, l1 = orc.attend_gathered(qq[:, 0].astype(np.float64), kk, vv, lo[r:r + 1], hi[r:r + 1], scale)
        st, o2, l2 = orc.varlen(kp, vp, "f32", qq, "f32", [0, 1], [int(hi[r])], None, np.array([[0]], np.int32),
                                scale, False, int(hi[r] - lo[r]))
        assert st == 0
        assert np.array_equal(o1[0], o2[0, 0]) and l1[0] == l2[0, 0], r
    # out of range rows are refused
    for bad_lo, bad_hi in ((-1, 5), (0, n + 1)):
        try:
            orc.attend_gathered(q[:1], K, V, [bad_lo], [bad_hi], scale)
        except RuntimeError:
            continue
        raise AssertionError(f"range [{bad_lo}, {bad_hi}) accepted")


def pin_row_mask_selects_rows(orc):
    """orc_varlen's row mask: every selected (token, head) row equals the unmasked
    call bit for bit, every other row is left as it was, and an empty mask computes
    nothing (a mask only chooses which rows of the one definition are computed)."""
    rng = np.random.default_rng(37)
    segments = [(0, 6), (12, 1), (25, 5), (3, 1)]
    lengths = [c + nq for c, nq in segments]
    case = Case(rng, lengths, H=6, Hkv=2, dk=16, dv=8, dtype="bf16", b=4)
    q, qsl, positions = _varlen_segments(rng, case, segments, True, 0)
    T = int(qsl[-1])
    st, full, full_lse = orc.varlen(case.k_pool, case.v_pool, "bf16", q, "bf16", qsl, lengths, positions,
                                    case.tables, 0.3, True, 5)
    assert st == 0 and np.all(np.isfinite(full)) and np.all(np.isfinite(full_lse))
    for trial in range(3):
        mask = rng.random((T, 6)) < 0.35
        mask[trial, trial] = True  # never empty
        sentinel = 123.0 + trial
        out = np.full((T, 6, 8), sentinel)
        lse = np.full((6, T), sentinel)
        st, out, lse = orc.varlen(case.k_pool, case.v_pool, "bf16", q, "bf16", qsl, lengths, positions, case.tables,
                                  0.3, True, 5, row_mask=mask, out=out, lse=lse)
        assert st == 0
        assert np.array_equal(out[mask], full[mask]) and np.array_equal(lse.T[mask], full_lse.T[mask])
        assert np.all(out[~mask] == sentinel) and np.all(lse.T[~mask] == sentinel)
    none = np.zeros((T, 6), dtype=bool)
    st, out, lse = orc.varlen(case.k_pool, case.v_pool, "bf16", q, "bf16", qsl, lengths, positions, case.tables,
                              0.3, True, 5, row_mask=none)
    assert st == 0 and np.all(np.isnan(out)) and np.all(np.isnan(lse))


PINS = [pin_hand_example, pin_hand_example_per_block, pin_hand_example_written_through_slots,
        pin_decode_matches_dense, pin_varlen_matches_dense, pin_empty_rows, pin_decoders,
        pin_permutation_invariance, pin_closed_forms, pin_partitions_reduce_to_unsplit,
        pin_merge_halves_equal_whole, pin_merge_edge_rules, pin_invariance, pin_write_kv_round_trip,
        pin_rejections, pin_sink_is_a_zero_value_position, pin_sink_closed_forms, pin_encoders,
        pin_gather_returns_logical_rows, pin_gather_rejections, pin_e4m3_decoder,
        pin_fp8_pool_is_the_dequantized_cache, pin_scale_closed_forms, pin_alibi_matches_the_pages_bias,
        pin_alibi_closed_forms, pin_attend_gathered_matches_dense, pin_row_mask_selects_rows]


def run_all(path):
    """Run every pin against the oracle built at `path`; print one JSON line naming
    the pins that failed (used on mutant builds, in a child process)."""
    import sys

    here = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, os.path.dirname(here))
    from oracle.oracle import Oracle

    orc = Oracle(path)
    failed = []
    for pin in PINS:
        try:
            pin(orc)
        except Exception as e:  # noqa: BLE001 - any failure kills the mutant
            failed.append([pin.__name__, type(e).__name__])
    print(json.dumps({"failed": failed}))
