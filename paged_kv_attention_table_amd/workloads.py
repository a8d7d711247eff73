"""Seeded synthetic inputs for paged attention over a block-pooled KV cache.

This module builds inputs only: sequence lengths, block tables, slot mappings,
positions, query packing, and normally distributed values rounded to the storage
type.  It performs none of the attention arithmetic, so both the GPU path and the
CPU oracle can consume what it produces.

Layouts follow the TensorSharp "ManagedPagedAttention.cs" page (class summary):
q [tokens, heads, dim]; K/V pools [blocks, block_size, kv_heads, dim]; per-sequence
query_start_loc, seq_lens, block tables, positions and a slot mapping where
slot = block_id * block_size + offset.  The "Paged attention for decode in C" page
(section 2.1) fixes where a position lives: block table[j // b], offset j % b.

Every array is numpy.  bf16 values are carried as uint16 bit patterns and fp8
(E4M3) values as uint8 bit patterns.  Slots that
no sequence may read (unused blocks, the tail of each last block, the padding block
that pads short table rows, and the slots of tokens that are still to be written)
hold NaN, so a stray read shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8_e4m3": np.uint8}
NAN_BITS = {"f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0), "fp8_e4m3": np.uint8(0x7F)}

_CHUNK = 1 << 22


def _round_to(values_f32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type, round-to-nearest-even."""
    if dtype == "f32":
        return values_f32
    if dtype == "f16":
        return values_f32.astype(np.float16)
    import torch  # bfloat16 rounding via torch's RNE conversion

    t = torch.from_numpy(values_f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal(seed: int, tag: int, shape, dtype: str, workers: int | None = None) -> np.ndarray:
    """N(0, 1) float32 draws rounded to `dtype`.  The stream is split in fixed
    chunks, each seeded from (seed, tag, chunk index), so the result does not depend
    on how many threads draw it."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=STORAGE[dtype])
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tag, i)))
        out[lo:hi] = _round_to(rng.standard_normal(hi - lo, dtype=np.float32), dtype)

    if nchunks == 1:
        fill(0)
    else:
        w = workers or min(16, os.cpu_count() or 1)
        with ThreadPoolExecutor(max_workers=w) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def nan_value(dtype: str):
    return np.float32(np.nan) if dtype == "f32" else NAN_BITS[dtype]


@dataclass
class Paged:
    """One attention call's inputs on a paged pool."""

    name: str
    kind: str  # "decode" or "varlen"
    dtype: str
    block_size: int
    num_heads: int
    num_kv_heads: int
    dk: int
    dv: int
    k_pool: np.ndarray
    v_pool: np.ndarray
    q: np.ndarray  # [T, H, dk]
    query_start_loc: np.ndarray  # [S + 1]
    seq_lens: np.ndarray  # [S]
    positions: np.ndarray  # [T]
    block_tables: np.ndarray  # [S, max_blocks]
    k_new: np.ndarray  # [T_new, Hkv, dk]
    v_new: np.ndarray  # [T_new, Hkv, dv]
    slot_mapping: np.ndarray  # [T_new]
    scale: float
    causal: bool = True
    sliding_window: int = 0
    partition_size: int = 0
    max_partitions: int = 0
    seed: int = 0
    meta: dict = field(default_factory=dict)
    q_dtype: str = ""     # the queries' storage type when it differs from the pools' (fp8 pools)
    k_scale: float = 1.0  # the pools' per-tensor scales: element = stored value * scale
    v_scale: float = 1.0

    @property
    def query_dtype(self):
        return self.q_dtype or self.dtype

    @property
    def num_seqs(self):
        return int(self.seq_lens.size)

    @property
    def num_tokens(self):
        return int(self.q.shape[0])

    @property
    def num_blocks(self):
        return int(self.k_pool.shape[0])

    @property
    def max_blocks(self):
        return int(self.block_tables.shape[1])


def _allocate_tables(rng, lengths, block_size, shared=None, pool_blocks=None):
    """Assign physical blocks to sequences through one seeded permutation.

    lengths: tokens per sequence.  shared: optional (seq indices, prefix_blocks); the
    listed sequences name the same physical blocks for their first prefix_blocks
    logical blocks.  Returns (tables, num_blocks, pad_block, used_blocks) where the
    last physical block is a padding block that no sequence uses."""
    need = [(n + block_size - 1) // block_size for n in lengths]
    shared_seqs, shared_blocks = (list(shared[0]), int(shared[1])) if shared else ([], 0)
    fresh = sum(need) - max(0, len(shared_seqs) - 1) * shared_blocks
    total = (pool_blocks if pool_blocks is not None else fresh + 1)
    assert total >= fresh + 1, "pool too small"
    perm = rng.permutation(total - 1) if pool_blocks is None else rng.permutation(total)
    max_blocks = max(1, max(need))
    pad_block = int(perm[fresh]) if pool_blocks is not None else total - 1
    tables = np.full((len(lengths), max_blocks), pad_block, dtype=np.int32)
    cursor = 0
    prefix = None
    for s, k in enumerate(need):
        start = 0
        if s in shared_seqs and prefix is not None:
            tables[s, :shared_blocks] = prefix
            start = shared_blocks
        ids = perm[cursor:cursor + (k - start)]
        cursor += k - start
        tables[s, start:k] = ids
        if s in shared_seqs and prefix is None:
            prefix = tables[s, :shared_blocks].copy()
    used = np.zeros(total, dtype=bool)
    for s, k in enumerate(need):
        used[tables[s, :k]] = True
    return tables, total, pad_block, used


def _slot(tables, s, j, block_size):
    return int(tables[s, j // block_size]) * block_size + j % block_size


def _poison(pool, dtype, tables, lengths, used, block_size, extra_slots=()):
    """NaN into every slot no sequence may read, plus `extra_slots` (to be written)."""
    nan = nan_value(dtype)
    pool[~used] = nan
    for s, n in enumerate(lengths):
        if n % block_size:
            pool[tables[s, (n - 1) // block_size], n % block_size:] = nan
    flat = pool.reshape(-1, *pool.shape[2:])
    for slot in extra_slots:
        flat[slot] = nan


def make_paged(name, seed, *, dtype, block_size, num_heads, num_kv_heads, dk, dv, segments,
               scale=None, causal=True, sliding_window=0, partition_size=0, max_partitions=None,
               shared=None, pool_blocks=None, kind="varlen"):
    """General builder.  segments: list of (context_tokens, new_tokens) per sequence;
    the sequence holds context + new tokens, its queries are the new tokens at
    positions context .. context + new - 1, and the new tokens' K/V arrive through
    the slot mapping (their pool slots start as NaN)."""
    rng = np.random.default_rng(seed)
    lengths = [c + n for c, n in segments]
    tables, nb, pad_block, used = _allocate_tables(rng, lengths, block_size, shared, pool_blocks)
    S = len(segments)
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum([n for _, n in segments])
    T = int(qsl[-1])
    positions = np.concatenate([np.arange(c, c + n, dtype=np.int32) for c, n in segments]) \
        if T else np.zeros(0, dtype=np.int32)
    slots = np.array([_slot(tables, s, j, block_size)
                      for s, (c, n) in enumerate(segments) for j in range(c, c + n)], dtype=np.int32)
    k_pool = normal(seed, 1, (nb, block_size, num_kv_heads, dk), dtype)
    v_pool = normal(seed, 2, (nb, block_size, num_kv_heads, dv), dtype)
    _poison(k_pool, dtype, tables, lengths, used, block_size, slots)
    _poison(v_pool, dtype, tables, lengths, used, block_size, slots)
    q = normal(seed, 3, (T, num_heads, dk), dtype)
    k_new = normal(seed, 4, (T, num_kv_heads, dk), dtype)
    v_new = normal(seed, 5, (T, num_kv_heads, dv), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    if partition_size and max_partitions is None:
        max_partitions = max(1, max((n + partition_size - 1) // partition_size for n in lengths))
    return Paged(name=name, kind=kind, dtype=dtype, block_size=block_size, num_heads=num_heads,
                 num_kv_heads=num_kv_heads, dk=dk, dv=dv, k_pool=k_pool, v_pool=v_pool, q=q,
                 query_start_loc=qsl, seq_lens=np.array(lengths, dtype=np.int32), positions=positions,
                 block_tables=tables, k_new=k_new, v_new=v_new, slot_mapping=slots, scale=float(scale),
                 causal=causal, sliding_window=sliding_window, partition_size=partition_size,
                 max_partitions=max_partitions or 0, seed=seed,
                 meta={"pad_block": pad_block, "segments": list(segments)})


def make_decode(name, seed, *, seq_lens, dtype, num_heads, num_kv_heads, head_dim, block_size=16,
                scale=None, sliding_window=0, partition_size=0, max_partitions=None, shared=None,
                pool_blocks=None):
    """Decode: one query per sequence at the newest position n - 1; that token's K/V
    is the one written through the slot mapping."""
    segments = [(int(n) - 1, 1) for n in seq_lens]
    return make_paged(name, seed, dtype=dtype, block_size=block_size, num_heads=num_heads,
                      num_kv_heads=num_kv_heads, dk=head_dim, dv=head_dim, segments=segments,
                      scale=scale, causal=True, sliding_window=sliding_window,
                      partition_size=partition_size, max_partitions=max_partitions, shared=shared,
                      pool_blocks=pool_blocks, kind="decode")


# ---------------------------------------------------------------------------------
# The five workloads, at full size and scaled down (same structure, fewer tokens).
# ---------------------------------------------------------------------------------

def tiny_decode():
    """Tiny decode: seqLens {1, 17, 33, 100}, H=4, Hkv=2, D=64, b=16, fp32, pool of 64
    blocks whose ids come from one seeded permutation, scale 1/8, causal, no window."""
    return make_decode("tiny-decode", 1001, seq_lens=[1, 17, 33, 100], dtype="f32", num_heads=4,
                       num_kv_heads=2, head_dim=64, scale=1.0 / 8.0, pool_blocks=64)


def batched_decode(small=False, partition_size=512):
    """Batched decode, Llama-8B-like: 64 sequences, lengths uniform in [512, 4096],
    H=32, Hkv=8, D=128, f16, scale 1/sqrt(128); 8 forks share their first 256 tokens."""
    seed = 1002
    rng = np.random.default_rng(seed + 10_000)
    S, lo, hi, forks, prefix = (64, 512, 4096, 8, 256) if not small else (12, 40, 700, 3, 32)
    lens = rng.integers(lo, hi, size=S, endpoint=True)
    fork_ids = sorted(rng.choice(S, size=forks, replace=False).tolist())
    return make_decode("batched-decode" + ("-small" if small else ""), seed, seq_lens=lens, dtype="f16",
                       num_heads=32, num_kv_heads=8, head_dim=128, partition_size=partition_size,
                       shared=(fork_ids, prefix // 16))


def long_decode(small=False):
    """Long-context split-KV decode: 8 sequences, lengths uniform in [32768, 131072],
    H=64, Hkv=8, D=128, bf16, partitions of 512 (up to 256 of them)."""
    seed = 1003
    rng = np.random.default_rng(seed + 10_000)
    S, lo, hi, pmax = (8, 32768, 131072, 256) if not small else (3, 600, 3000, 8)
    lens = rng.integers(lo, hi, size=S, endpoint=True)
    return make_decode("long-split-decode" + ("-small" if small else ""), seed, seq_lens=lens,
                       dtype="bf16", num_heads=64, num_kv_heads=8, head_dim=128, partition_size=512,
                       max_partitions=pmax)


def mixed_varlen(small=False, shuffle=False):
    """Mixed continuous batching: 4 prefill chunks of 512 new tokens on contexts uniform
    in [0, 2048], then 12 decode tokens on contexts uniform in [256, 8192], packed in
    one query_start_loc; H=32, Hkv=8, D=128, bf16, causal, window 1024."""
    seed = 1004
    rng = np.random.default_rng(seed + 10_000)
    if small:
        pre = [(int(c), 70) for c in rng.integers(0, 200, size=2, endpoint=True)]
        dec = [(int(c), 1) for c in rng.integers(20, 600, size=3, endpoint=True)]
        window = 128
    else:
        pre = [(int(c), 512) for c in rng.integers(0, 2048, size=4, endpoint=True)]
        dec = [(int(c), 1) for c in rng.integers(256, 8192, size=12, endpoint=True)]
        window = 1024
    segments = pre + dec
    if shuffle:
        order = rng.permutation(len(segments))
        segments = [segments[i] for i in order]
    return make_paged("mixed-varlen" + ("-small" if small else "") + ("-shuffled" if shuffle else ""),
                      seed, dtype="bf16", block_size=16, num_heads=32, num_kv_heads=8, dk=128, dv=128,
                      segments=segments, causal=True, sliding_window=window)


@dataclass
class ChunkedPrefill:
    """MLA-style chunked prefill: each request's new tokens attend non-causally to its
    prior context (read in chunks) and causally to themselves."""

    name: str
    dtype: str
    block_size: int
    num_heads: int
    dk: int
    dv: int
    chunk: int
    ctx_lens: np.ndarray  # [R]
    new_lens: np.ndarray  # [R]
    k_pool: np.ndarray
    v_pool: np.ndarray
    ctx_tables: np.ndarray  # [R, ceil(max ctx / b)]
    new_tables: np.ndarray  # [R, ceil(max new / b)]
    q: np.ndarray  # [sum new, H, dk]
    query_start_loc: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    slot_mapping: np.ndarray
    scale: float
    seed: int
    q_dtype: str = ""     # the queries' storage type when it differs from the pools' (fp8 pools)
    k_scale: float = 1.0  # the pools' per-tensor scales: element = stored value * scale
    v_scale: float = 1.0

    @property
    def query_dtype(self):
        return self.q_dtype or self.dtype

    @property
    def num_tokens(self):
        return int(self.q.shape[0])


def make_chunked_prefill(name, seed, *, ctx_lens, new_lens, num_heads, dk, dv, dtype="bf16",
                         block_size=16, chunk=4096, permuted=False):
    """Context and new tokens of each request start on a block boundary.  With
    permuted=False the blocks are laid out in request order (identity tables);
    permuted=True draws them from one seeded permutation instead."""
    rng = np.random.default_rng(seed)
    R = len(ctx_lens)
    cb = [(c + block_size - 1) // block_size for c in ctx_lens]
    nbk = [(n + block_size - 1) // block_size for n in new_lens]
    used_blocks = sum(cb) + sum(nbk)
    nb = used_blocks + 1  # last block pads short table rows
    ids = rng.permutation(used_blocks) if permuted else np.arange(used_blocks)
    pad = nb - 1
    ctx_tables = np.full((R, max(1, max(cb))), pad, dtype=np.int32)
    new_tables = np.full((R, max(1, max(nbk))), pad, dtype=np.int32)
    cur = 0
    for r in range(R):
        ctx_tables[r, :cb[r]] = ids[cur:cur + cb[r]]
        cur += cb[r]
        new_tables[r, :nbk[r]] = ids[cur:cur + nbk[r]]
        cur += nbk[r]
    used = np.zeros(nb, dtype=bool)
    used[:used_blocks] = True
    used[pad] = False
    qsl = np.zeros(R + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(new_lens)
    T = int(qsl[-1])
    slots = np.array([_slot(new_tables, r, j, block_size) for r in range(R) for j in range(new_lens[r])],
                     dtype=np.int32)
    k_pool = normal(seed, 1, (nb, block_size, num_heads, dk), dtype)
    v_pool = normal(seed, 2, (nb, block_size, num_heads, dv), dtype)
    lens_all = list(ctx_lens) + list(new_lens)
    padded = np.full((2 * R, max(ctx_tables.shape[1], new_tables.shape[1])), pad, dtype=np.int32)
    padded[:R, :ctx_tables.shape[1]] = ctx_tables
    padded[R:, :new_tables.shape[1]] = new_tables
    _poison(k_pool, dtype, padded, lens_all, used, block_size, slots)
    _poison(v_pool, dtype, padded, lens_all, used, block_size, slots)
    q = normal(seed, 3, (T, num_heads, dk), dtype)
    k_new = normal(seed, 4, (T, num_heads, dk), dtype)
    v_new = normal(seed, 5, (T, num_heads, dv), dtype)
    return ChunkedPrefill(name=name, dtype=dtype, block_size=block_size, num_heads=num_heads, dk=dk, dv=dv,
                          chunk=chunk, ctx_lens=np.array(ctx_lens, dtype=np.int32),
                          new_lens=np.array(new_lens, dtype=np.int32), k_pool=k_pool, v_pool=v_pool,
                          ctx_tables=ctx_tables, new_tables=new_tables, q=q, query_start_loc=qsl,
                          k_new=k_new, v_new=v_new, slot_mapping=slots, scale=1.0 / math.sqrt(dk),
                          seed=seed)


def mla_chunked(small=False, permuted=False):
    """MLA-style chunked prefill: 8 requests, new tokens uniform in [256, 1024]
    (causal), context uniform in [0, 16384] read in non-causal chunks of 4096;
    H=128 (no GQA), QK dim 192, V dim 128, bf16."""
    seed = 1005
    rng = np.random.default_rng(seed + 10_000)
    if small:
        R, nlo, nhi, clo, chi, chunk, H = 3, 20, 150, 0, 700, 256, 4
    else:
        R, nlo, nhi, clo, chi, chunk, H = 8, 256, 1024, 0, 16384, 4096, 128
    new = rng.integers(nlo, nhi, size=R, endpoint=True).tolist()
    ctx = rng.integers(clo, chi, size=R, endpoint=True).tolist()
    if small:
        ctx[0] = 0  # a request without context exercises the all-(-inf) merge rows
    return make_chunked_prefill("mla-chunked-prefill" + ("-small" if small else "")
                                + ("-permuted" if permuted else ""), seed, ctx_lens=ctx, new_lens=new,
                                num_heads=H, dk=192, dv=128, chunk=chunk, permuted=permuted)


@dataclass
class LatentGather:
    """A paged latent cache and the index arrays of one gather of every context row."""
    name: str
    dtype: str
    cache: np.ndarray         # [num_blocks, block_size, head_dim] storage
    block_tables: np.ndarray  # [R, max_blocks] int32, seeded permutation of block ids
    ctx_lens: np.ndarray      # [R]
    cu_seq_lens: np.ndarray   # [R + 1]
    token_to_seq: np.ndarray  # [T]
    seed: int


def latent_gather(small=False):
    """The context of the MLA-style chunked-prefill requests (the same seeded lengths,
    uniform in [0, 16384]) as a paged latent cache of 576-wide bf16 rows (a 512-wide
    compressed KV row plus a 64-wide rotary key), block size 16, block ids a seeded
    permutation; the gather reads every context row of every request once."""
    seed = 1005
    rng = np.random.default_rng(seed + 10_000)
    R, clo, chi = (3, 0, 700) if small else (8, 0, 16384)
    rng.integers(20 if small else 256, 150 if small else 1024, size=R, endpoint=True)  # new tokens (unused)
    ctx = rng.integers(clo, chi, size=R, endpoint=True).astype(np.int64)
    if small:
        ctx[0] = 0
    b, D = 16, 576
    need = [(int(n) + b - 1) // b for n in ctx]
    nb = max(1, sum(need)) + 1
    grng = np.random.default_rng(seed + 20_000)
    ids = grng.permutation(nb).astype(np.int32)
    tables = np.full((R, max(1, max(need))), ids[-1], dtype=np.int32)
    cur = 0
    for r, k in enumerate(need):
        tables[r, :k] = ids[cur:cur + k]
        cur += k
    cache = normal(seed, 50, (nb, b, D), "bf16")
    cu = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    t2s = np.repeat(np.arange(R), ctx).astype(np.int32)
    return LatentGather("mla-latent-gather" + ("-small" if small else ""), "bf16", cache, tables,
                        ctx.astype(np.int32), cu, t2s, seed)


def chunk_tables(cp: ChunkedPrefill, c: int):
    """Per-request (seq_lens, block table slice) of context chunk c."""
    per = cp.chunk // cp.block_size
    lens = np.clip(cp.ctx_lens - c * cp.chunk, 0, cp.chunk).astype(np.int32)
    pad = cp.k_pool.shape[0] - 1
    tab = np.full((cp.ctx_tables.shape[0], per), pad, dtype=np.int32)
    src = cp.ctx_tables[:, c * per:(c + 1) * per]
    tab[:, :src.shape[1]] = src
    return lens, tab


def num_chunks(cp: ChunkedPrefill) -> int:
    return int((int(cp.ctx_lens.max()) + cp.chunk - 1) // cp.chunk) if cp.ctx_lens.size else 0


def merge_case(seed, num_tokens, num_heads, head_dim, special_fraction=0.05):
    """Two attention states for a merge, with a seeded fraction of rows whose lse is
    forced to +inf or -inf on either or both sides.  Returns fp32 arrays."""
    rng = np.random.default_rng(seed)
    po = normal(seed, 11, (num_tokens, num_heads, head_dim), "f32")
    so = normal(seed, 12, (num_tokens, num_heads, head_dim), "f32")
    pl = (rng.standard_normal((num_heads, num_tokens)) * 3).astype(np.float32)
    sl = (rng.standard_normal((num_heads, num_tokens)) * 3).astype(np.float32)
    special = rng.random((num_heads, num_tokens)) < special_fraction
    kinds = rng.integers(0, 5, size=(num_heads, num_tokens))
    inf, ninf = np.float32(np.inf), np.float32(-np.inf)
    # 0: prefix +inf, 1: suffix +inf, 2: both -inf, 3: +inf and -inf, 4: both +inf
    pl[special & (kinds == 0)] = inf
    sl[special & (kinds == 1)] = inf
    pl[special & (kinds == 2)] = ninf
    sl[special & (kinds == 2)] = ninf
    pl[special & (kinds == 3)] = inf
    sl[special & (kinds == 3)] = ninf
    pl[special & (kinds == 4)] = inf
    sl[special & (kinds == 4)] = inf
    return po, pl, so, sl, special


# ---------------------------------------------------------------------------------
# fp8 (E4M3) caches
# ---------------------------------------------------------------------------------

def widen_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bits -> float32 values (numpy / torch conversions)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(a).astype(np.float32)
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).float().numpy()


def quantize_e4m3(values_f32: np.ndarray, scale: float) -> np.ndarray:
    """values / scale rounded to E4M3 bits by torch's float8_e4m3fn conversion (NaN
    stays NaN)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32) / np.float32(scale))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def chunked_to_fp8(cp: ChunkedPrefill, k_scale: float = 1.0 / 16, v_scale: float = 1.0 / 32) -> ChunkedPrefill:
    """The chunked prefill over an fp8 (E4M3) cache, as to_fp8 does for a Paged
    workload: pools and new tokens divided by their scales and rounded to E4M3, the
    queries kept in the workload's 16-bit type."""
    fp8 = lambda a, sc: quantize_e4m3(widen_storage(a, cp.dtype), sc)  # noqa: E731
    return dataclasses.replace(cp, name=cp.name + "-fp8", dtype="fp8_e4m3", k_pool=fp8(cp.k_pool, k_scale),
                               v_pool=fp8(cp.v_pool, v_scale), k_new=fp8(cp.k_new, k_scale),
                               v_new=fp8(cp.v_new, v_scale), q_dtype=cp.dtype, k_scale=float(k_scale),
                               v_scale=float(v_scale))


def to_fp8(w: Paged, k_scale: float = 1.0 / 16, v_scale: float = 1.0 / 32, q_dtype: str | None = None) -> Paged:
    """The same workload over an fp8 (E4M3) cache with per-tensor scales: every K / V
    value (pools and new tokens, NaN poison included) is divided by its scale and
    rounded to E4M3, so a stored element times the scale approximates the original
    N(0, 1) value; the queries keep their values in q_dtype (the workload's f16 or
    bf16 by default)."""
    q_dtype = q_dtype or w.dtype
    assert q_dtype in ("f16", "bf16")
    q = w.q if q_dtype == w.dtype else _round_to(widen_storage(w.q, w.dtype), q_dtype)
    fp8 = lambda a, sc: quantize_e4m3(widen_storage(a, w.dtype), sc)  # noqa: E731
    return Paged(name=w.name + "-fp8", kind=w.kind, dtype="fp8_e4m3", block_size=w.block_size,
                 num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, dk=w.dk, dv=w.dv,
                 k_pool=fp8(w.k_pool, k_scale), v_pool=fp8(w.v_pool, v_scale), q=q,
                 query_start_loc=w.query_start_loc, seq_lens=w.seq_lens, positions=w.positions,
                 block_tables=w.block_tables, k_new=fp8(w.k_new, k_scale), v_new=fp8(w.v_new, v_scale),
                 slot_mapping=w.slot_mapping, scale=w.scale, causal=w.causal, sliding_window=w.sliding_window,
                 partition_size=w.partition_size, max_partitions=w.max_partitions, seed=w.seed, meta=dict(w.meta),
                 q_dtype=q_dtype, k_scale=float(k_scale), v_scale=float(v_scale))
