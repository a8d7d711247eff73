"""Python marshalling for the CPU oracle in ``oracle.c``.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The GPU library and its
binding never import it; the two implementations share no code.

Arrays are numpy.  Stored element types are named ``"f32"``, ``"f16"``, ``"bf16"`` or
``"fp8_e4m3"``; bf16 arrays are carried as ``uint16`` and fp8 arrays as ``uint8`` bit
patterns.  Every result is float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

OK, EINVAL, ESHAPE, EUNSUPPORTED = 0, 1, 2, 3
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8_e4m3": 3}
NUMPY_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8_e4m3": np.uint8}

_c_int_p = ctypes.POINTER(ctypes.c_int32)
_c_dbl_p = ctypes.POINTER(ctypes.c_double)


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (plain C11, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def _ptr(a):
    return ctypes.c_void_p(0) if a is None else ctypes.c_void_p(a.ctypes.data)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _storage(a, dtype):
    return np.ascontiguousarray(a, dtype=NUMPY_STORAGE[dtype])


def _sinks(sinks, num_heads):
    """Per-head values (sink logits, ALiBi slopes) as a contiguous float64 [H] array,
    or None."""
    if sinks is None:
        return None
    a = np.ascontiguousarray(sinks, dtype=np.float64)
    assert a.shape == (num_heads,)
    return a


def default_threads() -> int:
    return os.cpu_count() or 1


class OracleError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: oracle status {status}")
        self.status = status


class Oracle:
    """Handle on a built ``liboracle.so`` (or a mutant build of it, in the tests)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path) and path == LIBRARY:
            build()
        self.path = path
        self.lib = ctypes.CDLL(path)
        for name in ("orc_decode_elems", "orc_gather", "orc_attend_gathered", "orc_varlen",
                     "orc_decode", "orc_reduce_partitions", "orc_merge_states", "orc_write_kv",
                     "orc_encode_elems", "orc_gather_cache"):
            getattr(self.lib, name).restype = ctypes.c_int

    # -- element decoding ------------------------------------------------------------
    def decode_elems(self, src, dtype):
        src = _storage(src, dtype)
        out = np.empty(src.size, dtype=np.float64)
        st = self.lib.orc_decode_elems(_ptr(src), DTYPE_CODE[dtype], ctypes.c_int64(src.size), _ptr(out))
        if st:
            raise OracleError(st, "decode_elems")
        return out.reshape(src.shape)

    # -- gather ----------------------------------------------------------------------
    def gather(self, pool, dtype, block_size, table, seq_len):
        """pool [NB, b, Hkv, D] -> gathered [seq_len, Hkv, D] float64."""
        pool = _storage(pool, dtype)
        nb, b, hkv, d = pool.shape
        assert b == block_size
        table = _i32(table)
        out = np.empty((seq_len, hkv, d), dtype=np.float64)
        st = self.lib.orc_gather(_ptr(pool), DTYPE_CODE[dtype], ctypes.c_int64(nb), block_size, hkv, d,
                                 _ptr(table), ctypes.c_int32(table.size), ctypes.c_int32(seq_len), _ptr(out))
        if st:
            raise OracleError(st, "gather")
        return out

    # -- two-pass core on explicit arrays --------------------------------------------
    def attend_gathered(self, q, K, V, lo, hi, scale):
        q = np.ascontiguousarray(q, dtype=np.float64)
        K = np.ascontiguousarray(K, dtype=np.float64)
        V = np.ascontiguousarray(V, dtype=np.float64)
        lo = np.ascontiguousarray(lo, dtype=np.int64)
        hi = np.ascontiguousarray(hi, dtype=np.int64)
        rows, dk = q.shape
        n, dv = V.shape
        out = np.empty((rows, dv), dtype=np.float64)
        lse = np.empty(rows, dtype=np.float64)
        st = self.lib.orc_attend_gathered(_ptr(q), _ptr(K), _ptr(V), ctypes.c_int64(n), dk, dv, _ptr(lo),
                                          _ptr(hi), ctypes.c_int64(rows), ctypes.c_double(scale),
                                          _ptr(out), _ptr(lse))
        if st:
            raise OracleError(st, "attend_gathered")
        return out, lse

    # -- varlen ----------------------------------------------------------------------
    def varlen(self, k_pool, v_pool, kv_dtype, q, q_dtype, query_start_loc, seq_lens, positions,
               block_tables, scale, causal, sliding_window, row_mask=None, threads=None,
               out=None, lse=None, sinks=None, k_scale=1.0, v_scale=1.0, alibi_slopes=None):
        """Returns (status, out [T, H, dv], lse [H, T]).  Rows outside row_mask stay NaN.
        sinks: [H] sink logits (float64) or None.  k_scale / v_scale multiply every
        stored K / V element.  alibi_slopes: [H] ALiBi slopes or None."""
        k_pool = _storage(k_pool, kv_dtype)
        v_pool = _storage(v_pool, kv_dtype)
        nb, b, hkv, dk = k_pool.shape
        dv = v_pool.shape[3]
        q = _storage(q, q_dtype)
        T, H, _ = q.shape
        qsl = _i32(query_start_loc)
        sl = _i32(seq_lens)
        pos = _i32(positions)
        bt = _i32(block_tables)
        S = sl.size
        max_blocks = bt.shape[1] if bt.ndim == 2 else 0
        if out is None:
            out = np.full((T, H, dv), np.nan, dtype=np.float64)
        if lse is None:
            lse = np.full((H, T), np.nan, dtype=np.float64)
        mask = None if row_mask is None else np.ascontiguousarray(row_mask, dtype=np.uint8)
        st = self.lib.orc_varlen(_ptr(k_pool), _ptr(v_pool), DTYPE_CODE[kv_dtype], ctypes.c_int64(nb), b, hkv,
                                 dk, dv, _ptr(q), DTYPE_CODE[q_dtype], H, ctypes.c_int64(T), _ptr(qsl), S,
                                 _ptr(sl), _ptr(pos), _ptr(bt), max_blocks, ctypes.c_double(scale),
                                 int(bool(causal)), int(sliding_window), _ptr(mask), _ptr(out), _ptr(lse),
                                 _ptr(_sinks(sinks, H)), _ptr(_sinks(alibi_slopes, H)), ctypes.c_double(k_scale),
                                 ctypes.c_double(v_scale), threads or default_threads())
        return st, out, lse

    # -- decode ----------------------------------------------------------------------
    def decode(self, k_pool, v_pool, kv_dtype, q, q_dtype, block_tables, seq_lens, scale,
               sliding_window=0, partition_size=0, max_partitions=0, threads=None, out=None, sinks=None,
               k_scale=1.0, v_scale=1.0, alibi_slopes=None):
        """Unsplit: (status, out [S, H, dv], lse [H, S]).
        Split (partition_size > 0): (status, max_logits, exp_sums, tmp_out), entries
        past each sequence's partition count NaN."""
        k_pool = _storage(k_pool, kv_dtype)
        v_pool = _storage(v_pool, kv_dtype)
        nb, b, hkv, dk = k_pool.shape
        dv = v_pool.shape[3]
        q = _storage(q, q_dtype)
        S, H, _ = q.shape
        bt = _i32(block_tables)
        sl = _i32(seq_lens)
        max_blocks = bt.shape[1]
        thr = threads or default_threads()
        if partition_size <= 0:
            if out is None:
                out = np.full((S, H, dv), np.nan, dtype=np.float64)
            lse = np.full((H, S), np.nan, dtype=np.float64)
            st = self.lib.orc_decode(_ptr(k_pool), _ptr(v_pool), DTYPE_CODE[kv_dtype], ctypes.c_int64(nb), b,
                                     hkv, dk, dv, _ptr(q), DTYPE_CODE[q_dtype], H, _ptr(bt), max_blocks,
                                     _ptr(sl), S, ctypes.c_double(scale), int(sliding_window),
                                     int(partition_size), int(max_partitions), _ptr(out), _ptr(lse),
                                     None, None, None, _ptr(_sinks(sinks, H)), _ptr(_sinks(alibi_slopes, H)),
                                     ctypes.c_double(k_scale), ctypes.c_double(v_scale), thr)
            return st, out, lse
        ml = np.full((S, H, max_partitions), np.nan, dtype=np.float64)
        es = np.full((S, H, max_partitions), np.nan, dtype=np.float64)
        to = np.full((S, H, max_partitions, dv), np.nan, dtype=np.float64)
        st = self.lib.orc_decode(_ptr(k_pool), _ptr(v_pool), DTYPE_CODE[kv_dtype], ctypes.c_int64(nb), b, hkv,
                                 dk, dv, _ptr(q), DTYPE_CODE[q_dtype], H, _ptr(bt), max_blocks, _ptr(sl), S,
                                 ctypes.c_double(scale), int(sliding_window), int(partition_size),
                                 int(max_partitions), None, None, _ptr(ml), _ptr(es), _ptr(to),
                                 _ptr(_sinks(sinks, H)), _ptr(_sinks(alibi_slopes, H)), ctypes.c_double(k_scale),
                                 ctypes.c_double(v_scale), thr)
        return st, ml, es, to

    def reduce_partitions(self, max_logits, exp_sums, tmp_out, seq_lens, partition_size, sinks=None):
        ml = np.ascontiguousarray(max_logits, dtype=np.float64)
        es = np.ascontiguousarray(exp_sums, dtype=np.float64)
        to = np.ascontiguousarray(tmp_out, dtype=np.float64)
        sl = _i32(seq_lens)
        S, H, pmax, dv = to.shape
        out = np.empty((S, H, dv), dtype=np.float64)
        st = self.lib.orc_reduce_partitions(_ptr(ml), _ptr(es), _ptr(to), _ptr(sl), S, H, int(partition_size),
                                            pmax, dv, _ptr(_sinks(sinks, H)), _ptr(out))
        if st:
            raise OracleError(st, "reduce_partitions")
        return out

    # -- merge -----------------------------------------------------------------------
    def merge_states(self, prefix_out, prefix_lse, suffix_out, suffix_lse, dtype="f32",
                     prefill_tokens_with_context=-1):
        po = _storage(prefix_out, dtype)
        so = _storage(suffix_out, dtype)
        pl = np.ascontiguousarray(prefix_lse, dtype=np.float32)
        sl = np.ascontiguousarray(suffix_lse, dtype=np.float32)
        T, H, D = po.shape
        out = np.empty((T, H, D), dtype=np.float64)
        out_lse = np.empty((H, T), dtype=np.float64)
        st = self.lib.orc_merge_states(_ptr(po), _ptr(pl), _ptr(so), _ptr(sl), DTYPE_CODE[dtype],
                                       ctypes.c_int64(T), H, D, ctypes.c_int64(prefill_tokens_with_context),
                                       _ptr(out), _ptr(out_lse))
        if st:
            raise OracleError(st, "merge_states")
        return out, out_lse

    # -- latent-cache gather -----------------------------------------------------------
    def encode_elems(self, values, dtype):
        """float64 values (each a binary32 value) -> storage array of `dtype`."""
        v = np.ascontiguousarray(values, dtype=np.float64)
        out = np.empty(v.shape, dtype=NUMPY_STORAGE[dtype])
        st = self.lib.orc_encode_elems(_ptr(v), DTYPE_CODE[dtype], ctypes.c_int64(v.size), _ptr(out))
        if st:
            raise OracleError(st, "encode_elems")
        return out

    def gather_cache(self, cache, src_dtype, block_table, cu_seq_lens, token_to_seq, seq_starts, dst_dtype,
                     num_tokens, dst=None):
        """Gather rows of a paged cache [num_blocks, block_size, head_dim] into dst
        [num_tokens, head_dim] of dst_dtype (rows that are skipped keep dst's
        contents; a NaN-filled dst by default).  Returns (status, dst)."""
        c = _storage(cache, src_dtype)
        nb, b, D = c.shape
        bt = _i32(block_table)
        cu = _i32(cu_seq_lens)
        t2s = _i32(token_to_seq)
        starts = None if seq_starts is None else _i32(seq_starts)
        if dst is None:
            nan = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dst_dtype]
            dst = np.full((num_tokens, D), nan, dtype=NUMPY_STORAGE[dst_dtype])
        st = self.lib.orc_gather_cache(_ptr(c), DTYPE_CODE[src_dtype], ctypes.c_int64(nb), b, D,
                                       ctypes.c_int64(b * D), ctypes.c_int64(D), _ptr(dst), DTYPE_CODE[dst_dtype],
                                       ctypes.c_int64(D), _ptr(bt), bt.shape[1], _ptr(cu), _ptr(t2s),
                                       _ptr(starts), cu.size - 1, ctypes.c_int64(num_tokens))
        return st, dst

    # -- KV write --------------------------------------------------------------------
    def write_kv(self, k_pool, v_pool, dtype, k_new, v_new, slot_mapping):
        """Scatter in place into k_pool / v_pool (numpy arrays of the storage type)."""
        assert k_pool.dtype == NUMPY_STORAGE[dtype] and k_pool.flags.c_contiguous
        assert v_pool.dtype == NUMPY_STORAGE[dtype] and v_pool.flags.c_contiguous
        nb, b, hkv, dk = k_pool.shape
        dv = v_pool.shape[3]
        kn = _storage(k_new, dtype)
        vn = _storage(v_new, dtype)
        sm = _i32(slot_mapping)
        return self.lib.orc_write_kv(_ptr(k_pool), _ptr(v_pool), DTYPE_CODE[dtype], ctypes.c_int64(nb), b, hkv,
                                     dk, dv, _ptr(kn), _ptr(vn), _ptr(sm), ctypes.c_int64(sm.size))


_default = None


def get() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default
