"""ctypes binding of libpa.so: the entry points of include/pa.h under the same
names, taking torch tensors that live on the GPU.

The binding only marshals arguments (device pointers, sizes, dtype codes, the
current HIP stream); every step of the computation runs in the library's kernels.
If libpa.so has not been built the first call raises -- there is no fallback.
torch is imported before the library is loaded so that libpa.so binds to the HIP
runtime torch already loaded, and streams and pointers are shared.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libpa.so")

PA_OK, PA_EINVAL, PA_ESHAPE, PA_EUNSUPPORTED, PA_EDEVICE, PA_ESCRATCH = 0, 1, 2, 3, 4, 5
PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
DTYPE_CODE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
              torch.float8_e4m3fn: PA_FP8_E4M3}

EXPORTS = ("pa_strerror", "pa_write_kv", "pa_decode", "pa_decode_noalloc", "pa_varlen", "pa_varlen_merge",
           "pa_varlen_ctx_new", "pa_merge_states", "pa_gather_cache")


class PaKvPool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("num_blocks", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libpa.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m paged_kv_attention_table_amd.build`")
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    pool_p = ctypes.POINTER(PaKvPool)
    lib.pa_strerror.restype = ctypes.c_char_p
    lib.pa_strerror.argtypes = [ctypes.c_int]
    lib.pa_write_kv.restype = ctypes.c_int
    lib.pa_write_kv.argtypes = [pool_p, vp, vp, vp, i64, vp, vp]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode.argtypes = [pool_p, vp, i32, vp, i32, vp, i32, vp, i32, i32, f32, i32, i32, i32, vp, vp, vp,
                              vp, vp, vp, vp]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [pool_p, vp, i32, vp, i32, vp, i32, vp, i32, i32, f32, i32, i32, vp, vp, vp, vp]
    lib.pa_varlen.restype = ctypes.c_int
    lib.pa_varlen.argtypes = [pool_p, vp, i32, vp, i32, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, f32, i32, i32,
                              i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.pa_varlen_merge.restype = ctypes.c_int
    lib.pa_varlen_merge.argtypes = [pool_p, vp, i32, vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, f32, i32, i32,
                                    vp, vp, vp, vp]
    lib.pa_varlen_ctx_new.restype = ctypes.c_int
    lib.pa_varlen_ctx_new.argtypes = [pool_p, vp, i32, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, i32, i32, i64, i32, i32,
                                      f32, vp, vp, vp]
    lib.pa_merge_states.restype = ctypes.c_int
    lib.pa_merge_states.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i64, i32, vp]
    lib.pa_gather_cache.restype = ctypes.c_int
    lib.pa_gather_cache.argtypes = [vp, i32, i64, i32, i32, i64, i64, vp, i32, i64, vp, i32, vp, vp, vp, i32, i64,
                                    vp, vp]
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().pa_strerror(int(status)).decode()


# ------------------------------------------------------------------------------------
# marshalling helpers
# ------------------------------------------------------------------------------------

def _dev(t, name, dtype=None, ndim=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _shape(t, shape, name):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check(status, what):
    if status != PA_OK:
        raise PaError(status, what)


def _code(t, name):
    if t.dtype not in DTYPE_CODE:
        raise TypeError(f"{name}: no element type code for {t.dtype}")
    return DTYPE_CODE[t.dtype]


def make_pool(k_pool: torch.Tensor, v_pool: torch.Tensor, k_scale: float = 1.0, v_scale: float = 1.0) -> PaKvPool:
    """Descriptor for pools [num_blocks, block_size, num_kv_heads, head_dim] (f32, f16,
    bf16 or float8_e4m3fn); K / V elements count as stored value times k_scale /
    v_scale."""
    _dev(k_pool, "k_pool", ndim=4)
    _dev(v_pool, "v_pool", dtype=k_pool.dtype, ndim=4)
    nb, b, hkv, dk = k_pool.shape
    if tuple(v_pool.shape[:3]) != (nb, b, hkv):
        raise ValueError("k_pool and v_pool disagree on blocks / block size / kv heads")
    return PaKvPool(k_pool.data_ptr(), v_pool.data_ptr(), nb, b, hkv, dk, v_pool.shape[3],
                    _code(k_pool, "k_pool"), float(k_scale), float(v_scale))


# ------------------------------------------------------------------------------------
# entry points
# ------------------------------------------------------------------------------------

def pa_write_kv(k_pool, v_pool, k_new, v_new, slot_mapping, status=None, stream=None):
    """Scatter k_new / v_new [T, Hkv, D] into the pools at slot_mapping [T] (int32)."""
    pool = make_pool(k_pool, v_pool)
    _dev(k_new, "k_new", dtype=k_pool.dtype)
    _dev(v_new, "v_new", dtype=k_pool.dtype)
    _dev(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    _dev(status, "status", dtype=torch.int32)
    T = slot_mapping.numel()
    _shape(k_new, (T, pool.num_kv_heads, pool.head_dim_k), "k_new")
    _shape(v_new, (T, pool.num_kv_heads, pool.head_dim_v), "v_new")
    st = load().pa_write_kv(ctypes.byref(pool), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                            slot_mapping.numel(), _ptr(status), _stream(stream))
    _check(st, "pa_write_kv")


def pa_decode(k_pool, v_pool, q, out, block_tables, seq_lens, scale, sliding_window=0, partition_size=0,
              max_logits=None, exp_sums=None, tmp_out=None, status=None, stream=None, sinks=None, k_scale=1.0,
              v_scale=1.0, alibi_slopes=None):
    """One decode step; q [S, H, D] (the pools' dtype; f16 / bf16 over fp8 pools), out
    [S, H, D] (float32 or q's dtype); sinks [H] float32 attention-sink logits or None;
    k_scale / v_scale: the pools' per-tensor scales; alibi_slopes [H] float32 or None."""
    pool = make_pool(k_pool, v_pool, k_scale, v_scale)
    _dev(q, "q", ndim=3)
    _dev(out, "out", ndim=3)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(seq_lens, "seq_lens", dtype=torch.int32, ndim=1)
    _dev(max_logits, "max_logits", dtype=torch.float32)
    _dev(exp_sums, "exp_sums", dtype=torch.float32)
    _dev(tmp_out, "tmp_out", dtype=torch.float32)
    _dev(status, "status", dtype=torch.int32)
    _dev(sinks, "sinks", dtype=torch.float32, ndim=1)
    _dev(alibi_slopes, "alibi_slopes", dtype=torch.float32, ndim=1)
    S, H, _ = q.shape
    _shape(sinks, (H,), "sinks")
    _shape(alibi_slopes, (H,), "alibi_slopes")
    _shape(q, (S, H, pool.head_dim_k), "q")
    _shape(out, (S, H, pool.head_dim_v), "out")
    _shape(seq_lens, (S,), "seq_lens")
    if block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per sequence")
    max_partitions = 0
    if partition_size:
        if max_logits is None or exp_sums is None or tmp_out is None:
            raise ValueError("split-KV decode needs max_logits, exp_sums and tmp_out")
        max_partitions = max_logits.shape[-1]
        _shape(max_logits, (S, H, max_partitions), "max_logits")
        _shape(exp_sums, (S, H, max_partitions), "exp_sums")
        _shape(tmp_out, (S, H, max_partitions, pool.head_dim_v), "tmp_out")
    st = load().pa_decode(ctypes.byref(pool), _ptr(q), _code(q, "q"), _ptr(out), _code(out, "out"),
                          _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, H, float(scale),
                          int(sliding_window), int(partition_size), int(max_partitions), _ptr(max_logits),
                          _ptr(exp_sums), _ptr(tmp_out), _ptr(sinks), _ptr(alibi_slopes), _ptr(status),
                          _stream(stream))
    _check(st, "pa_decode")


def pa_decode_noalloc(k_pool, v_pool, q, out, block_tables, seq_lens, scale, sliding_window=0, partition_size=0,
                      status=None, stream=None, sinks=None, k_scale=1.0, v_scale=1.0, alibi_slopes=None):
    """pa_decode whose split-KV partition states live in the library's static device
    buffer (no workspace arguments, nothing allocated by the call)."""
    pool = make_pool(k_pool, v_pool, k_scale, v_scale)
    _dev(q, "q", ndim=3)
    _dev(out, "out", ndim=3)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(seq_lens, "seq_lens", dtype=torch.int32, ndim=1)
    _dev(status, "status", dtype=torch.int32)
    _dev(sinks, "sinks", dtype=torch.float32, ndim=1)
    _dev(alibi_slopes, "alibi_slopes", dtype=torch.float32, ndim=1)
    S, H, _ = q.shape
    _shape(sinks, (H,), "sinks")
    _shape(alibi_slopes, (H,), "alibi_slopes")
    _shape(q, (S, H, pool.head_dim_k), "q")
    _shape(out, (S, H, pool.head_dim_v), "out")
    _shape(seq_lens, (S,), "seq_lens")
    if block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per sequence")
    st = load().pa_decode_noalloc(ctypes.byref(pool), _ptr(q), _code(q, "q"), _ptr(out), _code(out, "out"),
                                  _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, H, float(scale),
                                  int(sliding_window), int(partition_size), _ptr(sinks), _ptr(alibi_slopes),
                                  _ptr(status), _stream(stream))
    _check(st, "pa_decode_noalloc")


def pa_varlen(k_pool, v_pool, q, out, query_start_loc, seq_lens, positions, block_tables, max_query_len, scale,
              causal=True, sliding_window=0, lse=None, status=None, stream=None, sinks=None, k_scale=1.0,
              v_scale=1.0, alibi_slopes=None, partition_size=0, max_logits=None, exp_sums=None, tmp_out=None):
    """Varlen attention; q [T, H, Dk], out [T, H, Dv], lse [H, T] (optional); sinks
    [H] float32 attention-sink logits or None; k_scale / v_scale: the pools'
    per-tensor scales; alibi_slopes [H] float32 or None.  partition_size > 0 splits
    sequences of one query token over partitions, with float32 scratch max_logits /
    exp_sums [S, H, P] and tmp_out [S, H, P, Dv]."""
    pool = make_pool(k_pool, v_pool, k_scale, v_scale)
    _dev(q, "q", ndim=3)
    _dev(out, "out", ndim=3)
    _dev(lse, "lse", dtype=torch.float32, ndim=2)
    _dev(query_start_loc, "query_start_loc", dtype=torch.int32, ndim=1)
    _dev(seq_lens, "seq_lens", dtype=torch.int32, ndim=1)
    _dev(positions, "positions", dtype=torch.int32, ndim=1)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(status, "status", dtype=torch.int32)
    _dev(sinks, "sinks", dtype=torch.float32, ndim=1)
    _dev(alibi_slopes, "alibi_slopes", dtype=torch.float32, ndim=1)
    _dev(max_logits, "max_logits", dtype=torch.float32)
    _dev(exp_sums, "exp_sums", dtype=torch.float32)
    _dev(tmp_out, "tmp_out", dtype=torch.float32)
    T, H, _ = q.shape
    _shape(sinks, (H,), "sinks")
    _shape(alibi_slopes, (H,), "alibi_slopes")
    max_partitions = 0
    if partition_size:
        if max_logits is None or exp_sums is None or tmp_out is None:
            raise ValueError("split single-token rows need max_logits, exp_sums and tmp_out")
        max_partitions = max_logits.shape[-1]
        S_ = seq_lens.numel()
        _shape(max_logits, (S_, H, max_partitions), "max_logits")
        _shape(exp_sums, (S_, H, max_partitions), "exp_sums")
        _shape(tmp_out, (S_, H, max_partitions, pool.head_dim_v), "tmp_out")
    S = seq_lens.numel()
    _shape(q, (T, H, pool.head_dim_k), "q")
    _shape(out, (T, H, pool.head_dim_v), "out")
    _shape(lse, (H, T), "lse")
    _shape(query_start_loc, (S + 1,), "query_start_loc")
    _shape(positions, (T,), "positions")
    if block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per sequence")
    st = load().pa_varlen(ctypes.byref(pool), _ptr(q), _code(q, "q"), _ptr(out), _code(out, "out"),
                          _ptr(lse), _ptr(query_start_loc), _ptr(seq_lens), _ptr(positions), _ptr(block_tables),
                          block_tables.shape[1], seq_lens.numel(), T, int(max_query_len), H, float(scale),
                          int(bool(causal)), int(sliding_window), int(partition_size), int(max_partitions),
                          _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out), _ptr(sinks), _ptr(alibi_slopes),
                          _ptr(status), _stream(stream))
    _check(st, "pa_varlen")


def pa_varlen_merge(k_pool, v_pool, q, out, query_start_loc, seq_lens, positions, block_tables, max_query_len, scale,
                    causal=True, sliding_window=0, lse=None, status=None, stream=None, sinks=None, k_scale=1.0,
                    v_scale=1.0, alibi_slopes=None):
    """pa_varlen's arguments; the attention is merged into the state held by out
    [T, H, Dv] float32 and lse [H, T] float32 (required), both updated in place."""
    if lse is None:
        raise ValueError("pa_varlen_merge needs the state's lse")
    pool = make_pool(k_pool, v_pool, k_scale, v_scale)
    _dev(q, "q", ndim=3)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    _dev(lse, "lse", dtype=torch.float32, ndim=2)
    _dev(query_start_loc, "query_start_loc", dtype=torch.int32, ndim=1)
    _dev(seq_lens, "seq_lens", dtype=torch.int32, ndim=1)
    _dev(positions, "positions", dtype=torch.int32, ndim=1)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(status, "status", dtype=torch.int32)
    _dev(sinks, "sinks", dtype=torch.float32, ndim=1)
    _dev(alibi_slopes, "alibi_slopes", dtype=torch.float32, ndim=1)
    T, H, _ = q.shape
    S = seq_lens.numel()
    _shape(sinks, (H,), "sinks")
    _shape(alibi_slopes, (H,), "alibi_slopes")
    _shape(out, (T, H, pool.head_dim_v), "out")
    _shape(lse, (H, T), "lse")
    _shape(query_start_loc, (S + 1,), "query_start_loc")
    _shape(positions, (T,), "positions")
    if block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per sequence")
    st = load().pa_varlen_merge(ctypes.byref(pool), _ptr(q), _code(q, "q"), _ptr(out), _ptr(lse),
                                _ptr(query_start_loc), _ptr(seq_lens), _ptr(positions), _ptr(block_tables),
                                block_tables.shape[1], S, T, int(max_query_len), H, float(scale), int(bool(causal)),
                                int(sliding_window), _ptr(sinks), _ptr(alibi_slopes), _ptr(status), _stream(stream))
    _check(st, "pa_varlen_merge")


def pa_varlen_ctx_new(k_pool, v_pool, q, out, lse, query_start_loc, ctx_lens, ctx_tables, new_lens, new_positions,
                      new_tables, max_query_len, scale, merge=False, sinks=None, status=None, stream=None, k_scale=1.0,
                      v_scale=1.0):
    """Attention of q [T, H, Dk] over each sequence's context segment (ctx_lens,
    ctx_tables; non-causal) and its new tokens (new_lens, new_tables; causal by
    new_positions [T]); out [T, H, Dv] and lse [H, T] float32 receive the result, or
    hold a state it is merged into (merge=True)."""
    pool = make_pool(k_pool, v_pool, k_scale, v_scale)
    _dev(q, "q", ndim=3)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    _dev(lse, "lse", dtype=torch.float32, ndim=2)
    _dev(query_start_loc, "query_start_loc", dtype=torch.int32, ndim=1)
    for t, name in ((ctx_lens, "ctx_lens"), (new_lens, "new_lens"), (new_positions, "new_positions")):
        _dev(t, name, dtype=torch.int32, ndim=1)
    _dev(ctx_tables, "ctx_tables", dtype=torch.int32, ndim=2)
    _dev(new_tables, "new_tables", dtype=torch.int32, ndim=2)
    _dev(status, "status", dtype=torch.int32)
    _dev(sinks, "sinks", dtype=torch.float32, ndim=1)
    T, H, _ = q.shape
    S = ctx_lens.numel()
    _shape(sinks, (H,), "sinks")
    _shape(out, (T, H, pool.head_dim_v), "out")
    _shape(lse, (H, T), "lse")
    _shape(query_start_loc, (S + 1,), "query_start_loc")
    _shape(new_lens, (S,), "new_lens")
    _shape(new_positions, (T,), "new_positions")
    if ctx_tables.shape[0] != S or new_tables.shape[0] != S:
        raise ValueError("ctx_tables and new_tables must have one row per sequence")
    st = load().pa_varlen_ctx_new(ctypes.byref(pool), _ptr(q), _code(q, "q"), _ptr(out), _ptr(lse), int(bool(merge)),
                                  _ptr(query_start_loc), _ptr(ctx_lens), _ptr(ctx_tables), ctx_tables.shape[1],
                                  _ptr(new_lens), _ptr(new_positions), _ptr(new_tables), new_tables.shape[1], S, T,
                                  int(max_query_len), H, float(scale), _ptr(sinks), _ptr(status), _stream(stream))
    _check(st, "pa_varlen_ctx_new")


def pa_merge_states(out, out_lse, prefix_out, prefix_lse, suffix_out, suffix_lse, prefill_tokens_with_context=-1,
                    stream=None):
    """Merge two states; outputs [T, H, D], lse [H, T] float32; out_lse optional."""
    _dev(out, "out", ndim=3)
    _dev(prefix_out, "prefix_out", dtype=out.dtype, ndim=3)
    _dev(suffix_out, "suffix_out", dtype=out.dtype, ndim=3)
    _dev(out_lse, "out_lse", dtype=torch.float32, ndim=2)
    _dev(prefix_lse, "prefix_lse", dtype=torch.float32, ndim=2)
    _dev(suffix_lse, "suffix_lse", dtype=torch.float32, ndim=2)
    T, H, D = out.shape
    for t, name in ((prefix_out, "prefix_out"), (suffix_out, "suffix_out")):
        _shape(t, (T, H, D), name)
    for t, name in ((out_lse, "out_lse"), (prefix_lse, "prefix_lse"), (suffix_lse, "suffix_lse")):
        _shape(t, (H, T), name)
    st = load().pa_merge_states(_ptr(out), _ptr(out_lse), _ptr(prefix_out), _ptr(prefix_lse), _ptr(suffix_out),
                                _ptr(suffix_lse), T, H, D, int(prefill_tokens_with_context), DTYPE_CODE[out.dtype],
                                _stream(stream))
    _check(st, "pa_merge_states")


def pa_gather_cache(cache, dst, block_table, cu_seq_lens, token_to_seq, seq_starts=None, status=None, stream=None):
    """Gather rows of a paged cache [num_blocks, block_size, head_dim] (or any view
    whose last dim is contiguous) into dst [num_tokens, head_dim] (rows may be
    strided; dtype may differ)."""
    _dev(cache, "cache", ndim=3)
    _dev(block_table, "block_table", dtype=torch.int32, ndim=2)
    _dev(cu_seq_lens, "cu_seq_lens", dtype=torch.int32, ndim=1)
    _dev(token_to_seq, "token_to_seq", dtype=torch.int32, ndim=1)
    _dev(seq_starts, "seq_starts", dtype=torch.int32, ndim=1)
    _dev(status, "status", dtype=torch.int32)
    if not isinstance(dst, torch.Tensor) or dst.device.type != "cuda" or dst.dim() != 2 or dst.stride(1) != 1:
        raise ValueError("dst must be a 2-d GPU tensor with contiguous rows")
    nb, b, D = cache.shape
    T = token_to_seq.numel()
    S = cu_seq_lens.numel() - 1
    _shape(dst, (T, D), "dst")
    if block_table.shape[0] != S:
        raise ValueError("block_table must have one row per sequence")
    _shape(seq_starts, (S,), "seq_starts")
    st = load().pa_gather_cache(_ptr(cache), DTYPE_CODE[cache.dtype], nb, b, D, b * D, D, dst.data_ptr(),
                                DTYPE_CODE[dst.dtype], dst.stride(0), _ptr(block_table), block_table.shape[1],
                                _ptr(cu_seq_lens), _ptr(token_to_seq), _ptr(seq_starts), S, T, _ptr(status),
                                _stream(stream))
    _check(st, "pa_gather_cache")
