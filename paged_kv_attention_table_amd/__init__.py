"""Batched paged attention over a block-pooled KV cache for AMD MI355X (gfx950).

The compute lives in libpa.so (hand-written HIP kernels behind the C ABI of
include/pa.h); ``binding`` exposes its entry points to torch tensors on the GPU.
"""
from .binding import (PaError, PaKvPool, load, make_pool, pa_decode, pa_decode_noalloc, pa_gather_cache,  # noqa: F401
                      pa_merge_states, pa_varlen, pa_varlen_ctx_new, pa_varlen_merge, pa_write_kv, strerror)
