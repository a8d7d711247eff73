"""Chunked-context prefill: each request's new tokens attend non-causally to its
cached context, read in fixed-size chunks, and causally to themselves; the partial
states are merged by their log-sum-exp ("cpu_mla_prefill.cpp": MlaPrefillAttention
for each piece, MergeAttnStates to combine them).

The page cites this composition (a chunked-context driver over the gather, prefill
and merge kernels) without printing it; the order used here is
    state <- chunk 0;  state <- merge(state, chunk c) for c = 1 .. C-1,
where a request's new tokens (causal) join the call of its last context chunk as a
second key segment (pa_varlen_ctx_new): merge(state, chunk c, then new) is taken as
one merge of one softmax over both, which is the same state up to rounding and
spares a separate pass over the new tokens.  A request without context joins chunk
0's call with its new tokens alone; a request whose context ends before chunk c
contributes an empty (-inf) state for it, which the merge rules absorb.  Every merge
is fused into the attention call that produces its suffix, so the state lives in
the caller's out / lse and no piece is written out and read back.

The plan holds only device metadata; ``run`` issues pa_varlen_ctx_new calls (or one
causal pa_varlen when no request has context) on the current stream.  No arithmetic
happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from .binding import pa_varlen, pa_varlen_ctx_new


class ChunkedPrefillPlan:
    def __init__(self, *, ctx_lens, new_lens, ctx_tables, new_tables, chunk, block_size, num_heads, head_dim_v,
                 scale, device="cuda"):
        ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
        new_lens = np.asarray(new_lens, dtype=np.int64)
        if chunk % block_size:
            raise ValueError("chunk must be a multiple of block_size")
        R = ctx_lens.size
        per = chunk // block_size
        self.scale = float(scale)
        self.num_chunks = int((ctx_lens.max() + chunk - 1) // chunk) if R and ctx_lens.max() > 0 else 0
        pad = int(ctx_tables.max()) if ctx_tables.size else 0
        # a request's new tokens join the call of its last context chunk (chunk 0 when
        # it has no context)
        last_chunk = np.maximum(0, (ctx_lens + chunk - 1) // chunk - 1)
        self.chunks = []
        for c in range(self.num_chunks):
            lens = np.clip(ctx_lens - c * chunk, 0, chunk).astype(np.int32)
            tab = np.full((R, per), pad, dtype=np.int32)
            src = np.asarray(ctx_tables)[:, c * per:(c + 1) * per]
            tab[:, :src.shape[1]] = src
            joins = np.where(last_chunk == c, new_lens, 0).astype(np.int32)
            self.chunks.append((torch.from_numpy(lens).to(device), torch.from_numpy(tab).to(device),
                                torch.from_numpy(joins).to(device)))
        qsl = np.zeros(R + 1, dtype=np.int32)
        qsl[1:] = np.cumsum(new_lens)
        self.T = int(qsl[-1])
        self.max_q = int(new_lens.max()) if R else 0
        self.qsl = torch.from_numpy(qsl).to(device)
        self.new_lens = torch.from_numpy(new_lens.astype(np.int32)).to(device)
        self.new_tables = torch.from_numpy(np.ascontiguousarray(new_tables, dtype=np.int32)).to(device)
        self.positions = torch.from_numpy(
            np.concatenate([np.arange(n, dtype=np.int32) for n in new_lens]) if self.T else np.zeros(0, np.int32)
        ).to(device)
        self.state_lse = torch.empty((num_heads, self.T), dtype=torch.float32, device=device)

    def run(self, k_pool, v_pool, q, out, out_lse=None, stream=None, k_scale=1.0, v_scale=1.0):
        """out [T, H, Dv] (float32) <- attention of q over context chunks + new tokens;
        out_lse [H, T] (optional) <- its lse.  k_scale / v_scale: the pools' per-tensor
        scales (fp8 pools)."""
        lse = self.state_lse if out_lse is None else out_lse
        if not self.chunks:
            pa_varlen(k_pool, v_pool, q, out, self.qsl, self.new_lens, self.positions, self.new_tables, self.max_q,
                      self.scale, causal=True, lse=lse, stream=stream, k_scale=k_scale, v_scale=v_scale)
            return
        for c, (lens, tab, joins) in enumerate(self.chunks):
            pa_varlen_ctx_new(k_pool, v_pool, q, out, lse, self.qsl, lens, tab, joins, self.positions,
                              self.new_tables, self.max_q, self.scale, merge=c > 0, stream=stream, k_scale=k_scale,
                              v_scale=v_scale)
