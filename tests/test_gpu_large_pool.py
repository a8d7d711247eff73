"""Pools past 2^31 elements on the GPU against the CPU oracle: small seeded workloads
whose blocks sit at the top of a pool of more than 2^31 elements (so every element
offset a kernel forms for them exceeds 31 bits), the rest of the pool NaN.  Covered:
pa_write_kv, the MFMA decode kernel (unsplit and split, 16-bit and fp8 caches), the
tiled prefill kernel with single-token rows, the per-row kernel (fp32) and the
latent-cache gather.  The oracle sees the same logical cache in a compact pool."""
import math

import numpy as np
import pytest
import torch

from paged_kv_attention_table_amd import pa_decode, pa_gather_cache, pa_varlen, pa_write_kv
from paged_kv_attention_table_amd import workloads as W
from tests.gpu_util import TOL, assert_close, bits_equal, dev, host, threads, workload

pytestmark = pytest.mark.gpu

NAN_BITS = {"f32": (torch.int32, 0x7FC00000), "f16": (torch.int16, 0x7E00), "bf16": (torch.int16, 0x7FC0),
            "fp8_e4m3": (torch.uint8, 0x7F)}
VIEW = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn}


def offset_blocks(elems_per_block):
    """Blocks to place before the workload's so that its first element sits past 2^31."""
    return math.ceil((1 << 31) / elems_per_block) + 1


def big_pool(compact, dtype, off):
    """[off + nb, ...] device pool of NaN with `compact` (numpy storage) at blocks off.."""
    it, bits = NAN_BITS[dtype]
    shape = (off + compact.shape[0],) + tuple(compact.shape[1:])
    t = torch.full(shape, bits, dtype=it, device="cuda").view(VIEW[dtype])
    t[off:] = dev(compact, dtype)
    return t


class BigDevice:
    """A workloads.Paged placed at the top of pools of more than 2^31 elements."""

    def __init__(self, w):
        self.w = w
        per_block = w.block_size * w.num_kv_heads * max(w.dk, w.dv)
        self.off = off = offset_blocks(w.block_size * w.num_kv_heads * min(w.dk, w.dv))
        assert off * w.block_size * w.num_kv_heads * min(w.dk, w.dv) >= 1 << 31 and per_block > 0
        self.k_pool = big_pool(w.k_pool, w.dtype, off)
        self.v_pool = big_pool(w.v_pool, w.dtype, off)
        self.q = dev(w.q, w.query_dtype)
        self.qsl = dev(w.query_start_loc)
        self.seq_lens = dev(w.seq_lens)
        self.positions = dev(w.positions)
        self.tables = dev(w.block_tables + off)
        status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        pa_write_kv(self.k_pool, self.v_pool, dev(w.k_new, w.dtype), dev(w.v_new, w.dtype),
                    dev(w.slot_mapping + off * w.block_size), status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0

    def top(self, pool):
        return host(pool[self.off:])

    def free(self):
        del self.k_pool, self.v_pool
        torch.cuda.empty_cache()


def oracle_pools(orc, w):
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    assert orc.write_kv(kp, vp, w.dtype, w.k_new, w.v_new, w.slot_mapping) == 0
    return kp, vp


@pytest.mark.parametrize("name,fp8,P", [("batched-decode-small", False, 0), ("batched-decode-small", False, 512),
                                        ("batched-decode-small", True, 0), ("long-decode-small", True, 512),
                                        ("tiny-decode", False, 0), ("tiny-decode", False, 16)])
def test_decode_past_2_31_elements(orc, name, fp8, P):
    w = workload(name)
    if fp8:
        w = W.to_fp8(w)
    d = BigDevice(w)
    kp, vp = oracle_pools(orc, w)
    assert bits_equal(d.top(d.k_pool), kp) and bits_equal(d.top(d.v_pool), vp), "pa_write_kv"
    S, H = w.num_seqs, w.num_heads
    out = torch.full((S, H, w.dv), float("nan"), device="cuda")
    ws = (None, None, None)
    if P:
        pm = -(-int(w.seq_lens.max()) // P)
        ws = tuple(torch.full(sh, float("nan"), device="cuda") for sh in ((S, H, pm), (S, H, pm), (S, H, pm, w.dv)))
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_decode(d.k_pool, d.v_pool, d.q, out, d.tables, d.seq_lens, w.scale, sliding_window=w.sliding_window,
              partition_size=P, max_logits=ws[0], exp_sums=ws[1], tmp_out=ws[2], status=status, k_scale=w.k_scale,
              v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    st, ref, _ = orc.decode(kp, vp, w.dtype, w.q, w.query_dtype, w.block_tables, w.seq_lens, w.scale,
                            sliding_window=w.sliding_window, threads=threads(), k_scale=w.k_scale,
                            v_scale=w.v_scale)
    assert st == 0
    assert_close(host(out), ref, TOL[w.dtype], f"{w.name} P={P}")
    d.free()


def test_varlen_past_2_31_elements(orc):
    """Prefill tiles (the kernel forms 32-bit pool rows and 64-bit byte offsets) and
    the single-token rows of the mixed workload."""
    w = workload("mixed-varlen-small")
    d = BigDevice(w)
    kp, vp = oracle_pools(orc, w)
    T, H = w.num_tokens, w.num_heads
    out = torch.full((T, H, w.dv), float("nan"), device="cuda")
    lse = torch.full((H, T), float("nan"), device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    max_q = int(np.diff(w.query_start_loc).max())
    pa_varlen(d.k_pool, d.v_pool, d.q, out, d.qsl, d.seq_lens, d.positions, d.tables, max_q, w.scale, causal=True,
              sliding_window=w.sliding_window, lse=lse, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    st, ref, rlse = orc.varlen(kp, vp, w.dtype, w.q, w.dtype, w.query_start_loc, w.seq_lens, w.positions,
                               w.block_tables, w.scale, True, w.sliding_window, threads=threads())
    assert st == 0
    assert_close(host(out), ref, TOL[w.dtype], "out")
    assert_close(host(lse), rlse, TOL[w.dtype], "lse")
    d.free()


def test_gather_past_2_31_elements(orc):
    """The latent-cache gather with its blocks past 2^31 elements, bit for bit."""
    g = W.latent_gather(small=True)
    nb, b, D = g.cache.shape
    off = offset_blocks(b * D)
    cache = big_pool(g.cache, "bf16", off)
    T = int(g.cu_seq_lens[-1])
    dst = torch.full((T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pa_gather_cache(cache, dst, dev(g.block_tables + off), dev(g.cu_seq_lens), dev(g.token_to_seq), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    st, ref = orc.gather_cache(g.cache, "bf16", g.block_tables, g.cu_seq_lens, g.token_to_seq, None, "bf16", T)
    assert st == 0
    assert bits_equal(host(dst), ref)
    del cache
    torch.cuda.empty_cache()
