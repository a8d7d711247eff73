"""The C-ABI library without a GPU: it loads, exports every function include/pa.h
declares, and refuses bad arguments synchronously (these checks run on the host
before any HIP call, so they need no device)."""
import ctypes
import os
import re

import pytest

from paged_kv_attention_table_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(pa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("pa_write_kv", "pa_decode", "pa_decode_noalloc", "pa_varlen", "pa_varlen_merge", "pa_varlen_ctx_new",
              "pa_merge_states", "pa_gather_cache", "pa_strerror"):
        assert n in names, names


def test_library_exports_every_declared_symbol():
    lib = binding.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(binding.EXPORTS)


def test_strerror_texts():
    for code in range(6):
        assert binding.strerror(code) != "unknown status"
    assert binding.strerror(99) == "unknown status"


def _pool(**kw):
    d = dict(k=0x1000, v=0x2000, num_blocks=4, block_size=16, num_kv_heads=2, head_dim_k=64, head_dim_v=64,
             dtype=binding.PA_F16, k_scale=1.0, v_scale=1.0)
    d.update(kw)
    return binding.PaKvPool(d["k"], d["v"], d["num_blocks"], d["block_size"], d["num_kv_heads"], d["head_dim_k"],
                            d["head_dim_v"], d["dtype"], d["k_scale"], d["v_scale"])


FAKE = ctypes.c_void_p(0x3000)  # never dereferenced: every case below fails before any launch


@pytest.mark.parametrize("pool,H,expect", [
    (None, 4, binding.PA_EINVAL),
    (dict(k=0), 4, binding.PA_EINVAL),
    (dict(num_blocks=0), 4, binding.PA_EINVAL),
    (dict(dtype=7), 4, binding.PA_EUNSUPPORTED),
    ({}, 3, binding.PA_ESHAPE),
    (dict(head_dim_k=64, head_dim_v=32), 4, binding.PA_EUNSUPPORTED),
    (dict(head_dim_k=48, head_dim_v=48), 4, binding.PA_EUNSUPPORTED),
    ({}, 2 * 17, binding.PA_EUNSUPPORTED),
])
def test_decode_host_checks(pool, H, expect):
    lib = binding.load()
    p = None if pool is None else ctypes.byref(_pool(**pool))
    st = lib.pa_decode(p, FAKE, binding.PA_F16, FAKE, binding.PA_F32, FAKE, 4, FAKE, 2, H, 0.1, 0, 0, 0, None,
                       None, None, None, None, None, None)
    assert st == expect


def test_decode_partition_checks():
    lib = binding.load()
    p = ctypes.byref(_pool())
    args = lambda P, pmax, ws: (p, FAKE, binding.PA_F16, FAKE, binding.PA_F32, FAKE, 4, FAKE, 2, 4, 0.1, 0, P, pmax,
                                ws, ws, ws, None, None, None, None)
    assert lib.pa_decode(*args(24, 4, FAKE)) == binding.PA_EINVAL      # not a multiple of the block size
    assert lib.pa_decode(*args(32, 0, FAKE)) == binding.PA_EINVAL      # no partitions
    assert lib.pa_decode(*args(32, 4, None)) == binding.PA_EINVAL      # missing workspace
    assert lib.pa_decode(*args(-16, 4, FAKE)) == binding.PA_EINVAL
    # q dtype must match the pool, out must be f32 or q's dtype
    assert lib.pa_decode(p, FAKE, binding.PA_BF16, FAKE, binding.PA_F32, FAKE, 4, FAKE, 2, 4, 0.1, 0, 0, 0, None,
                         None, None, None, None, None, None) == binding.PA_EUNSUPPORTED
    assert lib.pa_decode(p, FAKE, binding.PA_F16, FAKE, binding.PA_BF16, FAKE, 4, FAKE, 2, 4, 0.1, 0, 0, 0, None,
                         None, None, None, None, None, None) == binding.PA_EUNSUPPORTED


def test_varlen_host_checks():
    lib = binding.load()
    p = ctypes.byref(_pool())
    # causal without positions
    assert lib.pa_varlen(p, FAKE, binding.PA_F16, FAKE, binding.PA_F32, None, FAKE, FAKE, None, FAKE, 4, 2, 10, 8,
                         4, 0.1, 1, 0, 0, 0, None, None, None, None, None, None, None) == binding.PA_EINVAL
    # no query_start_loc
    assert lib.pa_varlen(p, FAKE, binding.PA_F16, FAKE, binding.PA_F32, None, None, FAKE, FAKE, FAKE, 4, 2, 10, 8,
                         4, 0.1, 1, 0, 0, 0, None, None, None, None, None, None, None) == binding.PA_EINVAL
    # tokens but no sequences
    assert lib.pa_varlen(p, FAKE, binding.PA_F16, FAKE, binding.PA_F32, None, FAKE, FAKE, FAKE, FAKE, 4, 0, 10, 8,
                         4, 0.1, 1, 0, 0, 0, None, None, None, None, None, None, None) == binding.PA_EINVAL
    assert lib.pa_varlen(p, FAKE, binding.PA_F16, FAKE, binding.PA_F32, None, FAKE, FAKE, FAKE, FAKE, 4, 2, 10, 8,
                         5, 0.1, 1, 0, 0, 0, None, None, None, None, None, None, None) == binding.PA_ESHAPE


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan")])
def test_scale_must_be_positive_and_finite(scale):
    lib = binding.load()
    p = ctypes.byref(_pool())
    assert lib.pa_decode(p, FAKE, binding.PA_F16, FAKE, binding.PA_F32, FAKE, 4, FAKE, 2, 4, scale, 0, 0, 0, None,
                         None, None, None, None, None, None) == binding.PA_EINVAL
    assert lib.pa_varlen(p, FAKE, binding.PA_F16, FAKE, binding.PA_F32, None, FAKE, FAKE, FAKE, FAKE, 4, 2, 10, 8,
                         4, scale, 1, 0, 0, 0, None, None, None, None, None, None, None) == binding.PA_EINVAL


def test_write_and_merge_host_checks():
    lib = binding.load()
    p = ctypes.byref(_pool())
    assert lib.pa_write_kv(p, FAKE, FAKE, FAKE, -1, None, None) == binding.PA_EINVAL
    assert lib.pa_write_kv(p, None, FAKE, FAKE, 3, None, None) == binding.PA_EINVAL
    assert lib.pa_write_kv(ctypes.byref(_pool(head_dim_k=1, head_dim_v=1, num_kv_heads=1)), FAKE, FAKE, FAKE, 3,
                           None, None) == binding.PA_EUNSUPPORTED
    assert lib.pa_merge_states(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 0, 8, -1, 0, None) == binding.PA_EINVAL
    assert lib.pa_merge_states(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 2, 8, -1, 9, None) == binding.PA_EUNSUPPORTED
    assert lib.pa_merge_states(FAKE, None, None, FAKE, FAKE, FAKE, 4, 2, 8, -1, 0, None) == binding.PA_EINVAL


def test_gather_host_checks():
    lib = binding.load()
    ok = (FAKE, binding.PA_BF16, 8, 16, 64, 16 * 64, 64, FAKE, binding.PA_BF16, 64, FAKE, 4, FAKE, FAKE, None, 2, 10,
          None, None)

    def call(change):
        a = list(ok)
        for k, v in change.items():
            a[k] = v
        return lib.pa_gather_cache(*a)

    assert call({1: 7}) == binding.PA_EUNSUPPORTED      # cache dtype
    assert call({8: 9}) == binding.PA_EUNSUPPORTED      # dst dtype
    assert call({16: -1}) == binding.PA_EINVAL          # negative token count
    assert call({2: 0}) == binding.PA_EINVAL            # no blocks
    assert call({6: 63}) == binding.PA_EINVAL           # slot stride below the row
    assert call({9: 32}) == binding.PA_EINVAL           # output rows overlap
    assert call({0: None}) == binding.PA_EINVAL         # no cache
    assert call({13: None}) == binding.PA_EINVAL        # no token_to_seq
    assert call({15: 0}) == binding.PA_EINVAL           # tokens but no sequences


def test_binding_refuses_host_tensors():
    import torch

    t = torch.zeros(2, 2, 2, 2)
    with pytest.raises(TypeError):
        binding.make_pool(t, t)


def _decode(pool, q_dtype=binding.PA_BF16, out_dtype=binding.PA_F32, H=4, scale=0.1):
    return binding.load().pa_decode(ctypes.byref(pool), FAKE, q_dtype, FAKE, out_dtype, FAKE, 4, FAKE, 2, H, scale,
                                    0, 0, 0, None, None, None, None, None, None, None)


def _varlen(pool, q_dtype=binding.PA_BF16, max_query_len=1, scale=0.1):
    return binding.load().pa_varlen(ctypes.byref(pool), FAKE, q_dtype, FAKE, binding.PA_F32, None, FAKE, FAKE, FAKE,
                                    FAKE, 4, 2, 10, max_query_len, 4, scale, 1, 0, 0, 0, None, None, None, None, None, None, None)


FP8 = dict(dtype=binding.PA_FP8_E4M3, head_dim_k=128, head_dim_v=128)


@pytest.mark.parametrize("change,q_dtype,out_dtype,H", [
    ({}, binding.PA_F32, binding.PA_F32, 4),                       # fp8 pools take f16 / bf16 queries
    ({}, binding.PA_FP8_E4M3, binding.PA_F32, 4),                  # ... never fp8 ones
    ({}, binding.PA_BF16, binding.PA_F16, 4),                      # out: f32 or the queries' type
    (dict(head_dim_k=64, head_dim_v=64), binding.PA_BF16, binding.PA_F32, 4),   # head dims 128 only
    (dict(block_size=8), binding.PA_BF16, binding.PA_F32, 4),      # power-of-two blocks of >= 16
    (dict(block_size=48), binding.PA_F16, binding.PA_F32, 4),
    ({}, binding.PA_BF16, binding.PA_F32, 2 * 17),                 # at most 16 q heads per kv head
])
def test_fp8_decode_unsupported(change, q_dtype, out_dtype, H):
    assert _decode(_pool(**{**FP8, **change}), q_dtype, out_dtype, H) == binding.PA_EUNSUPPORTED


def test_fp8_varlen_and_value_types():
    # varlen over an fp8 pool: queries of several tokens on the tiled kernel's fp8 shapes
    # (head dims 128 / 128 or 192 / 128, power-of-two blocks of >= 16) only
    for change in (dict(head_dim_k=64, head_dim_v=64), dict(head_dim_k=256, head_dim_v=256), dict(block_size=8)):
        assert _varlen(_pool(**{**FP8, **change}), max_query_len=2) == binding.PA_EUNSUPPORTED
    assert _varlen(_pool(**FP8), q_dtype=binding.PA_F32) == binding.PA_EUNSUPPORTED
    # the context-and-new-tokens call likewise
    lib = binding.load()
    for change, qd in ((dict(head_dim_k=64, head_dim_v=64), binding.PA_BF16), ({}, binding.PA_F32),
                       ({}, binding.PA_FP8_E4M3)):
        assert lib.pa_varlen_ctx_new(ctypes.byref(_pool(**{**FP8, **change})), FAKE, qd, FAKE, FAKE, 0, FAKE, FAKE,
                                     FAKE, 4, FAKE, FAKE, FAKE, 4, 2, 10, 8, 4, 0.1, None, None,
                                     None) == binding.PA_EUNSUPPORTED
    # a non-fp8 pool still wants queries of its own type
    assert _decode(_pool(dtype=binding.PA_BF16), q_dtype=binding.PA_F16) == binding.PA_EUNSUPPORTED
    lib = binding.load()
    # merged states and gathered latent rows are value types, never fp8
    assert lib.pa_merge_states(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 2, 8, -1, binding.PA_FP8_E4M3,
                               None) == binding.PA_EUNSUPPORTED
    ok = [FAKE, binding.PA_BF16, 8, 16, 64, 16 * 64, 64, FAKE, binding.PA_BF16, 64, FAKE, 4, FAKE, FAKE, None, 2, 10,
          None, None]
    for idx in (1, 8):
        a = list(ok)
        a[idx] = binding.PA_FP8_E4M3
        assert lib.pa_gather_cache(*a) == binding.PA_EUNSUPPORTED


@pytest.mark.parametrize("bad", [0.0, -2.0, float("inf"), float("nan")])
@pytest.mark.parametrize("which", ["k_scale", "v_scale"])
def test_pool_scales_must_be_positive_and_finite(bad, which):
    for pool in (_pool(**{which: bad}), _pool(**FP8, **{which: bad})):
        q = binding.PA_F16 if pool.dtype == binding.PA_F16 else binding.PA_BF16
        assert _decode(pool, q_dtype=q) == binding.PA_EINVAL
        assert _varlen(pool, q_dtype=q) == binding.PA_EINVAL
        assert binding.load().pa_write_kv(ctypes.byref(pool), FAKE, FAKE, FAKE, 3, None, None) == binding.PA_EINVAL


def test_folded_scale_must_stay_finite():
    # scale * k_scale overflows / underflows binary32
    assert _decode(_pool(**FP8, k_scale=1e30), scale=1e30) == binding.PA_EINVAL
    assert _decode(_pool(**FP8, k_scale=1e-30), scale=1e-30) == binding.PA_EINVAL
    assert _varlen(_pool(**FP8, k_scale=1e30), scale=1e30) == binding.PA_EINVAL


def test_varlen_split_host_checks():
    lib = binding.load()
    p = ctypes.byref(_pool())

    def call(P, pmax, ws):
        return lib.pa_varlen(p, FAKE, binding.PA_F16, FAKE, binding.PA_F32, None, FAKE, FAKE, FAKE, FAKE, 4, 2, 10, 8,
                             4, 0.1, 1, 0, P, pmax, ws, ws, ws, None, None, None, None)

    assert call(-16, 4, FAKE) == binding.PA_EINVAL      # negative partition size
    assert call(24, 4, FAKE) == binding.PA_EINVAL       # not a multiple of the block size
    assert call(32, 0, FAKE) == binding.PA_EINVAL       # no partitions
    assert call(32, 4, None) == binding.PA_EINVAL       # missing workspace
    assert call(32, 8193, FAKE) == binding.PA_EUNSUPPORTED


def test_varlen_merge_host_checks():
    lib = binding.load()
    p = ctypes.byref(_pool())
    # the state's lse is required
    assert lib.pa_varlen_merge(p, FAKE, binding.PA_F16, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 2, 10, 8, 4, 0.1, 1, 0,
                               None, None, None, None) == binding.PA_EINVAL
    # the usual pa_varlen checks apply: q dtype, shape, scale
    assert lib.pa_varlen_merge(p, FAKE, binding.PA_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 10, 8, 4, 0.1, 1,
                               0, None, None, None, None) == binding.PA_EUNSUPPORTED
    assert lib.pa_varlen_merge(p, FAKE, binding.PA_F16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 10, 8, 5, 0.1, 1, 0,
                               None, None, None, None) == binding.PA_ESHAPE
    assert lib.pa_varlen_merge(p, FAKE, binding.PA_F16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 10, 8, 4, 0.0, 1, 0,
                               None, None, None, None) == binding.PA_EINVAL


def test_decode_noalloc_host_checks():
    """The static-workspace decode refuses calls whose partition states would not fit
    its buffer (or exceed pa_decode's partition limit) before any HIP call."""
    lib = binding.load()
    big = _pool(num_kv_heads=8, head_dim_k=128, head_dim_v=128)

    def call(pool, S, H, max_blocks, P):
        p = None if pool is None else ctypes.byref(pool)
        return lib.pa_decode_noalloc(p, FAKE, binding.PA_F16, FAKE, binding.PA_F32, FAKE, max_blocks, FAKE, S, H, 0.1,
                                     0, P, None, None, None, None)

    assert call(None, 2, 4, 4, 16) == binding.PA_EINVAL
    assert call(big, 1024, 64, 8192, 16) == binding.PA_ESCRATCH      # 2^29 partition states
    assert call(big, 64, 64, 8192, 512) == binding.PA_ESCRATCH       # 64 * 64 * 256 * 130 * 4 B > 96 MiB
    assert call(big, 2, 64, 8192 * 2, 16) == binding.PA_EUNSUPPORTED  # 16384 partitions (pa_decode's limit: 8192)
    assert call(big, 2, 4, 4, 24) == binding.PA_EINVAL               # not a multiple of the block size
    assert call(big, 2, 4, 4, -16) == binding.PA_EINVAL
    assert binding.strerror(binding.PA_ESCRATCH) != "unknown status"


def test_varlen_ctx_new_host_checks():
    lib = binding.load()
    p = ctypes.byref(_pool(head_dim_k=128, head_dim_v=128))

    def call(**kw):
        a = dict(pool=p, q_dtype=binding.PA_F16, lse=FAKE, merge=0, ctx_lens=FAKE, new_positions=FAKE, ctx_mb=4,
                 new_mb=4, S=2, T=10, H=4, scale=0.1)
        a.update(kw)
        return lib.pa_varlen_ctx_new(a["pool"], FAKE, a["q_dtype"], FAKE, a["lse"], a["merge"], FAKE, a["ctx_lens"],
                                     FAKE, a["ctx_mb"], FAKE, a["new_positions"], FAKE, a["new_mb"], a["S"], a["T"], 8,
                                     a["H"], a["scale"], None, None, None)

    assert call(lse=None) == binding.PA_EINVAL            # the state's lse is required
    assert call(new_positions=None) == binding.PA_EINVAL  # causal new tokens need their positions
    assert call(ctx_lens=None) == binding.PA_EINVAL
    assert call(ctx_mb=0) == binding.PA_EINVAL
    assert call(H=5) == binding.PA_ESHAPE
    assert call(q_dtype=binding.PA_BF16) == binding.PA_EUNSUPPORTED                      # q of the pool's type
    assert call(pool=ctypes.byref(_pool(head_dim_k=32, head_dim_v=32))) == binding.PA_EUNSUPPORTED  # tiled shapes only
    assert call(pool=ctypes.byref(_pool(head_dim_k=128, head_dim_v=128, block_size=8))) == binding.PA_EUNSUPPORTED
    assert call(scale=0.0) == binding.PA_EINVAL
