"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments with the documented status before
anything is launched (fake device pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import indexer_top_sparse_amd as isa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_decode.h")
FAKE = 0x10000  # 16-byte aligned, never touched on the host


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(sparse_\w+)\s*\(",
                                 text, re.M)))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) >= 10
    lib = ctypes.CDLL(isa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror():
    assert isa.sparse_abi_version() == 2
    L = isa.lib()
    assert L.sparse_strerror(0) == b"ok"
    assert L.sparse_strerror(3) == b"workspace too small"
    assert L.sparse_strerror(99) == b"unknown status"


def _lightning(B=2, n=1000, H=64, D=128):
    a = isa.IndexArgs()
    a.kind, a.batch, a.n = isa.SCORE_LIGHTNING, B, n
    a.n_heads, a.head_dim = H, D
    a.q, a.q_dtype, a.q_stride_b, a.q_stride_h = FAKE, isa.BF16, H * D, D
    a.head_w, a.w_stride_b = FAKE, H
    a.keys, a.k_dtype, a.k_stride_b, a.k_stride_t = FAKE, isa.E4M3FN, n * D, D
    a.k_scale, a.ks_stride_b = FAKE, n
    a.block_size = 1
    return a


def _mla_attn(B=2, n=1000):
    a = isa.AttnArgs()
    a.batch, a.n, a.n_q_heads, a.n_kv_heads = B, n, 128, 1
    a.d_qk, a.d_v, a.dtype = 576, 512, isa.BF16
    a.q, a.q_stride_b, a.q_stride_h = FAKE, 128 * 576, 576
    a.k_cache, a.kv_stride_t = FAKE, 576
    a.page_table, a.pt_stride_b, a.page_size = FAKE, (n + 63) // 64, 64
    a.sm_scale = 576 ** -0.5
    return a


def _rc(fn, *args):
    return fn(*args)


def test_workspace_size_and_monotone():
    L = isa.lib()
    out = ctypes.c_size_t()
    ia, aa = _lightning(), _mla_attn()
    assert L.sparse_workspace_size(ctypes.byref(ia), ctypes.byref(aa), 256,
                                   ctypes.byref(out)) == 0
    small = out.value
    ia2 = _lightning(B=4)
    aa2 = _mla_attn(B=4)
    assert L.sparse_workspace_size(ctypes.byref(ia2), ctypes.byref(aa2), 256,
                                   ctypes.byref(out)) == 0
    assert out.value > small > 0
    # index-only workspace is smaller than the fused one
    assert L.sparse_workspace_size(ctypes.byref(ia), None, 256, ctypes.byref(out)) == 0
    assert out.value < small
    assert isa.sparse_topk_workspace_size(32, 131072, 2048) > 32 * 131072 * 8


def test_index_validation_codes():
    L = isa.lib()
    out = ctypes.c_size_t()
    a = _lightning()
    a.head_dim = 64
    assert L.sparse_workspace_size(ctypes.byref(a), None, 1, ctypes.byref(out)) == \
        isa.SPARSE_EUNSUPPORTED
    a = _lightning()
    a.n_heads = 48
    assert L.sparse_index_score(ctypes.byref(a), FAKE, None, 0, None) == \
        isa.SPARSE_EUNSUPPORTED
    a = _lightning()
    a.q = FAKE + 4  # misaligned
    assert L.sparse_index_score(ctypes.byref(a), FAKE, None, 0, None) == isa.SPARSE_EINVAL
    a = _lightning()
    a.kind = 7
    assert L.sparse_index_score(ctypes.byref(a), FAKE, None, 0, None) == isa.SPARSE_EINVAL
    assert L.sparse_index_score(None, FAKE, None, 0, None) == isa.SPARSE_EINVAL
    a = _lightning()
    a.kind, a.k_dtype, a.q_dtype = isa.SCORE_DOT, isa.F32, isa.BF16
    assert L.sparse_index_score(ctypes.byref(a), FAKE, None, 0, None) == \
        isa.SPARSE_EUNSUPPORTED
    a.k_dtype, a.q_dtype, a.block_size = isa.BF16, isa.BF16, 32
    assert L.sparse_index_score(ctypes.byref(a), FAKE, None, 0, None) == \
        isa.SPARSE_EUNSUPPORTED
    # bit budget beyond 4 planes x D
    a = _lightning()
    a.kind, a.n_heads, a.n_kv_heads = isa.SCORE_BITPLANE, 32, 8
    a.planes = a.chan_zero = a.chan_scale = a.chan_var = FAKE
    a.bit_budget = 513
    assert L.sparse_index_score(ctypes.byref(a), FAKE, FAKE, 1 << 30, None) == \
        isa.SPARSE_EINVAL
    a.bit_budget, a.n_heads = 92, 30  # 30 % 8 != 0
    assert L.sparse_index_score(ctypes.byref(a), FAKE, FAKE, 1 << 30, None) == \
        isa.SPARSE_EINVAL
    # fixed read depths are for the bit-plane scan only
    a = _lightning()
    a.depth_in = FAKE
    assert L.sparse_index_score(ctypes.byref(a), FAKE, None, 0, None) == isa.SPARSE_EINVAL
    # with fixed depths the variances may be absent; without them they may not
    a = _lightning()
    a.kind, a.n_heads, a.n_kv_heads, a.bit_budget = isa.SCORE_BITPLANE, 32, 8, 92
    a.planes = a.chan_zero = a.chan_scale = FAKE
    a.chan_var = None
    assert L.sparse_index_score(ctypes.byref(a), FAKE, FAKE, 1 << 30, None) == \
        isa.SPARSE_EINVAL
    assert L.sparse_abi_version() == 2
    # at most 4194304 tokens per request
    a = _lightning(n=(1 << 22) + 1)
    assert L.sparse_workspace_size(ctypes.byref(a), None, 1, ctypes.byref(out)) == \
        isa.SPARSE_EUNSUPPORTED
    # the fp8 scan addresses one request's keys with 32-bit byte offsets:
    # padded rows that take a request past 2^31 bytes are refused
    a = _lightning(n=1 << 22)
    a.k_stride_t = 512  # 2 GiB of keys per request
    assert L.sparse_workspace_size(ctypes.byref(a), None, 1, ctypes.byref(out)) == \
        isa.SPARSE_EUNSUPPORTED
    a.k_stride_t = 496  # below 2^31 bytes
    assert L.sparse_workspace_size(ctypes.byref(a), None, 1, ctypes.byref(out)) == isa.SPARSE_OK
    # empty batch: nothing to do, nothing launched
    a = _lightning(B=0)
    assert L.sparse_index_score(ctypes.byref(a), None, None, 0, None) == isa.SPARSE_OK


def test_topk_validation_codes():
    L = isa.lib()
    assert L.sparse_topk(FAKE, 4, 100, 100, None, 1, 0, FAKE, None, FAKE, 1 << 20,
                         None) == isa.SPARSE_EINVAL  # k = 0
    assert L.sparse_topk(FAKE, 4, 100, 50, None, 1, 8, FAKE, None, FAKE, 1 << 20,
                         None) == isa.SPARSE_EINVAL  # row_stride < n_units
    assert L.sparse_topk(FAKE, 4, 100, 100, None, 1, 8, FAKE, None, FAKE, 16,
                         None) == isa.SPARSE_EWORKSPACE
    assert L.sparse_topk(FAKE, 4, 5000000, 5000000, None, 1, 8, FAKE, None, FAKE,
                         1 << 30, None) == isa.SPARSE_EUNSUPPORTED
    assert L.sparse_topk(FAKE, 0, 100, 100, None, 1, 8, None, None, None, 0,
                         None) == isa.SPARSE_OK  # no rows


def test_attention_validation_codes():
    L = isa.lib()
    a = _mla_attn()
    assert L.sparse_gather_attn_decode(ctypes.byref(a), FAKE, 1, 0, 1, FAKE, None,
                                       FAKE, 1 << 30, None) == isa.SPARSE_EINVAL
    assert L.sparse_gather_attn_decode(ctypes.byref(a), FAKE, 1, 16, 3, FAKE, None,
                                       FAKE, 1 << 30, None) == isa.SPARSE_EUNSUPPORTED
    assert L.sparse_gather_attn_decode(ctypes.byref(a), FAKE, 2, 16, 1, FAKE, None,
                                       FAKE, 1 << 30, None) == isa.SPARSE_EINVAL
    a.d_v = 256
    assert L.sparse_gather_attn_decode(ctypes.byref(a), FAKE, 1, 16, 1, FAKE, None,
                                       FAKE, 1 << 30, None) == isa.SPARSE_EUNSUPPORTED
    a = _mla_attn()
    a.n_q_heads = 96  # not a multiple of 64
    assert L.sparse_gather_attn_decode(ctypes.byref(a), FAKE, 1, 16, 1, FAKE, None,
                                       FAKE, 1 << 30, None) == isa.SPARSE_EUNSUPPORTED
    a = _mla_attn()
    assert L.sparse_gather_attn_decode(ctypes.byref(a), FAKE, 1, 2048, 1, FAKE, None,
                                       FAKE, 16, None) == isa.SPARSE_EWORKSPACE
    msg = L.sparse_last_error()
    assert b"workspace" in msg


def test_decode_step_consistency_codes():
    L = isa.lib()
    ia, aa = _lightning(B=2), _mla_attn(B=3)
    assert L.sparse_decode_step(ctypes.byref(ia), ctypes.byref(aa), 16, FAKE, FAKE,
                                None, FAKE, 1 << 30, None) == isa.SPARSE_EINVAL
    ia, aa = _lightning(B=2), _mla_attn(B=2)
    assert L.sparse_decode_step(ctypes.byref(ia), ctypes.byref(aa), 16, FAKE, FAKE,
                                None, FAKE, 64, None) == isa.SPARSE_EWORKSPACE


def test_append_validation_codes():
    L = isa.lib()
    assert L.sparse_append_token(None, None, FAKE, FAKE, FAKE, None, None) == isa.SPARSE_EINVAL
    a = _lightning()
    a.head_dim = 64
    assert L.sparse_append_token(ctypes.byref(a), None, FAKE, FAKE, None, None, None) == \
        isa.SPARSE_EUNSUPPORTED
    a = _lightning()
    assert L.sparse_append_token(ctypes.byref(a), None, None, FAKE, None, None, None) == \
        isa.SPARSE_EINVAL  # pos NULL
    assert L.sparse_append_token(ctypes.byref(a), None, FAKE, None, None, None, None) == \
        isa.SPARSE_EINVAL  # new key NULL
    a.k_dtype = isa.BF16
    assert L.sparse_append_token(ctypes.byref(a), None, FAKE, FAKE, None, None, None) == \
        isa.SPARSE_EINVAL  # lightning keys must be e4m3fn
    a = _lightning(B=0)
    assert L.sparse_append_token(ctypes.byref(a), None, None, None, None, None, None) == \
        isa.SPARSE_OK


def _hot_attn(B=2, n=1000):
    a = _mla_attn(B, n)
    a.k_cache, a.page_table, a.pt_stride_b, a.page_size = None, None, 0, 0
    a.hot_slot, a.hs_stride_b = FAKE, n
    a.hot_kv, a.hot_stride_b, a.hot_stride_s = FAKE, 64 * 576, 576
    a.host_kv, a.host_stride_b, a.host_stride_t = FAKE, n * 576, 576
    return a


def test_hot_update_validation_codes():
    L = isa.lib()
    big = 1 << 30
    a = _hot_attn()
    ok = (FAKE, 16, 1, 64, 3, FAKE, FAKE, FAKE, big, None)
    # no hot buffer in the arguments
    assert L.sparse_hot_update(None, ctypes.byref(_mla_attn()), *ok) == isa.SPARSE_EINVAL
    # slot count, step and selection size limits
    assert L.sparse_hot_update(None, ctypes.byref(a), FAKE, 16, 1, 0, 3, FAKE, FAKE, FAKE,
                               big, None) == isa.SPARSE_EUNSUPPORTED
    assert L.sparse_hot_update(None, ctypes.byref(a), FAKE, 16, 1, 8193, 3, FAKE, FAKE, FAKE,
                               big, None) == isa.SPARSE_EUNSUPPORTED
    assert L.sparse_hot_update(None, ctypes.byref(a), FAKE, 16, 1, 64, -1, FAKE, FAKE, FAKE,
                               big, None) == isa.SPARSE_EINVAL
    assert L.sparse_hot_update(None, ctypes.byref(a), FAKE, 4097, 1, 64, 3, FAKE, FAKE, FAKE,
                               big, None) == isa.SPARSE_EUNSUPPORTED
    # NULL state, too small a workspace, a unit that differs from the index's
    assert L.sparse_hot_update(None, ctypes.byref(a), FAKE, 16, 1, 64, 3, None, FAKE, FAKE,
                               big, None) == isa.SPARSE_EINVAL
    assert L.sparse_hot_update(None, ctypes.byref(a), FAKE, 16, 1, 64, 3, FAKE, FAKE, FAKE,
                               16, None) == isa.SPARSE_EWORKSPACE
    ia = _lightning()
    assert L.sparse_hot_update(ctypes.byref(ia), ctypes.byref(a), FAKE, 16, 64, 64, 3, FAKE,
                               FAKE, FAKE, big, None) == isa.SPARSE_EINVAL
    # an empty batch is a no-op
    assert L.sparse_hot_update(None, ctypes.byref(_hot_attn(B=0)), *ok) == isa.SPARSE_OK


def test_hot_prefetch_validation_codes():
    L = isa.lib()
    a = _hot_attn()
    f = L.sparse_hot_prefetch
    # no hot buffer, no candidates, too many candidates
    assert f(ctypes.byref(_mla_attn()), FAKE, 16, 64, 3, FAKE, FAKE, None) == isa.SPARSE_EINVAL
    assert f(ctypes.byref(a), FAKE, 0, 64, 3, FAKE, FAKE, None) == isa.SPARSE_EINVAL
    assert f(ctypes.byref(a), FAKE, 4097, 64, 3, FAKE, FAKE, None) == isa.SPARSE_EUNSUPPORTED
    # slot count and step limits
    assert f(ctypes.byref(a), FAKE, 16, 0, 3, FAKE, FAKE, None) == isa.SPARSE_EUNSUPPORTED
    assert f(ctypes.byref(a), FAKE, 16, 8193, 3, FAKE, FAKE, None) == isa.SPARSE_EUNSUPPORTED
    assert f(ctypes.byref(a), FAKE, 16, 64, -1, FAKE, FAKE, None) == isa.SPARSE_EINVAL
    # NULL candidates or state
    assert f(ctypes.byref(a), None, 16, 64, 3, FAKE, FAKE, None) == isa.SPARSE_EINVAL
    assert f(ctypes.byref(a), FAKE, 16, 64, 3, FAKE, None, None) == isa.SPARSE_EINVAL
    # no pinned host KV to read from
    b = _hot_attn()
    b.host_kv = None
    assert f(ctypes.byref(b), FAKE, 16, 64, 3, FAKE, FAKE, None) == isa.SPARSE_EINVAL
    # an empty batch is a no-op
    assert f(ctypes.byref(_hot_attn(B=0)), FAKE, 16, 64, 3, FAKE, FAKE, None) == isa.SPARSE_OK


def test_decode_step_noalloc_checks_before_any_device_call():
    L = isa.lib()
    # above the fixed scratch: 32 requests at 1M tokens need far more than 128 MiB
    ia, aa = _lightning(B=32, n=1 << 20), _mla_attn(B=32, n=1 << 20)
    rc = L.sparse_decode_step_noalloc(ctypes.byref(ia), ctypes.byref(aa), 2048, FAKE, FAKE,
                                      None, None)
    assert rc == isa.SPARSE_EWORKSPACE
    assert b"no-allocation" in L.sparse_last_error()
    # the same argument checks as sparse_decode_step
    ia, aa = _lightning(B=2), _mla_attn(B=3)
    assert L.sparse_decode_step_noalloc(ctypes.byref(ia), ctypes.byref(aa), 16, FAKE, FAKE,
                                        None, None) == isa.SPARSE_EINVAL
    ia, aa = _lightning(B=2), _mla_attn(B=2)
    assert L.sparse_decode_step_noalloc(ctypes.byref(ia), ctypes.byref(aa), 16, None, FAKE,
                                        None, None) == isa.SPARSE_EINVAL
    # an empty batch is a valid no-op
    ia, aa = _lightning(B=0), _mla_attn(B=0)
    assert L.sparse_decode_step_noalloc(ctypes.byref(ia), ctypes.byref(aa), 16, None, None,
                                        None, None) == isa.SPARSE_OK
