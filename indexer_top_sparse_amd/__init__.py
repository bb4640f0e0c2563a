"""Python binding of libsparse_decode (argument marshalling only).

Every step of the decode path runs in the HIP library; this module only
turns torch tensors into the C structs of ``include/sparse_decode.h``,
passes ``data_ptr()`` values and the current HIP stream, and turns error
codes into exceptions.  There is no fallback: if the library is missing or
fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_decode.so")

# enums (mirror of the header)
SPARSE_OK, SPARSE_EINVAL, SPARSE_EUNSUPPORTED, SPARSE_EWORKSPACE, SPARSE_EHIP = range(5)
F32, BF16, E4M3FN = 0, 1, 2
SCORE_DOT, SCORE_LIGHTNING, SCORE_BITPLANE = 0, 1, 2

_i32, _i64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class IndexArgs(ctypes.Structure):
    _fields_ = [
        ("kind", _i32), ("batch", _i32), ("n", _i32), ("seq_lens", _vp),
        ("n_heads", _i32), ("head_dim", _i32),
        ("q", _vp), ("q_dtype", _i32), ("q_stride_b", _i64), ("q_stride_h", _i64),
        ("head_w", _vp), ("w_stride_b", _i64),
        ("keys", _vp), ("k_dtype", _i32), ("k_stride_b", _i64), ("k_stride_t", _i64),
        ("k_scale", _vp), ("ks_stride_b", _i64),
        ("block_size", _i32),
        ("n_kv_heads", _i32), ("planes", _vp), ("chan_zero", _vp),
        ("chan_scale", _vp), ("chan_var", _vp), ("bit_budget", _i32),
        ("depth_in", _vp),
    ]


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("batch", _i32), ("n", _i32), ("seq_lens", _vp),
        ("n_q_heads", _i32), ("n_kv_heads", _i32), ("d_qk", _i32), ("d_v", _i32),
        ("dtype", _i32),
        ("q", _vp), ("q_stride_b", _i64), ("q_stride_h", _i64),
        ("k_cache", _vp), ("v_cache", _vp),
        ("kv_stride_b", _i64), ("kv_stride_t", _i64), ("kv_stride_h", _i64),
        ("page_table", _vp), ("pt_stride_b", _i64), ("page_size", _i32),
        ("sm_scale", _f32),
        ("hot_slot", _vp), ("hs_stride_b", _i64),
        ("hot_kv", _vp), ("hot_stride_b", _i64), ("hot_stride_s", _i64),
        ("host_kv", _vp), ("host_stride_b", _i64), ("host_stride_t", _i64),
    ]


class SparseError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it is not built or cannot load."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m indexer_top_sparse_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.sparse_abi_version.restype = ctypes.c_int
        L.sparse_strerror.restype = ctypes.c_char_p
        L.sparse_strerror.argtypes = [ctypes.c_int]
        L.sparse_last_error.restype = ctypes.c_char_p
        L.sparse_workspace_size.argtypes = [P(IndexArgs), P(AttnArgs), _i32,
                                            P(ctypes.c_size_t)]
        L.sparse_topk_workspace_size.argtypes = [_i32, _i32, _i32, P(ctypes.c_size_t)]
        L.sparse_read_depth.argtypes = [P(IndexArgs), _vp, _vp]
        L.sparse_index_score.argtypes = [P(IndexArgs), _vp, _vp, ctypes.c_size_t, _vp]
        L.sparse_topk.argtypes = [_vp, _i32, _i32, _i64, _vp, _i32, _i32, _vp, _vp,
                                  _vp, ctypes.c_size_t, _vp]
        L.sparse_gather_attn_decode.argtypes = [P(AttnArgs), _vp, _i32, _i32, _i32,
                                                _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.sparse_decode_step.argtypes = [P(IndexArgs), P(AttnArgs), _i32, _vp, _vp,
                                         _vp, _vp, ctypes.c_size_t, _vp]
        L.sparse_decode_step_noalloc.argtypes = [P(IndexArgs), P(AttnArgs), _i32, _vp, _vp,
                                                 _vp, _vp]
        L.sparse_host_device_pointer.argtypes = [_vp, P(_vp)]
        L.sparse_append_token.argtypes = [P(IndexArgs), P(AttnArgs), _vp, _vp, _vp, _vp, _vp]
        L.sparse_hot_update.argtypes = [P(IndexArgs), P(AttnArgs), _vp, _i32, _i32, _i32,
                                        _i32, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.sparse_hot_prefetch.argtypes = [P(AttnArgs), _vp, _i32, _i32, _i32, _vp, _vp, _vp]
        for f in ("sparse_workspace_size", "sparse_topk_workspace_size",
                  "sparse_read_depth", "sparse_index_score", "sparse_topk",
                  "sparse_gather_attn_decode", "sparse_decode_step",
                  "sparse_decode_step_noalloc",
                  "sparse_host_device_pointer", "sparse_append_token", "sparse_hot_update",
                  "sparse_hot_prefetch"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != SPARSE_OK:
        detail = lib().sparse_last_error().decode()
        raise SparseError(rc, f"{lib().sparse_strerror(rc).decode()}: {detail}")


def _p(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None) -> int | None:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.uint8: E4M3FN,
       torch.float8_e4m3fn: E4M3FN}


class _Holder:
    """Keeps the tensors behind a C struct's raw pointers alive."""

    def __init__(self, struct, *tensors):
        self.c = struct
        self.refs = tensors

    def ref(self):
        return ctypes.byref(self.c)


# ------------------------------------------------------------ arg builders
def dot_index_args(q: torch.Tensor, keys: torch.Tensor, block_size: int = 1,
                   seq_lens: torch.Tensor | None = None) -> _Holder:
    """Head-summed dot index.  q [B][H][D], keys [B][n][D] (any row strides)."""
    a = IndexArgs()
    a.kind = SCORE_DOT
    a.batch, a.n = keys.shape[0], keys.shape[1]
    a.seq_lens = _p(seq_lens)
    a.n_heads, a.head_dim = q.shape[1], q.shape[2]
    a.q, a.q_dtype = _p(q), _DT[q.dtype]
    a.q_stride_b, a.q_stride_h = q.stride(0), q.stride(1)
    a.keys, a.k_dtype = _p(keys), _DT[keys.dtype]
    a.k_stride_b, a.k_stride_t = keys.stride(0), keys.stride(1)
    a.block_size = block_size
    return _Holder(a, q, keys, seq_lens)


def lightning_index_args(q: torch.Tensor, head_w: torch.Tensor, k8: torch.Tensor,
                         k_scale: torch.Tensor,
                         seq_lens: torch.Tensor | None = None) -> _Holder:
    """Lightning indexer.  q [B][H][D] bf16, head_w [B][H] fp32, k8 [B][n][D]
    e4m3fn bytes, k_scale [B][n] fp32."""
    a = IndexArgs()
    a.kind = SCORE_LIGHTNING
    a.batch, a.n = k8.shape[0], k8.shape[1]
    a.seq_lens = _p(seq_lens)
    a.n_heads, a.head_dim = q.shape[1], q.shape[2]
    a.q, a.q_dtype = _p(q), _DT[q.dtype]
    a.q_stride_b, a.q_stride_h = q.stride(0), q.stride(1)
    a.head_w, a.w_stride_b = _p(head_w), head_w.stride(0)
    a.keys, a.k_dtype = _p(k8), E4M3FN
    a.k_stride_b, a.k_stride_t = k8.stride(0), k8.stride(1)
    a.k_scale, a.ks_stride_b = _p(k_scale), k_scale.stride(0)
    a.block_size = 1
    return _Holder(a, q, head_w, k8, k_scale, seq_lens)


def bitplane_index_args(q: torch.Tensor, planes: torch.Tensor,
                        chan_zero: torch.Tensor, chan_scale: torch.Tensor,
                        chan_var: torch.Tensor | None, bit_budget: int, n: int,
                        seq_lens: torch.Tensor | None = None,
                        depth_in: torch.Tensor | None = None) -> _Holder:
    """Fathom scan.  q [B][Hq][D] bf16, planes [B][Hkv][D][4][ceil(n/32)]
    (int32/uint32 bit words; a pinned host tensor is read in place through
    its device alias), chan_* [B][Hkv][D] fp32, depth_in (optional) [B][Hkv][D]
    int8 fixed read depths."""
    for t in (planes, chan_zero, chan_scale, chan_var, depth_in):
        if t is not None and not t.is_contiguous():
            raise ValueError("planes and channel tensors must be contiguous")
    a = IndexArgs()
    a.kind = SCORE_BITPLANE
    a.batch, a.n = q.shape[0], n
    a.seq_lens = _p(seq_lens)
    a.n_heads, a.head_dim = q.shape[1], q.shape[2]
    a.q, a.q_dtype = _p(q), _DT[q.dtype]
    a.q_stride_b, a.q_stride_h = q.stride(0), q.stride(1)
    a.block_size = 1
    a.n_kv_heads = planes.shape[1]
    a.planes = host_device_pointer(planes) if planes.device.type == "cpu" else _p(planes)
    a.chan_zero = _p(chan_zero)
    a.chan_scale, a.chan_var = _p(chan_scale), _p(chan_var)
    a.bit_budget = bit_budget
    a.depth_in = _p(depth_in)
    return _Holder(a, q, planes, chan_zero, chan_scale, chan_var, seq_lens, depth_in)


def attn_args(q: torch.Tensor, k_cache: torch.Tensor | None,
              v_cache: torch.Tensor | None = None, *, n: int, d_v: int,
              sm_scale: float,
              page_table: torch.Tensor | None = None, page_size: int = 0,
              seq_lens: torch.Tensor | None = None,
              hot_slot: torch.Tensor | None = None,
              hot_kv: torch.Tensor | None = None,
              host_kv: torch.Tensor | None = None) -> _Holder:
    """Sparse attention arguments.

    q [B][Hq][d_qk].  k_cache / v_cache: [B][n][Hkv][d] contiguous-per-request
    caches, or (latent, v_cache None) [B][n][d_qk], or with a page table a
    pool [pages][page_size][d_qk] (or [pages][page_size][Hkv][d]).  Hot
    buffer: hot_slot [B][n] int32, hot_kv [B][slots][d_qk], host_kv pinned
    [B][n][d_qk] (its device alias is looked up here).  d_v (the value
    width; latent rows use their first d_v elements as the value) and
    sm_scale (the softmax scale) are the caller's: nothing is inferred."""
    a = AttnArgs()
    B, Hq, dqk = q.shape
    a.batch, a.n, a.seq_lens = B, n, _p(seq_lens)
    a.n_q_heads, a.d_qk, a.d_v = Hq, dqk, d_v
    a.sm_scale = sm_scale
    a.dtype = _DT[q.dtype]
    a.q, a.q_stride_b, a.q_stride_h = _p(q), q.stride(0), q.stride(1)
    refs = [q, k_cache, v_cache, page_table, seq_lens, hot_slot, hot_kv, host_kv]
    latent = v_cache is None
    if hot_slot is not None:
        a.n_kv_heads = 1
        a.hot_slot, a.hs_stride_b = _p(hot_slot), hot_slot.stride(0)
        a.hot_kv, a.hot_stride_b, a.hot_stride_s = _p(hot_kv), hot_kv.stride(0), hot_kv.stride(1)
        dev = host_device_pointer(host_kv)
        a.host_kv, a.host_stride_b, a.host_stride_t = dev, host_kv.stride(0), host_kv.stride(1)
    elif latent:
        a.n_kv_heads = 1
        a.k_cache = _p(k_cache)
        if page_table is not None:
            a.kv_stride_t = k_cache.stride(-2)
        else:
            a.kv_stride_b, a.kv_stride_t = k_cache.stride(0), k_cache.stride(1)
    else:
        a.n_kv_heads = k_cache.shape[-2]
        if v_cache.shape[-1] != d_v:
            raise ValueError(f"v_cache rows hold {v_cache.shape[-1]} values, d_v is {d_v}")
        if v_cache.stride() != k_cache.stride():
            raise ValueError("k_cache and v_cache must share strides")
        a.k_cache, a.v_cache = _p(k_cache), _p(v_cache)
        if page_table is not None:
            a.kv_stride_t, a.kv_stride_h = k_cache.stride(-3), k_cache.stride(-2)
        else:
            a.kv_stride_b, a.kv_stride_t, a.kv_stride_h = (
                k_cache.stride(0), k_cache.stride(1), k_cache.stride(2))
    if page_table is not None:
        a.page_table, a.pt_stride_b, a.page_size = (
            _p(page_table), page_table.stride(0), page_size)
    return _Holder(a, *refs)


# ------------------------------------------------------------- entry points
def sparse_abi_version() -> int:
    return lib().sparse_abi_version()


def sparse_workspace_size(ia: _Holder | None, aa: _Holder | None, k: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().sparse_workspace_size(ia.ref() if ia else None,
                                       aa.ref() if aa else None, k, ctypes.byref(out)))
    return out.value


def sparse_topk_workspace_size(rows: int, n_units: int, k: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().sparse_topk_workspace_size(rows, n_units, k, ctypes.byref(out)))
    return out.value


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A workspace buffer (uint8, 256-byte aligned by the torch allocator)."""
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def sparse_read_depth(ia: _Holder, depth_out: torch.Tensor, stream=None) -> None:
    _check(lib().sparse_read_depth(ia.ref(), _p(depth_out), _stream(stream)))


def sparse_index_score(ia: _Holder, scores: torch.Tensor, ws: torch.Tensor | None,
                       stream=None) -> None:
    _check(lib().sparse_index_score(ia.ref(), _p(scores), _p(ws),
                                    ws.numel() if ws is not None else 0, _stream(stream)))


def sparse_topk(scores: torch.Tensor, k: int, idx_out: torch.Tensor,
                val_out: torch.Tensor | None = None,
                valid_units: torch.Tensor | None = None, rows_per_valid: int = 1,
                ws: torch.Tensor | None = None, stream=None) -> None:
    """scores [rows][n_units] fp32 (row stride from the tensor)."""
    rows, n_units = scores.shape
    _check(lib().sparse_topk(_p(scores), rows, n_units, scores.stride(0),
                             _p(valid_units), rows_per_valid, k, _p(idx_out),
                             _p(val_out), _p(ws), ws.numel() if ws is not None else 0,
                             _stream(stream)))


def sparse_gather_attn_decode(aa: _Holder, sel: torch.Tensor, sel_heads: int, k: int,
                              sel_unit: int, out: torch.Tensor,
                              lse: torch.Tensor | None, ws: torch.Tensor | None,
                              stream=None) -> None:
    _check(lib().sparse_gather_attn_decode(
        aa.ref(), _p(sel), sel_heads, k, sel_unit, _p(out), _p(lse), _p(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))


def sparse_decode_step(ia: _Holder, aa: _Holder, k: int, topk_out: torch.Tensor,
                       out: torch.Tensor, lse: torch.Tensor | None,
                       ws: torch.Tensor, stream=None) -> None:
    _check(lib().sparse_decode_step(ia.ref(), aa.ref(), k, _p(topk_out), _p(out),
                                    _p(lse), _p(ws), ws.numel(), _stream(stream)))


def sparse_decode_step_noalloc(ia: _Holder, aa: _Holder, k: int, topk_out: torch.Tensor,
                               out: torch.Tensor, lse: torch.Tensor | None,
                               stream=None) -> None:
    """sparse_decode_step with its scratch in the library's fixed device
    array instead of a caller workspace (no allocation anywhere)."""
    _check(lib().sparse_decode_step_noalloc(ia.ref(), aa.ref(), k, _p(topk_out), _p(out),
                                            _p(lse), _stream(stream)))


def sparse_append_token(ia: _Holder | None, aa: _Holder | None, pos: torch.Tensor,
                        index_key_new: torch.Tensor | None, k_new: torch.Tensor | None,
                        v_new: torch.Tensor | None = None, stream=None) -> None:
    """Append each request's new token (at position pos[b]) to the structures
    the next step reads: the KV rows of `aa`'s layout (k_new [B][Hkv][d_qk],
    v_new [B][Hkv][d_v] when V is separate) and the index entry of `ia`'s kind
    from the fp32 key index_key_new ([B][D], or [B][Hkv][D] for bit planes)."""
    for t in (pos, index_key_new, k_new, v_new):
        if t is not None and not t.is_contiguous():
            raise ValueError("append inputs must be contiguous")
    _check(lib().sparse_append_token(ia.ref() if ia is not None else None,
                                     aa.ref() if aa is not None else None,
                                     _p(pos), _p(index_key_new), _p(k_new), _p(v_new),
                                     _stream(stream)))


def sparse_hot_update(ia: _Holder | None, aa: _Holder, sel: torch.Tensor, k: int,
                      sel_unit: int, n_slots: int, step: int, slot_token: torch.Tensor,
                      slot_stamp: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    """Least-recently-used replacement in the hot buffer of `aa` after the
    step (sparse_decode_step with `ia`, or sparse_gather_attn_decode with
    ia None) that selected `sel` and staged its misses in `ws`.  slot_token
    and slot_stamp: [B][n_slots] int32, updated with aa's hot_slot / hot_kv."""
    for t in (sel, slot_token, slot_stamp):
        if not t.is_contiguous() or t.dtype != torch.int32:
            raise ValueError("sel / slot_token / slot_stamp must be contiguous int32")
    _check(lib().sparse_hot_update(ia.ref() if ia is not None else None, aa.ref(), _p(sel),
                                   k, sel_unit, n_slots, step, _p(slot_token),
                                   _p(slot_stamp), _p(ws), ws.numel(), _stream(stream)))


def sparse_hot_prefetch(aa: _Holder, cand: torch.Tensor, m: int, n_slots: int, step: int,
                        slot_token: torch.Tensor, slot_stamp: torch.Tensor,
                        stream=None) -> None:
    """Preload the non-resident tokens of `cand` ([B][m] int32, -1 padding)
    into the hot buffer of `aa`, least recently used slots first, never
    replacing a slot stamped `step` or a resident candidate; rows come from
    aa's pinned host KV.  slot_token / slot_stamp as for sparse_hot_update."""
    for t in (cand, slot_token, slot_stamp):
        if not t.is_contiguous() or t.dtype != torch.int32:
            raise ValueError("cand / slot_token / slot_stamp must be contiguous int32")
    _check(lib().sparse_hot_prefetch(aa.ref(), _p(cand), m, n_slots, step, _p(slot_token),
                                     _p(slot_stamp), _stream(stream)))


def host_device_pointer(host: torch.Tensor) -> int:
    if not host.is_pinned():
        raise ValueError("host tensor must be pinned host memory")
    dev = ctypes.c_void_p(0)
    _check(lib().sparse_host_device_pointer(_p(host), ctypes.byref(dev)))
    return dev.value
