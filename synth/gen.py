"""Seeded input generation (torch, on any device).

Every tensor draws from its own torch.Generator seeded with
``workload.seed * 1000 + slot`` so that a tensor's values do not depend on the
order other tensors are drawn in, and large tensors are drawn in chunks so the
peak memory stays close to the stored size.

Stored formats (all little-endian, row-major):

* bf16 tensors hold fp32 N(0,1) draws rounded to nearest-even.
* The fp8 K-index holds OCP e4m3fn bytes of k / sigma_t, where
  sigma_t = max_d |k_t,d| / 448 is stored as fp32 (one scale per token).
* The Fathom K cache holds 4-bit codes per (request, KV head, channel):
  zero = min over the tokens, cell = (max - min) / 16 (both stored fp32),
  code = min(floor((k - zero) / cell), 15) evaluated in fp64.  ``codes`` is [B][Hkv][n][D]
  uint8; ``planes`` is [B][Hkv][D][4][ceil(n/32)] uint32 where plane j holds
  bit (3 - j) of the code (most significant plane first) and bit i of word w
  belongs to token 32*w + i.  Words past n are zero.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .workloads import Workload

_CHUNK = 1 << 24  # elements per randn call for big tensors


def _gen(w: Workload, slot: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + slot)
    return g


def _randn(shape, g, device, dtype=torch.float32) -> torch.Tensor:
    """N(0,1) draws converted to `dtype` chunk by chunk."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    total = flat.numel()
    for lo in range(0, total, _CHUNK):
        hi = min(total, lo + _CHUNK)
        flat[lo:hi] = torch.randn(hi - lo, generator=g, device=device).to(dtype)
    return out


def _rand(shape, g, device) -> torch.Tensor:
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def _e4m3_with_scale(k: torch.Tensor):
    """fp32 keys [.., D] -> (e4m3fn bytes, fp32 per-row scale)."""
    amax = k.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    kq = (k / scale[..., None]).clamp_(-448.0, 448.0)
    return kq.to(torch.float8_e4m3fn).view(torch.uint8), scale.float()


def _pack_planes(codes: torch.Tensor) -> torch.Tensor:
    """codes [.., n] uint8 (0..15) -> planes [.., 4, ceil(n/32)] uint32 bits."""
    n = codes.shape[-1]
    nw = (n + 31) // 32
    pad = nw * 32 - n
    c = codes.to(torch.int64)
    if pad:
        c = torch.nn.functional.pad(c, (0, pad))
    c = c.view(*codes.shape[:-1], nw, 32)
    weights = (torch.ones(32, dtype=torch.int64, device=codes.device)
               << torch.arange(32, device=codes.device))
    planes = []
    for j in range(4):
        bits = (c >> (3 - j)) & 1
        word = (bits * weights).sum(dim=-1)  # < 2^32
        planes.append(word)
    p = torch.stack(planes, dim=-2)  # [.., 4, nw], values < 2^32
    # keep the low 32 bits; stored as int32 holding the uint32 bit pattern
    p = torch.where(p >= 2 ** 31, p - 2 ** 32, p)
    return p.to(torch.int32)


def quantize_4bit(k: torch.Tensor):
    """fp32 keys [n][D] -> (codes uint8 [n][D], zero fp32 [D], cell fp32 [D]).

    Per channel: zero = min, cell = (max - min) / 16, both stored in fp32;
    code = min(floor((k - zero) / cell), 15) computed in fp64 from the stored
    values (a constant channel gets cell 0 and code 0).
    """
    lo = k.amin(dim=0)
    hi = k.amax(dim=0)
    c = ((hi - lo) / 16.0).float()
    safe = torch.where(c > 0, c, torch.ones_like(c)).double()
    code = torch.floor((k.double() - lo.double()[None, :]) / safe[None, :])
    code = torch.where(c[None, :] > 0, code, torch.zeros_like(code))
    return code.clamp_(0, 15).to(torch.uint8), lo.float(), c


def make_inputs(w: Workload, device="cpu") -> dict:
    """All inputs of one decode step of workload `w`, on `device`."""
    dev = torch.device(device)
    B, n = w.B, w.n
    inp: dict = {"workload": w}
    if w.seq_lens is not None:
        inp["seq_lens"] = torch.tensor(w.seq_lens, dtype=torch.int32,
                                       device=dev)
    qdt = torch.float32 if w.dtype == "f32" else torch.bfloat16

    if w.kind == "dot":
        # index keys are the attention K cache; index query = attention query
        inp["q"] = _randn((B, w.hq, w.d_qk), _gen(w, 1, dev), dev, qdt)
        inp["k_cache"] = _randn((B, n, w.hkv, w.d_qk), _gen(w, 2, dev), dev,
                                qdt)
        inp["v_cache"] = _randn((B, n, w.hkv, w.d_v), _gen(w, 3, dev), dev,
                                qdt)
        return inp

    if w.kind == "lightning":
        inp["q_idx"] = _randn((B, w.idx_heads, w.idx_dim), _gen(w, 1, dev),
                              dev, torch.bfloat16)
        inp["head_w"] = _rand((B, w.idx_heads), _gen(w, 2, dev), dev)
        k8 = torch.empty((B, n, w.idx_dim), dtype=torch.uint8, device=dev)
        ks = torch.empty((B, n), dtype=torch.float32, device=dev)
        g = _gen(w, 3, dev)
        rows = max(1, _CHUNK // w.idx_dim)
        for b in range(B):
            for lo in range(0, n, rows):
                hi = min(n, lo + rows)
                kf = torch.randn((hi - lo, w.idx_dim), generator=g,
                                 device=dev)
                k8[b, lo:hi], ks[b, lo:hi] = _e4m3_with_scale(kf)
        inp["k8"], inp["k_scale"] = k8, ks
        inp["q"] = _randn((B, w.hq, w.d_qk), _gen(w, 4, dev), dev,
                          torch.bfloat16)
        if w.hot:
            # full latent KV lives in host memory (hot buffer built later);
            # drawn on `device` per request and copied into pinned memory
            pinned = dev.type == "cuda"
            host = torch.empty((B, n, w.d_qk), dtype=torch.bfloat16, pin_memory=pinned)
            g = _gen(w, 5, dev)
            for b in range(B):
                host[b].copy_(_randn((n, w.d_qk), g, dev, torch.bfloat16))
            inp["host_kv"] = host
        elif w.page:
            n_pages = (n + w.page - 1) // w.page
            inp["kv_pool"] = _randn((B * n_pages, w.page, w.d_qk),
                                    _gen(w, 5, dev), dev, torch.bfloat16)
            perm = torch.randperm(B * n_pages, generator=_gen(w, 6, "cpu"))
            inp["page_table"] = perm.view(B, n_pages).to(torch.int32).to(dev)
        else:
            inp["kv"] = _randn((B, n, w.d_qk), _gen(w, 5, dev), dev,
                               torch.bfloat16)
        return inp

    if w.kind == "block":
        inp["q_idx"] = _randn((B, w.idx_heads, w.idx_dim), _gen(w, 1, dev),
                              dev, torch.bfloat16)
        inp["k_idx"] = _randn((B, n, w.idx_dim), _gen(w, 2, dev), dev,
                              torch.bfloat16)
        layers = []
        for layer in range(w.layers):
            base = 10 * (layer + 1)
            layers.append({
                "q": _randn((B, w.hq, w.d_qk), _gen(w, base + 1, dev), dev,
                            torch.bfloat16),
                "k_cache": _randn((B, n, w.hkv, w.d_qk),
                                  _gen(w, base + 2, dev), dev, torch.bfloat16),
                "v_cache": _randn((B, n, w.hkv, w.d_v),
                                  _gen(w, base + 3, dev), dev, torch.bfloat16),
            })
        inp["layers"] = layers
        return inp

    if w.kind == "fathom":
        D, H = w.d_qk, w.hkv
        inp["q"] = _randn((B, w.hq, D), _gen(w, 1, dev), dev, torch.bfloat16)
        var = torch.exp(torch.randn((B, H, D), generator=_gen(w, 2, dev),
                                    device=dev))
        inp["chan_var"] = var.float()
        codes = torch.empty((B, H, n, D), dtype=torch.uint8, device=dev)
        zero = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        cell = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        kbf = torch.empty((B, n, H, D), dtype=torch.bfloat16, device=dev)
        g = _gen(w, 3, dev)
        for b in range(B):
            for h in range(H):
                k = torch.randn((n, D), generator=g, device=dev) * \
                    var[b, h].sqrt()[None, :]
                codes[b, h], zero[b, h], cell[b, h] = quantize_4bit(k)
                kbf[b, :, h] = k.to(torch.bfloat16)
        inp["codes"] = codes
        inp["chan_zero"], inp["chan_scale"] = zero, cell
        nw = (n + 31) // 32
        planes = torch.empty((B, H, D, 4, nw), dtype=torch.int32, device=dev)
        for b in range(B):
            for h in range(H):
                planes[b, h] = _pack_planes(
                    codes[b, h].transpose(0, 1).contiguous())
        inp["planes"] = planes
        inp["k_cache"] = kbf
        inp["v_cache"] = _randn((B, n, H, w.d_v), _gen(w, 4, dev), dev,
                                torch.bfloat16)
        return inp

    raise ValueError(f"unknown workload kind {w.kind}")


def build_hot_buffer(inp: dict, selection: torch.Tensor, device,
                     pinned: bool = True) -> dict:
    """Place rows of the host KV into a per-request hot buffer.

    selection: [B][k] int32 token ids (ascending, -1 padded) that the step
    will select.  Exactly round(miss_rate * m) of each request's m valid
    selected tokens are left out of the hot buffer (chosen by a seeded
    permutation); the other selected tokens get slots, and the remaining
    slots hold seeded filler tokens that are not selected.  Returns the
    hot-buffer tensors and moves the host KV into pinned memory.
    """
    w: Workload = inp["workload"]
    B, n, H = w.B, w.n, w.hot
    host = inp["host_kv"]
    if pinned and not host.is_pinned():
        pin = torch.empty(host.shape, dtype=host.dtype, pin_memory=True)
        pin.copy_(host)
        host = pin
    sel = selection.to("cpu").numpy()
    rng = np.random.Generator(np.random.PCG64(w.seed * 1000 + 77))
    slot = np.full((B, n), -1, dtype=np.int32)
    hot_tokens = np.zeros((B, H), dtype=np.int64)
    n_miss = np.zeros(B, dtype=np.int64)
    for b in range(B):
        valid = w.valid(b)
        s = sel[b][sel[b] >= 0]
        m = s.shape[0]
        miss = int(math.floor(w.miss_rate * m + 0.5))
        perm = rng.permutation(m)
        hits = np.sort(s[perm[miss:]])
        n_miss[b] = miss
        if hits.shape[0] > H:
            raise ValueError("hot buffer smaller than the selected hits")
        chosen = set(s.tolist())
        filler_pool = np.array([t for t in rng.permutation(valid)[: H * 2 + m]
                                if t not in chosen], dtype=np.int64)
        toks = np.concatenate([hits, filler_pool[: H - hits.shape[0]]])
        for i, t in enumerate(toks):
            slot[b, t] = i
        if toks.shape[0] < H:  # tiny contexts: unused rows copy token 0
            toks = np.concatenate([toks, np.zeros(H - toks.shape[0],
                                                  dtype=np.int64)])
        hot_tokens[b] = toks
    hot_kv = torch.empty((B, H, w.d_qk), dtype=torch.bfloat16, device=device)
    for b in range(B):
        idx = torch.from_numpy(hot_tokens[b])
        hot_kv[b] = host[b].index_select(0, idx).to(device)
    return {"host_kv": host, "hot_kv": hot_kv,
            "hot_slot": torch.from_numpy(slot).to(device),
            "n_miss": n_miss}


def fixed_depths(w: Workload, bits: int, device) -> torch.Tensor:
    """A fixed read allocation of `bits` bits per key for every (request,
    KV head): floor(bits / D) planes in every channel and one more in the
    first bits % D channels.  [B][Hkv][D] int8."""
    D = w.d_qk
    base, extra = divmod(bits, D)
    t = np.full((w.B, w.hkv, D), base, dtype=np.int8)
    t[:, :, :extra] += 1
    return torch.from_numpy(t).to(device)


def random_depths(w: Workload, device, seed: int = 7) -> torch.Tensor:
    """Seeded random read depths 0..4, [B][Hkv][D] int8."""
    rng = np.random.Generator(np.random.PCG64(w.seed * 1000 + seed))
    t = rng.integers(0, 5, size=(w.B, w.hkv, w.d_qk)).astype(np.int8)
    return torch.from_numpy(t).to(device)


def pinned_copy(t: torch.Tensor) -> torch.Tensor:
    """A copy of `t` in pinned host memory."""
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def host_view(t: torch.Tensor) -> np.ndarray:
    """A CPU numpy copy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
