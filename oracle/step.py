"""One decode step of each workload kind, request by request, in float64.

TEST INFRASTRUCTURE ONLY (see oracle/oracle.py).  Inputs are plain numpy
arrays in the stored formats (bf16 as uint16 bit patterns, e4m3fn as uint8
bytes, 4-bit codes as uint8, fp32 as float32, int32 tables); the step
decodes them exactly, scores every valid unit, selects the top-k, maps the
selected units to KV rows and runs exact softmax attention over those rows.

Index -> KV address (the row of token t):
  * paged latent KV: pool[page_table[b][t // page]][t % page]
    ("XM-Sparse" blog, Figure 1 caption: attention reads selected entries
    of a KV cache; the pages fix no layout, the paged pool with 64-token
    pages is the reading taken here),
  * contiguous KV: kv[b][t] (per KV head: kv[b][t][h]),
  * a selected 64-token block b stands for tokens 64b .. 64b+63
    ("MiniMax-M3" PR description: top-k KV blocks).
"""
from __future__ import annotations

import math

import numpy as np

from . import oracle as O


def _dec(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return O.decode_bf16(a)
    return O.decode_f32(a)


def _valid(p: dict, b: int) -> int:
    sl = p.get("seq_lens")
    return p["n"] if sl is None else int(sl[b])


def _pad_scores(s: np.ndarray, valid: int, n_units: int) -> np.ndarray:
    out = np.full(n_units, -np.inf)
    out[:valid] = s[:valid]
    return out


def dot_step(arr: dict, p: dict, sel_in: np.ndarray | None = None) -> dict:
    """Head-summed dot index over the K cache itself, GQA attention (fp32 or
    bf16 inputs).  p: n, k, hq, hkv, dtype, seq_lens.  With sel_in
    ([B][1][k]) the given selection is attended instead of the top-k."""
    q = _dec(arr["q"], p["dtype"])
    K = _dec(arr["k_cache"], p["dtype"])
    V = _dec(arr["v_cache"], p["dtype"])
    B, Hq, D = q.shape
    hkv = K.shape[2]
    G = Hq // hkv
    scale = 1.0 / math.sqrt(D)
    scores, sels, outs, lses = [], [], [], []
    for b in range(B):
        valid = _valid(p, b)
        # index keys: KV head 0 of the K cache (one KV head in this kind)
        s = O.score_dot_headsum(q[b], K[b, :valid, 0, :])
        s = _pad_scores(s, valid, p["n"])
        sel = O.topk(s, p["k"], valid) if sel_in is None else sel_in[b, 0]
        toks = O.expand_selection(sel, 1, valid)
        out = np.zeros((Hq, V.shape[3]))
        lse = np.zeros(Hq)
        for h in range(hkv):
            hs = slice(h * G, (h + 1) * G)
            out[hs], lse[hs] = O.attention(q[b, hs], K[b, toks, h],
                                           V[b, toks, h], scale)
        scores.append(s[None])
        sels.append(sel[None])
        outs.append(out)
        lses.append(lse)
    return {"scores": np.stack(scores), "sel": np.stack(sels),
            "out": np.stack(outs), "lse": np.stack(lses)}


def latent_rows(arr: dict, p: dict, b: int, toks: np.ndarray) -> np.ndarray:
    """Latent KV rows (bf16 -> float64) of request b's tokens."""
    if "kv_pool" in arr:
        page = p["page"]
        pt = arr["page_table"][b]
        phys = pt[toks // page]
        rows = arr["kv_pool"][phys, toks % page]
    elif "host_kv" in arr:
        rows = arr["host_kv"][b, toks]
    else:
        rows = arr["kv"][b, toks]
    return O.decode_bf16(rows)


def lightning_scores(arr: dict, p: dict, b: int) -> np.ndarray:
    valid = _valid(p, b)
    q = O.decode_bf16(arr["q_idx"][b])
    w = O.decode_f32(arr["head_w"][b])
    k8 = O.decode_e4m3fn(arr["k8"][b, :valid])
    ks = O.decode_f32(arr["k_scale"][b, :valid])
    s = O.score_lightning(q, w, k8, ks)
    return _pad_scores(s, valid, p["n"])


def lightning_step(arr: dict, p: dict, requests=None,
                   sel_in: np.ndarray | None = None) -> dict:
    """Lightning-indexer fp8 scores, top-k tokens, MLA attention over the
    selected latent rows (key = the whole row, value = its first d_v dims).
    With sel_in ([B][1][k]) scoring is skipped and that selection attended."""
    B = arr["q"].shape[0]
    d_qk, d_v = p["d_qk"], p["d_v"]
    scale = p.get("sm_scale", 1.0 / math.sqrt(d_qk))
    reqs = range(B) if requests is None else requests
    scores, sels, outs, lses = [], [], [], []
    for b in reqs:
        valid = _valid(p, b)
        if sel_in is None:
            s = lightning_scores(arr, p, b)
            sel = O.topk(s, p["k"], valid)
        else:
            s = np.zeros(p["n"])
            sel = sel_in[b, 0]
        toks = O.expand_selection(sel, 1, valid)
        rows = latent_rows(arr, p, b, toks)
        q = O.decode_bf16(arr["q"][b])
        out, lse = O.attention(q, rows[:, :d_qk], rows[:, :d_v], scale)
        scores.append(s[None])
        sels.append(sel[None])
        outs.append(out)
        lses.append(lse)
    return {"scores": np.stack(scores), "sel": np.stack(sels),
            "out": np.stack(outs), "lse": np.stack(lses)}


def gqa_attention(q: np.ndarray, K_raw: np.ndarray, V_raw: np.ndarray,
                  toks_per_kv_head: list, scale: float):
    """q [Hq][D] float64; K_raw, V_raw [n][Hkv][D] bf16 bit patterns.
    Query head h uses KV head h // (Hq / Hkv) and that KV head's selected
    tokens; only the selected rows are decoded."""
    Hq = q.shape[0]
    hkv = K_raw.shape[1]
    G = Hq // hkv
    out = np.zeros((Hq, V_raw.shape[2]))
    lse = np.zeros(Hq)
    for h in range(hkv):
        toks = toks_per_kv_head[h]
        hs = slice(h * G, (h + 1) * G)
        out[hs], lse[hs] = O.attention(q[hs], O.decode_bf16(K_raw[toks, h]),
                                       O.decode_bf16(V_raw[toks, h]), scale)
    return out, lse


def block_step(arr: dict, p: dict, sel_in: np.ndarray | None = None,
               requests=None) -> dict:
    """Block-sparse decode over several layers that share one selection.

    Layer 0 scores tokens with the head-summed dot, takes the max over each
    64-token block, and selects the top-k blocks; every later layer reuses
    that selection with its own q, K and V ("MiniMax-M3" PR, description
    and Correctness note).  arr["layers"] is a list of dicts (q, k_cache,
    v_cache).  If sel_in is given, no scoring is done and that selection is
    used by every layer.  `requests` limits the step to those requests
    (their results are stacked in that order).
    """
    B = arr["q_idx"].shape[0]
    reqs = list(range(B)) if requests is None else list(requests)
    blk = p["block"]
    n_units = (p["n"] + blk - 1) // blk
    scores, sels = [], []
    for b in reqs:
        valid = _valid(p, b)
        if sel_in is None:
            q = O.decode_bf16(arr["q_idx"][b])
            keys = O.decode_bf16(arr["k_idx"][b, :valid])
            ts = O.score_dot_headsum(q, keys)
            S = O.block_max(_pad_scores(ts, valid, p["n"]), blk, valid)
            sel = O.topk(S, p["k"], (valid + blk - 1) // blk)
            scores.append(S[None])
        else:
            sel = sel_in[b].reshape(-1)
        sels.append(sel[None])
    sels = np.stack(sels)
    layer_out = []
    for layer in arr["layers"]:
        outs, lses = [], []
        for i, b in enumerate(reqs):
            valid = _valid(p, b)
            toks = O.expand_selection(sels[i, 0], blk, valid)
            q = O.decode_bf16(layer["q"][b])
            D = q.shape[1]
            K, V = layer["k_cache"][b], layer["v_cache"][b]
            hkv = K.shape[1]
            out, lse = gqa_attention(q, K, V, [toks] * hkv, 1.0 / math.sqrt(D))
            outs.append(out)
            lses.append(lse)
        layer_out.append({"out": np.stack(outs), "lse": np.stack(lses)})
    res = {"sel": sels, "layers": layer_out, "n_units": n_units}
    if scores:
        res["scores"] = np.stack(scores)
    return res


def fathom_step(arr: dict, p: dict, requests=None,
                sel_in: np.ndarray | None = None) -> dict:
    """Fathom scan: per (request, KV head) read depth by reverse
    water-filling (or the fixed depths arr["depth_in"] when given),
    plane-prefix scores, top-k tokens per KV head, bf16 GQA attention of that
    head's query group over its own selection."""
    q_all = O.decode_bf16(arr["q"])
    B, Hq, D = q_all.shape
    hkv = arr["codes"].shape[1]
    G = Hq // hkv
    budget = p["budget"]
    reqs = range(B) if requests is None else requests
    scores, sels, outs, lses, depths = [], [], [], [], []
    for b in reqs:
        valid = _valid(p, b)
        srow, selrow, drow, toks = [], [], [], []
        for h in range(hkv):
            qbar = O.fathom_group_query(q_all[b, h * G:(h + 1) * G])
            var = O.decode_f32(arr["chan_var"][b, h])
            if "depth_in" in arr:  # a fixed allocation given by the caller
                t = np.clip(arr["depth_in"][b, h].astype(np.int64), 0, 4)
            else:
                t = O.fathom_read_depth(qbar, var, budget)
            s = O.score_fathom(qbar, arr["codes"][b, h, :valid],
                               O.decode_f32(arr["chan_zero"][b, h]),
                               O.decode_f32(arr["chan_scale"][b, h]), t)
            s = _pad_scores(s, valid, p["n"])
            sel = O.topk(s, p["k"], valid) if sel_in is None else sel_in[b, h]
            srow.append(s)
            selrow.append(sel)
            drow.append(t)
            toks.append(O.expand_selection(sel, 1, valid))
        out, lse = gqa_attention(q_all[b], arr["k_cache"][b],
                                 arr["v_cache"][b], toks, 1.0 / math.sqrt(D))
        scores.append(np.stack(srow))
        sels.append(np.stack(selrow))
        depths.append(np.stack(drow))
        outs.append(out)
        lses.append(lse)
    return {"scores": np.stack(scores), "sel": np.stack(sels),
            "depth": np.stack(depths), "out": np.stack(outs),
            "lse": np.stack(lses)}
