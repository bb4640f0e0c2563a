"""Test helpers: move generator tensors to numpy and run the oracle step."""
import numpy as np
import torch

import synth
from oracle import step as S


def arrays(inp: dict) -> dict:
    out = {}
    for k, v in inp.items():
        if isinstance(v, torch.Tensor):
            out[k] = synth.host_view(v)
        elif k == "layers":
            out[k] = [{kk: synth.host_view(vv) for kk, vv in L.items()} for L in v]
    return out


def params(w) -> dict:
    return {"n": w.n, "k": w.k, "hq": w.hq, "hkv": w.hkv, "dtype": w.dtype,
            "seq_lens": w.seq_lens, "page": w.page, "block": w.block,
            "budget": w.budget, "d_qk": w.d_qk, "d_v": w.d_v}


def oracle_step(w, arr, sel_in=None, requests=None):
    p = params(w)
    if w.kind == "dot":
        return S.dot_step(arr, p, sel_in=sel_in)
    if w.kind == "lightning":
        return S.lightning_step(arr, p, requests=requests, sel_in=sel_in)
    if w.kind == "block":
        return S.block_step(arr, p, sel_in=sel_in)
    if w.kind == "fathom":
        return S.fathom_step(arr, p, requests=requests, sel_in=sel_in)
    raise ValueError(w.kind)


def valid_units(w, b):
    v = w.valid(b)
    return (v + w.block - 1) // w.block
