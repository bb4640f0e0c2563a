"""GPU parity at the full workload sizes, in the launch configuration that
bench.py times (the fused step through the C ABI, same shapes and grids).

The oracle is run on sampled requests (all of their units) -- scores, the
band-rule selection and attention on the GPU's selection -- and properties
that hold at any size are checked on every row: exactly min(k, valid)
distinct in-range indices in ascending order, -1 padding after them, and a
bit-identical second run.
"""
import math

import numpy as np
import pytest
import torch

import synth
from synth.gen import build_hot_buffer
import indexer_top_sparse_amd as isa
from indexer_top_sparse_amd.runner import StepRunner
from oracle import compare as C
from oracle import oracle as O
from oracle import step as S

from helpers import params

pytestmark = pytest.mark.gpu


def _hv(t):
    return synth.host_view(t)


def _check_rows(topk: np.ndarray, w, unit=1):
    for b in range(topk.shape[0]):
        valid = (w.valid(b) + unit - 1) // unit
        k_eff = min(w.k, valid)
        for h in range(topk.shape[1]):
            row = topk[b, h]
            sel, pad = row[:k_eff], row[k_eff:]
            assert np.all(pad == -1)
            assert np.all(sel >= 0) and np.all(sel < valid)
            assert np.all(np.diff(sel) > 0)


def _rerun_identical(r):
    first = [t.clone() for t in r.outs + r.lses + [r.topk]]
    r.run()
    torch.cuda.synchronize()
    for a, b in zip(first, r.outs + r.lses + [r.topk]):
        assert torch.equal(a, b)


def _lightning_request(inp, b, w):
    """Request b's inputs as a one-request oracle input set."""
    arr = {
        "q_idx": _hv(inp["q_idx"][b:b + 1]), "head_w": _hv(inp["head_w"][b:b + 1]),
        "k8": _hv(inp["k8"][b:b + 1]), "k_scale": _hv(inp["k_scale"][b:b + 1]),
        "q": _hv(inp["q"][b:b + 1]),
    }
    if "kv_pool" in inp:
        pt = inp["page_table"][b].long()
        arr["kv_pool"] = _hv(inp["kv_pool"].index_select(0, pt))
        arr["page_table"] = np.arange(pt.numel(), dtype=np.int32)[None, :]
    else:
        arr["host_kv"] = _hv(inp["host_kv"][b:b + 1])
    p = params(w)
    p["seq_lens"] = None if w.seq_lens is None else (w.seq_lens[b],)
    return arr, p


def _check_lightning_sample(w, inp, r, scores, gsel, reqs):
    for b in reqs:
        arr, p = _lightning_request(inp, b, w)
        ref_s = S.lightning_scores(arr, p, 0)
        valid = w.valid(b)
        ok, err, tau = C.scores_ok(scores[b, 0], ref_s, w.k, valid)
        assert ok, (b, err, tau)
        ref_sel = O.topk(ref_s, w.k, valid)
        ok, why = C.selection_ok(gsel[b, 0], ref_sel, ref_s, w.k, valid)
        assert ok, (b, why)
        ref = S.lightning_step(arr, p, sel_in=gsel[b:b + 1].astype(np.int64))
        ok, err = C.attn_ok(r.outs[0][b].cpu().numpy(), ref["out"][0])
        assert ok, (b, err)
        lse = r.lses[0][b].cpu().numpy()
        ok, err = C.attn_ok(lse, ref["lse"][0])
        assert ok, (b, "lse", err)


def test_lightning_128k_full():
    w = synth.get("lightning_128k")
    print(f"[full] {w.name}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    gsel = r.topk.cpu().numpy()
    _check_rows(gsel, w)
    scores = r.index_scores().cpu().numpy()
    _check_lightning_sample(w, inp, r, scores, gsel, (0, 13, 31))
    _rerun_identical(r)


def test_lightning_long_spans_ragged():
    """The 128K batch at a token count that is not a multiple of a tile (nor
    of a workgroup's span), so the scan runs its long spans and the last
    workgroup of every request its ragged wave, with ragged valid lengths."""
    n = 131072 - 37
    seq = tuple([n, n - 1, 129999, 70001] + [n - 5 * i for i in range(4, 32)])
    w = synth.get("lightning_128k").with_(name="lightning_128k_ragged", n=n, seq_lens=seq,
                                          seed=1012)
    print(f"[full] {w.name} n={n}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    gsel = r.topk.cpu().numpy()
    _check_rows(gsel, w)
    scores = r.index_scores().cpu().numpy()
    _check_lightning_sample(w, inp, r, scores, gsel, (0, 1, 3))
    _rerun_identical(r)


def test_lightning_max_context():
    """One request at the largest context the boundary accepts (4194304
    tokens, 4.8 GB of paged latent rows): 512 histogram parts per row, so the
    top-k takes the bin, chunk-filter and select kernels."""
    n = 1 << 22
    w = synth.get("lightning_128k").with_(name="lightning_4m", B=1, n=n, seq_lens=(n - 5,),
                                          seed=1014)
    print(f"[full] {w.name} n={n}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    gsel = r.topk.cpu().numpy()
    _check_rows(gsel, w)
    scores = r.index_scores().cpu().numpy()
    _check_lightning_sample(w, inp, r, scores, gsel, (0,))
    _rerun_identical(r)


def test_block_sparse_80k_full():
    w = synth.get("block_sparse_80k")
    print(f"[full] {w.name}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    gsel = r.topk.cpu().numpy()
    _check_rows(gsel, w, w.block)
    scores = r.index_scores().cpu().numpy()
    for b in (0, 15):
        arr = {"q_idx": _hv(inp["q_idx"][b:b + 1]), "k_idx": _hv(inp["k_idx"][b:b + 1]),
               "layers": [{k: _hv(v[b:b + 1]) for k, v in L.items()} for L in inp["layers"]]}
        p = params(w)
        ref = S.block_step(arr, p)
        nu = w.n_units
        ok, err, tau = C.scores_ok(scores[b, 0], ref["scores"][0, 0], w.k, nu)
        assert ok, (b, err, tau)
        ok, why = C.selection_ok(gsel[b, 0], ref["sel"][0, 0], ref["scores"][0, 0], w.k, nu)
        assert ok, (b, why)
        # both layers attend over the first layer's (GPU) selection
        ref_g = S.block_step(arr, p, sel_in=gsel[b:b + 1].astype(np.int64))
        for li in range(w.layers):
            ok, err = C.attn_ok(r.outs[li][b].cpu().numpy(), ref_g["layers"][li]["out"][0])
            assert ok, (b, li, err)
    _rerun_identical(r)


def test_fathom_1m_full():
    w = synth.get("fathom_1m")
    print(f"[full] {w.name}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    gsel = r.topk.cpu().numpy()
    _check_rows(gsel, w)
    depth = torch.empty((w.B, w.hkv, w.d_qk), dtype=torch.int8, device="cuda")
    isa.sparse_read_depth(r.ia, depth)
    scores = r.index_scores().cpu().numpy()
    arr = {k: _hv(inp[k]) for k in ("q", "chan_var", "codes", "chan_zero", "chan_scale",
                                    "k_cache", "v_cache")}
    p = params(w)
    ref = S.fathom_step(arr, p, sel_in=gsel.astype(np.int64))
    assert np.array_equal(depth.cpu().numpy().astype(np.int64), ref["depth"])
    for h in range(w.hkv):
        ok, err, tau = C.scores_ok(scores[0, h], ref["scores"][0, h], w.k, w.n)
        assert ok, (h, err, tau)
        ref_sel = O.topk(ref["scores"][0, h], w.k, w.n)
        ok, why = C.selection_ok(gsel[0, h], ref_sel, ref["scores"][0, h], w.k, w.n)
        assert ok, (h, why)
    ok, err = C.attn_ok(r.outs[0].cpu().numpy(), ref["out"])
    assert ok, err
    _rerun_identical(r)


def test_tiny_fp32_full():
    w = synth.get("tiny_fp32")
    print(f"[full] {w.name}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    arr = {k: _hv(v) for k, v in inp.items() if isinstance(v, torch.Tensor)}
    ref = S.dot_step(arr, params(w))
    gsel = r.topk.cpu().numpy()
    ok, why = C.selection_ok(gsel[0, 0], ref["sel"][0, 0], ref["scores"][0, 0], w.k, w.n)
    assert ok, why
    ref_g = S.dot_step(arr, params(w), sel_in=gsel.astype(np.int64))
    ok, err = C.attn_ok(r.outs[0].cpu().numpy(), ref_g["out"])
    assert ok, err


def _library_selection(inp, w):
    """The step's own selection (library scores + top-k), used only to decide
    which rows start in the hot buffer."""
    ia = isa.lightning_index_args(inp["q_idx"], inp["head_w"], inp["k8"], inp["k_scale"],
                                  inp.get("seq_lens"))
    scores = torch.empty((w.B, w.n), dtype=torch.float32, device="cuda")
    ws = isa.workspace(max(isa.sparse_workspace_size(ia, None, w.k),
                           isa.sparse_topk_workspace_size(w.B, w.n, w.k)))
    isa.sparse_index_score(ia, scores, ws)
    sel = torch.empty((w.B, w.k), dtype=torch.int32, device="cuda")
    isa.sparse_topk(scores, w.k, sel, None, inp.get("seq_lens"), 1, ws)
    torch.cuda.synchronize()
    return sel


@pytest.mark.parametrize("name", ["hot_16k", "hot_128k"])
def test_hot_full(name):
    w = synth.get(name)
    print(f"[full] {w.name}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    sel = _library_selection(inp, w)
    hot = build_hot_buffer(inp, sel, "cuda")
    n_sel = np.full(w.B, w.k)
    assert np.all(hot["n_miss"] == np.floor(0.2 * n_sel + 0.5))
    r = StepRunner(inp, hot=hot)
    r.run()
    torch.cuda.synchronize()
    gsel = r.topk.cpu().numpy()
    assert np.array_equal(gsel[:, 0], sel.cpu().numpy())
    _check_rows(gsel, w)
    scores = r.index_scores().cpu().numpy()
    _check_lightning_sample(w, inp, r, scores, gsel, (0, w.B - 1))
    # every selected row hot: bit-identical output
    hot_all = build_hot_buffer(dict(inp, workload=w.with_(miss_rate=0.0)), sel, "cuda")
    r_all = StepRunner(inp, hot=hot_all)
    r_all.run()
    torch.cuda.synchronize()
    assert torch.equal(r.outs[0], r_all.outs[0])
    assert torch.equal(r.lses[0], r_all.lses[0])
