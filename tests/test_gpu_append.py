"""GPU: the decode-side append (sparse_append_token) against the oracle.

Every byte the append writes is compared bit for bit with the oracle's
encoding of the same new key (e4m3fn bytes and fp32 scale, bf16 rows, 4-bit
codes in the bit planes, copied KV rows), every other byte must be
unchanged, and a decode step run after the append must see the new token
(oracle parity on the updated inputs, as in test_gpu_parity).
"""
import numpy as np
import pytest
import torch

import indexer_top_sparse_amd as isa
from indexer_top_sparse_amd.runner import StepRunner
import synth
from oracle import append as A
from oracle import compare as C

from helpers import arrays, oracle_step

pytestmark = pytest.mark.gpu


def _positions(w):
    """The token after each request's history, or its last slot when full."""
    return [min(w.valid(b), w.n - 1) for b in range(w.B)]


def _randn(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return torch.from_numpy((g.normal(size=shape) * scale).astype(np.float32)).cuda()


def _hv(t):
    return synth.host_view(t).copy()


def _extended(w, pos):
    """The workload with the appended token counted as valid."""
    seq = tuple(max(w.valid(b), p + 1) for b, p in enumerate(pos))
    return w.with_(seq_lens=seq)


def _check_step(w, inp, r):
    arr = arrays(inp)
    ref = oracle_step(w, arr)
    r.run()
    torch.cuda.synchronize()
    g = r.topk.cpu().numpy()
    s = r.index_scores().cpu().numpy()
    for b in range(w.B):
        v = (w.valid(b) + w.block - 1) // w.block
        for h in range(g.shape[1]):
            ok, err, tau = C.scores_ok(s[b, h], ref["scores"][b, h], w.k, v)
            assert ok, (b, h, err, tau)
            ok, why = C.selection_ok(g[b, h], ref["sel"][b, h], ref["scores"][b, h], w.k, v)
            assert ok, (b, h, why)
    ref_g = oracle_step(w, arr, sel_in=g.astype(np.int64))
    outs = ref_g["layers"][0]["out"] if w.kind == "block" else ref_g["out"]
    ok, err = C.attn_ok(r.outs[0].cpu().numpy(), outs)
    assert ok, err


def test_append_lightning_paged_then_step():
    w = synth.get("lightning_small")
    print(f"[append] {w.name}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    pos = _positions(w)
    pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
    key_new = _randn((w.B, w.idx_dim), 11, 3.0)
    k_new = _randn((w.B, 1, w.d_qk), 12).to(torch.bfloat16)
    k8, ks, pool = _hv(inp["k8"]), _hv(inp["k_scale"]), _hv(inp["kv_pool"])
    r = StepRunner(inp)
    isa.sparse_append_token(r.ia, r.layer_args[0][0], pos_t, key_new, k_new)
    torch.cuda.synchronize()
    kn, pt, kb = key_new.cpu().numpy(), inp["page_table"].cpu().numpy(), _hv(k_new)
    for b, t in enumerate(pos):
        codes, sigma = A.quantize_index_key(kn[b])
        k8[b, t], ks[b, t] = codes, sigma
        pool[pt[b, t // w.page], t % w.page] = kb[b, 0]
    assert np.array_equal(_hv(inp["k8"]), k8)
    assert np.array_equal(_hv(inp["k_scale"]).view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(_hv(inp["kv_pool"]), pool)
    # the next step reads the appended token
    w2 = _extended(w, pos)
    inp["seq_lens"].copy_(torch.tensor(w2.seq_lens, dtype=torch.int32))
    inp["workload"] = w2
    _check_step(w2, inp, StepRunner(inp))


def test_append_fathom_planes_and_rows_then_step():
    w = synth.get("fathom_small")
    print(f"[append] {w.name}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    pos = _positions(w)
    pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
    # keys at the channels' scale, some outside their recorded range
    key_new = _randn((w.B, w.hkv, w.d_qk), 21) * inp["chan_var"].sqrt() * 1.5
    k_new = _randn((w.B, w.hkv, w.d_qk), 22).to(torch.bfloat16)
    v_new = _randn((w.B, w.hkv, w.d_v), 23).to(torch.bfloat16)
    planes, kc, vc = _hv(inp["planes"]), _hv(inp["k_cache"]), _hv(inp["v_cache"])
    zero, cell = _hv(inp["chan_zero"]), _hv(inp["chan_scale"])
    r = StepRunner(inp)
    isa.sparse_append_token(r.ia, r.layer_args[0][0], pos_t, key_new.contiguous(), k_new, v_new)
    torch.cuda.synchronize()
    kn = key_new.cpu().numpy()
    for b, t in enumerate(pos):
        for h in range(w.hkv):
            A.set_plane_bits(planes[b, h], t, A.fathom_code(kn[b, h], zero[b, h], cell[b, h]))
        kc[b, t] = _hv(k_new)[b]
        vc[b, t] = _hv(v_new)[b]
    assert np.array_equal(_hv(inp["planes"]), planes)
    assert np.array_equal(_hv(inp["k_cache"]), kc)
    assert np.array_equal(_hv(inp["v_cache"]), vc)
    w2 = _extended(w, pos)
    inp["seq_lens"].copy_(torch.tensor(w2.seq_lens, dtype=torch.int32))
    inp["workload"] = w2
    # the codes of the appended keys now stand for them in the oracle too
    codes = inp["codes"].cpu().numpy()
    for b, t in enumerate(pos):
        for h in range(w.hkv):
            codes[b, h, t] = A.fathom_code(kn[b, h], zero[b, h], cell[b, h])
    inp["codes"] = torch.from_numpy(codes)
    _check_step(w2, inp, StepRunner(inp))


def test_append_block_keys_and_layer_rows():
    w = synth.get("block_sparse_small")
    print(f"[append] {w.name}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    pos = _positions(w)
    pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
    key_new = _randn((w.B, w.idx_dim), 31)
    k_new = _randn((w.B, w.hkv, w.d_qk), 32).to(torch.bfloat16)
    v_new = _randn((w.B, w.hkv, w.d_v), 33).to(torch.bfloat16)
    kidx = _hv(inp["k_idx"])
    kc, vc = _hv(inp["layers"][1]["k_cache"]), _hv(inp["layers"][1]["v_cache"])
    r = StepRunner(inp)
    isa.sparse_append_token(r.ia, r.layer_args[1][0], pos_t, key_new, k_new, v_new)
    torch.cuda.synchronize()
    kn = key_new.cpu().numpy()
    for b, t in enumerate(pos):
        kidx[b, t] = A.bf16_rne(kn[b])
        kc[b, t] = _hv(k_new)[b]
        vc[b, t] = _hv(v_new)[b]
    assert np.array_equal(_hv(inp["k_idx"]), kidx)
    assert np.array_equal(_hv(inp["layers"][1]["k_cache"]), kc)
    assert np.array_equal(_hv(inp["layers"][1]["v_cache"]), vc)


def test_append_out_of_range_skipped_and_repeat_idempotent():
    w = synth.get("lightning_small")
    inp = synth.make_inputs(w, "cuda")
    r = StepRunner(inp)
    key_new = _randn((w.B, w.idx_dim), 41)
    k_new = _randn((w.B, 1, w.d_qk), 42).to(torch.bfloat16)
    before = [_hv(inp[k]) for k in ("k8", "k_scale", "kv_pool")]
    bad = torch.tensor([-1, w.n, -5][:w.B], dtype=torch.int32, device="cuda")
    isa.sparse_append_token(r.ia, r.layer_args[0][0], bad, key_new, k_new)
    torch.cuda.synchronize()
    for a, k in zip(before, ("k8", "k_scale", "kv_pool")):
        assert np.array_equal(_hv(inp[k]), a)
    pos_t = torch.tensor(_positions(w), dtype=torch.int32, device="cuda")
    isa.sparse_append_token(r.ia, r.layer_args[0][0], pos_t, key_new, k_new)
    torch.cuda.synchronize()
    once = [_hv(inp[k]) for k in ("k8", "k_scale", "kv_pool")]
    isa.sparse_append_token(r.ia, r.layer_args[0][0], pos_t, key_new, k_new)
    torch.cuda.synchronize()
    for a, k in zip(once, ("k8", "k_scale", "kv_pool")):
        assert np.array_equal(_hv(inp[k]), a)


def test_append_hot_buffer_writes_host_history():
    w = synth.get("hot_small")
    inp = synth.make_inputs(w, "cuda")
    from synth.gen import build_hot_buffer
    sel = torch.zeros((w.B, w.k), dtype=torch.int32, device="cuda")
    sel[:, :] = torch.arange(w.k, dtype=torch.int32, device="cuda")
    hot = build_hot_buffer(inp, sel, "cuda")
    r = StepRunner(inp, hot=hot)
    pos = _positions(w)
    pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
    k_new = _randn((w.B, 1, w.d_qk), 51).to(torch.bfloat16)
    hot_before = _hv(hot["hot_kv"])
    host = _hv(hot["host_kv"])
    isa.sparse_append_token(None, r.layer_args[0][0], pos_t, None, k_new)
    torch.cuda.synchronize()
    for b, t in enumerate(pos):
        host[b, t] = _hv(k_new)[b, 0]
    assert np.array_equal(_hv(hot["host_kv"]), host)
    assert np.array_equal(_hv(hot["hot_kv"]), hot_before)
