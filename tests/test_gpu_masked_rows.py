"""GPU: masked positions never read caller rows.

Padding entries (-1), tokens past a request's valid length and the pipeline
pad past a split's end get probability 0.  Their rows must not come from the
caller's memory: an unfilled hot-buffer slot or an unused page can hold NaN
or infinity, and a zero probability times NaN would poison every head of
the request.  Each case below fills rows that no valid selected token uses
(token 0's row, hot slot 0, an unused page) with NaN, selects a short
request with padding and k above the valid count, and checks every output
and log-sum-exp against the oracle, all finite.
"""
import numpy as np
import pytest
import torch

import indexer_top_sparse_amd as isa
from oracle import compare as C
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _selection(g, B, k, valid, avoid=(0,)):
    """[B][k] ascending token ids of each request's valid range minus
    `avoid`, at most k - 3 of them, with padding spread through the list."""
    sel = np.full((B, k), -1, dtype=np.int32)
    for b in range(B):
        pool = np.array([t for t in range(valid[b]) if t not in avoid])
        m = min(k - 3, pool.size)
        pick = np.sort(g.choice(pool, size=m, replace=False))
        pos = np.sort(g.choice(k, size=m, replace=False))
        sel[b, pos] = pick
    return sel


def _check(out, lse, ref_out, ref_lse):
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    ok, err = C.attn_ok(out, ref_out)
    assert ok, err
    ok, err = C.attn_ok(lse, ref_lse)
    assert ok, ("lse", err)


@pytest.mark.parametrize("paged", [False, True])
def test_latent_masked_positions_ignore_nan_rows(paged):
    print(f"[masked] latent paged={paged}", flush=True)
    g = np.random.default_rng(91 + paged)
    B, n, Hq, k = 2, 256, 64, 96
    valid = [40, 7]
    rows = g.normal(size=(B, n, 576)).astype(np.float32)
    q = torch.from_numpy(g.normal(size=(B, Hq, 576)).astype(np.float32)).to(torch.bfloat16).cuda()
    if paged:
        npg = n // 64
        # pool page 0 is unused and all NaN; request pages start at 1
        pool = np.full((B * npg + 1, 64, 576), np.nan, dtype=np.float32)
        perm = 1 + g.permutation(B * npg).astype(np.int32)
        pool[perm] = rows.reshape(B * npg, 64, 576)
        kc = torch.from_numpy(pool).to(torch.bfloat16).cuda()
        pt = torch.from_numpy(perm.reshape(B, npg)).cuda()
    else:
        rows_nan = rows.copy()
        rows_nan[:, 0] = np.nan  # token 0 is never selected
        kc = torch.from_numpy(rows_nan).to(torch.bfloat16).cuda()
        pt = None
    sel = _selection(g, B, k, valid)
    seq = torch.tensor(valid, dtype=torch.int32, device="cuda")
    aa = isa.attn_args(q, kc, None, n=n, d_v=512, sm_scale=576 ** -0.5, page_table=pt,
                       page_size=64 if paged else 0, seq_lens=seq)
    out = torch.empty((B, Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = isa.workspace(isa.sparse_workspace_size(None, aa, k))
    isa.sparse_gather_attn_decode(aa, torch.from_numpy(sel).cuda(), 1, k, 1, out, lse, ws)
    torch.cuda.synchronize()
    qn = O.decode_bf16(_bits(q))
    R = _bits(torch.from_numpy(rows).to(torch.bfloat16))
    for b in range(B):
        toks = O.expand_selection(sel[b], 1, valid[b])
        keys = O.decode_bf16(R[b, toks])
        ro, rl = O.attention(qn[b], keys, keys[:, :512], 576 ** -0.5)
        _check(out[b].cpu().numpy(), lse[b].cpu().numpy(), ro, rl)


def test_hot_buffer_masked_positions_ignore_nan_slot():
    print("[masked] hot buffer", flush=True)
    g = np.random.default_rng(93)
    B, n, Hq, k, S = 2, 300, 64, 64, 128
    valid = [50, 9]
    host = torch.from_numpy(g.normal(size=(B, n, 576)).astype(np.float32)).to(torch.bfloat16)
    host = host.pin_memory()
    sel = _selection(g, B, k, valid)
    # every selected token is hot, in slots 1.. ; slot 0 holds NaN
    slot = np.full((B, n), -1, dtype=np.int32)
    hot = np.full((B, S, 576), np.nan, dtype=np.float32)
    hb = host.float().numpy()
    for b in range(B):
        for i, t in enumerate(sel[b][sel[b] >= 0]):
            slot[b, t] = 1 + i
            hot[b, 1 + i] = hb[b, t]
    q = torch.from_numpy(g.normal(size=(B, Hq, 576)).astype(np.float32)).to(torch.bfloat16).cuda()
    seq = torch.tensor(valid, dtype=torch.int32, device="cuda")
    aa = isa.attn_args(q, None, n=n, d_v=512, sm_scale=576 ** -0.5, seq_lens=seq,
                       hot_slot=torch.from_numpy(slot).cuda(),
                       hot_kv=torch.from_numpy(hot).to(torch.bfloat16).cuda(), host_kv=host)
    out = torch.empty((B, Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = isa.workspace(isa.sparse_workspace_size(None, aa, k))
    isa.sparse_gather_attn_decode(aa, torch.from_numpy(sel).cuda(), 1, k, 1, out, lse, ws)
    torch.cuda.synchronize()
    qn = O.decode_bf16(_bits(q))
    R = _bits(host)
    for b in range(B):
        toks = O.expand_selection(sel[b], 1, valid[b])
        keys = O.decode_bf16(R[b, toks])
        ro, rl = O.attention(qn[b], keys, keys[:, :512], 576 ** -0.5)
        _check(out[b].cpu().numpy(), lse[b].cpu().numpy(), ro, rl)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gqa_and_fp32_masked_positions_ignore_nan_rows(dtype):
    print(f"[masked] GQA {dtype}", flush=True)
    g = np.random.default_rng(95)
    B, n, Hkv, G, k = 2, 200, 1 if dtype == "f32" else 2, 8, 40
    valid = [33, 5]
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    Hq = Hkv * G
    K = g.normal(size=(B, n, Hkv, 128)).astype(np.float32)
    V = g.normal(size=(B, n, Hkv, 128)).astype(np.float32)
    Kn, Vn = K.copy(), V.copy()
    Kn[:, 0], Vn[:, 0] = np.nan, np.nan  # token 0 is never selected
    q = torch.from_numpy(g.normal(size=(B, Hq, 128)).astype(np.float32)).to(tdt).cuda()
    kc = torch.from_numpy(Kn).to(tdt).cuda()
    vc = torch.from_numpy(Vn).to(tdt).cuda()
    sel = _selection(g, B, k, valid)
    seq = torch.tensor(valid, dtype=torch.int32, device="cuda")
    aa = isa.attn_args(q, kc, vc, n=n, d_v=128, sm_scale=128 ** -0.5, seq_lens=seq)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = isa.workspace(isa.sparse_workspace_size(None, aa, k))
    isa.sparse_gather_attn_decode(aa, torch.from_numpy(sel).cuda(), 1, k, 1, out, lse, ws)
    torch.cuda.synchronize()
    if dtype == "f32":
        qn = q.cpu().double().numpy()
        Kd, Vd = K.astype(np.float64), V.astype(np.float64)
    else:
        qn = O.decode_bf16(_bits(q))
        Kd = O.decode_bf16(_bits(torch.from_numpy(K).to(torch.bfloat16)))
        Vd = O.decode_bf16(_bits(torch.from_numpy(V).to(torch.bfloat16)))
    for b in range(B):
        toks = O.expand_selection(sel[b], 1, valid[b])
        for h in range(Hkv):
            hs = slice(h * G, (h + 1) * G)
            ro, rl = O.attention(qn[b, hs], Kd[b, toks, h], Vd[b, toks, h], 128 ** -0.5)
            _check(out[b, hs].cpu().numpy(), lse[b, hs].cpu().numpy(), ro, rl)
