"""GPU: latent (MLA) attention over a given selection at shapes the
workloads do not reach, against the oracle's exact attention.

Latent rows hold 576 bf16 values; the keys are the whole row and the values
its first 512.  The cases cover 64, 192 and 256 query heads (one, three and
four 64-head groups per request), contiguous and paged rows (a shuffled page
pool), ragged valid lengths, padding (-1) entries, a single split and
several.  Every output element and log-sum-exp is compared with the oracle
(bf16 rows decoded exactly, float64 softmax).
"""
import numpy as np
import pytest
import torch

import indexer_top_sparse_amd as isa
from oracle import compare as C
from oracle import oracle as O

pytestmark = pytest.mark.gpu

CASES = [
    # (B, n, Hq, k, paged, valid lengths or None, q scale)
    (2, 3000, 64, 500, False, [3000, 1700], 0.3),
    (1, 6000, 192, 2048, True, None, 0.3),
    (3, 4096, 256, 96, True, [4096, 4000, 100], 0.3),
    (1, 2500, 128, 64, False, None, 0.3),      # few tokens: one split
    # a peaked softmax at k = 2048: the logits of every head span more than
    # 8, so the few rows of largest weight decide the output and a wrong or
    # missing row moves it far beyond the bar
    (2, 8192, 128, 2048, True, None, 3.0),
    (1, 5000, 64, 2048, False, [4500], 4.0),
]


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("B,n,Hq,k,paged,valid,qs", CASES,
                         ids=[f"H{c[2]}-k{c[3]}-{'paged' if c[4] else 'flat'}-q{c[6]}"
                              for c in CASES])
def test_mla_attention_matches_oracle(B, n, Hq, k, paged, valid, qs):
    print(f"[mla] B={B} n={n} Hq={Hq} k={k} paged={paged} q scale {qs}", flush=True)
    g = np.random.default_rng(n + Hq + k)
    q = torch.from_numpy(g.normal(size=(B, Hq, 576)).astype(np.float32) * qs).to(torch.bfloat16).cuda()
    rows = g.normal(size=(B, n, 576)).astype(np.float32)
    if paged:
        page = 64
        npg = (n + page - 1) // page
        pad = np.zeros((B, npg * page, 576), dtype=np.float32)
        pad[:, :n] = rows
        perm = g.permutation(B * npg).astype(np.int32)
        pool = np.empty((B * npg, page, 576), dtype=np.float32)
        pool[perm] = pad.reshape(B * npg, page, 576)
        kc = torch.from_numpy(pool).to(torch.bfloat16).cuda()
        pt = torch.from_numpy(perm.reshape(B, npg)).cuda()
    else:
        kc = torch.from_numpy(rows).to(torch.bfloat16).cuda()
        pt = None
    sel = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        pick = np.sort(g.choice(n, size=min(k, n), replace=False))
        row = np.full(k, -1, dtype=np.int32)
        row[: pick.size] = pick
        row[g.choice(k, size=max(1, k // 40), replace=False)] = -1
        sel[b] = row
    seq = None if valid is None else torch.tensor(valid, dtype=torch.int32, device="cuda")
    aa = isa.attn_args(q, kc, None, n=n, d_v=512, sm_scale=576 ** -0.5, page_table=pt,
                       page_size=64 if paged else 0,
                       seq_lens=seq)
    out = torch.empty((B, Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = isa.workspace(isa.sparse_workspace_size(None, aa, k))
    isa.sparse_gather_attn_decode(aa, torch.from_numpy(sel).cuda(), 1, k, 1, out, lse, ws)
    torch.cuda.synchronize()
    qn = O.decode_bf16(_bits(q))
    R = _bits(torch.from_numpy(rows).to(torch.bfloat16))
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    scale = 1.0 / np.sqrt(576.0)
    for b in range(B):
        v = n if valid is None else valid[b]
        toks = O.expand_selection(sel[b], 1, v)
        keys = O.decode_bf16(R[b, toks])
        ro, rl = O.attention(qn[b], keys, keys[:, :512], scale)
        if qs >= 3.0:
            logits = scale * qn[b] @ keys.T
            assert np.all(logits.max(1) - logits.min(1) > 8.0)
        ok, err = C.attn_ok(go[b], ro)
        assert ok, (b, err)
        ok, err = C.attn_ok(gl[b], rl)
        assert ok, (b, "lse", err)
