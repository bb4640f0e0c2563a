"""GPU: GQA attention over a given selection (sparse_gather_attn_decode) at
shapes the workloads do not reach, against the oracle's exact attention.

The cases cover one query head per KV head (G = 1), an odd group (G = 3),
the largest group (G = 16), per-KV-head and shared selections, 64-token
blocks, ragged valid lengths, padding (-1) entries, a selection longer than
one split's 2048 tokens, and a single split.  Every output element and
every log-sum-exp is compared with the oracle (bf16 rows decoded exactly,
float64 softmax), to the attention bar of the other parity tests.
"""
import numpy as np
import pytest
import torch

import indexer_top_sparse_amd as isa
from oracle import compare as C
from oracle import oracle as O

pytestmark = pytest.mark.gpu

CASES = [
    # (B, n, Hkv, G, k, unit, per-KV-head selection, valid lengths or None, q scale)
    (2, 3000, 2, 1, 300, 1, True, [3000, 2100], 1.0),
    (2, 5000, 1, 16, 700, 1, False, None, 1.0),
    (1, 9000, 4, 3, 40, 64, False, [8500], 1.0),
    (3, 2048, 8, 8, 2048, 1, False, None, 1.0),       # every token selected
    (2, 8192, 2, 4, 64, 64, True, [8192, 5000], 1.0),  # 4096 tokens: several splits
    (1, 4000, 2, 8, 64, 1, False, None, 1.0),         # one split
    # a peaked softmax at 2048 selected tokens: logits spanning more than 8
    (2, 8192, 2, 8, 2048, 1, True, None, 3.0),
    (1, 9000, 8, 8, 32, 64, False, [8800], 3.0),
]


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("B,n,Hkv,G,k,unit,per_head,valid,qs", CASES,
                         ids=[f"G{c[3]}-k{c[4]}x{c[5]}-hkv{c[2]}-q{c[8]}" for c in CASES])
def test_gqa_attention_matches_oracle(B, n, Hkv, G, k, unit, per_head, valid, qs):
    print(f"[gqa] B={B} n={n} Hkv={Hkv} G={G} k={k} unit={unit} q scale {qs}", flush=True)
    g = np.random.default_rng(n + 7 * G + k)
    Hq = Hkv * G
    q = torch.from_numpy(g.normal(size=(B, Hq, 128)).astype(np.float32) * qs).to(torch.bfloat16).cuda()
    kc = torch.from_numpy(g.normal(size=(B, n, Hkv, 128)).astype(np.float32)).to(torch.bfloat16).cuda()
    vc = torch.from_numpy(g.normal(size=(B, n, Hkv, 128)).astype(np.float32)).to(torch.bfloat16).cuda()
    n_units = (n + unit - 1) // unit
    sel_heads = Hkv if per_head else 1
    sel = np.empty((B, sel_heads, k), dtype=np.int32)
    for b in range(B):
        for h in range(sel_heads):
            pick = np.sort(g.choice(n_units, size=min(k, n_units), replace=False))
            row = np.full(k, -1, dtype=np.int32)
            row[: pick.size] = pick
            # a few padding entries inside the list
            row[g.choice(k, size=max(1, k // 50), replace=False)] = -1
            sel[b, h] = row
    seq = None if valid is None else torch.tensor(valid, dtype=torch.int32, device="cuda")
    aa = isa.attn_args(q, kc, vc, n=n, d_v=128, sm_scale=128 ** -0.5, seq_lens=seq)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = isa.workspace(isa.sparse_workspace_size(None, aa, k * unit))
    isa.sparse_gather_attn_decode(aa, torch.from_numpy(sel).cuda(), sel_heads, k, unit,
                                  out, lse, ws)
    torch.cuda.synchronize()
    qn = O.decode_bf16(_bits(q))
    K, V = _bits(kc), _bits(vc)
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    scale = 1.0 / np.sqrt(128.0)
    for b in range(B):
        v = n if valid is None else valid[b]
        for h in range(Hkv):
            toks = O.expand_selection(sel[b, h if per_head else 0], unit, v)
            hs = slice(h * G, (h + 1) * G)
            Kh = O.decode_bf16(K[b, toks, h])
            ro, rl = O.attention(qn[b, hs], Kh, O.decode_bf16(V[b, toks, h]), scale)
            if qs >= 3.0:
                logits = scale * qn[b, hs] @ Kh.T
                assert np.all(logits.max(1) - logits.min(1) > 8.0)
            ok, err = C.attn_ok(go[b, hs], ro)
            assert ok, (b, h, err)
            ok, err = C.attn_ok(gl[b, hs], rl)
            assert ok, (b, h, "lse", err)
