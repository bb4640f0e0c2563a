"""GPU: whole decode steps at seeded random shapes of every score kind,
against the oracle.

Twenty shapes are drawn once from fixed seeds around the small workloads:
batch 1..4, context lengths that end mid-tile, valid lengths down to a
single token, k from 1 up to more than a request's valid units, 32 or 64
index heads, 64..256 latent attention heads, paged and contiguous latent
rows, and Fathom bit budgets from 8 to the full 512.  Each step is checked
as in the other parity tests: scores within tau, the selection equal
outside the near-tie band, the standalone top-k bit-exact on the GPU's own
scores, and attention within 2e-3 of the oracle's attention over the GPU's
selection.
"""
import numpy as np
import pytest
import torch

import indexer_top_sparse_amd as isa
from indexer_top_sparse_amd.runner import StepRunner
import synth
from oracle import compare as C
from oracle import oracle as O

from helpers import arrays, oracle_step, valid_units

pytestmark = pytest.mark.gpu


def _shapes():
    g = np.random.default_rng(20261203)
    out = []
    for i in range(4):
        B = int(g.integers(1, 5))
        n = int(g.integers(300, 7000))
        seq = tuple(int(x) for x in g.integers(1, n + 1, size=B))
        out.append(synth.get("lightning_small").with_(
            name=f"rand_lightning_{i}", B=B, n=n, seq_lens=seq,
            k=int(g.choice([1, 64, 300, 1024])), idx_heads=int(g.choice([32, 64])),
            hq=int(g.choice([64, 128, 192, 256])), page=int(g.choice([0, 64])),
            seed=3100 + i))
    for i in range(4):
        B = int(g.integers(1, 5))
        n = int(g.integers(200, 6000))
        seq = tuple(int(x) for x in g.integers(1, n + 1, size=B))
        out.append(synth.get("block_sparse_small").with_(
            name=f"rand_block_{i}", B=B, n=n, seq_lens=seq,
            k=int(g.choice([1, 4, 16, 200])), seed=3200 + i))
    for i in range(4):
        B = int(g.integers(1, 5))
        n = int(g.integers(100, 5000))
        seq = tuple(int(x) for x in g.integers(1, n + 1, size=B))
        out.append(synth.get("tiny_fp32_small").with_(
            name=f"rand_dot_{i}", B=B, n=n, seq_lens=seq,
            k=int(g.choice([1, 17, 256, 600])), seed=3300 + i))
    for i in range(4):
        B = int(g.integers(1, 3))
        n = int(g.integers(500, 40000))
        seq = tuple(int(x) for x in g.integers(1, n + 1, size=B))
        out.append(synth.get("fathom_small").with_(
            name=f"rand_fathom_{i}", B=B, n=n, seq_lens=seq,
            k=int(g.choice([1, 100, 300, 2048])), budget=int(g.choice([8, 92, 300, 512])),
            seed=3400 + i))
    # latent rows long enough that the attention selects from the fused
    # filter's candidates (a separate generator, so the shapes above stay)
    g2 = np.random.default_rng(20261204)
    for i in range(4):
        B = int(g2.integers(1, 4))
        n = int(g2.integers(12289, 60000))
        seq = tuple(int(x) for x in g2.integers(1, n + 1, size=B))
        out.append(synth.get("lightning_small").with_(
            name=f"rand_lightning_fused_{i}", B=B, n=n, seq_lens=seq,
            k=int(g2.choice([64, 300, 2048, 3000])), idx_heads=int(g2.choice([32, 64])),
            hq=int(g2.choice([64, 128, 256])), page=int(g2.choice([0, 64])),
            seed=3600 + i))
    return out


def _edges():
    """Boundary shapes: one tile plus one token, a span plus one, k at or above
    the valid units, a single block or word, rows just past the select-only
    size, requests with no valid token."""
    L = synth.get("lightning_small")
    Bk = synth.get("block_sparse_small")
    T = synth.get("tiny_fp32_small")
    F = synth.get("fathom_small")
    return [
        L.with_(name="edge_lightning_33", B=5, n=33, k=32, seq_lens=(33, 1, 32, 17, 33),
                page=64, seed=3501),
        L.with_(name="edge_lightning_span1", B=2, n=8193, k=8193, seq_lens=(8193, 4097),
                page=0, seed=3502),
        Bk.with_(name="edge_block_one", B=2, n=64, k=4, seq_lens=(64, 5), seed=3503),
        Bk.with_(name="edge_block_129", B=3, n=129, k=3, seq_lens=(129, 128, 65), seed=3504),
        T.with_(name="edge_dot_one", B=2, n=1, k=1, seq_lens=(1, 1), seed=3505),
        T.with_(name="edge_dot_12289", B=2, n=12289, k=600, seq_lens=(12289, 12288), seed=3506),
        F.with_(name="edge_fathom_31", B=2, n=31, k=5, budget=92, seq_lens=(31, 3), seed=3507),
        F.with_(name="edge_fathom_32769", B=1, n=32769, k=2048, budget=300, seq_lens=(32769,),
                seed=3508),
        # latent rows past the select-only size: the attention selects from
        # the fused filter's candidates itself (one row shorter than k pads)
        L.with_(name="edge_lightning_fused_12289", B=3, n=12289, k=2048,
                seq_lens=(12289, 2000, 6001), page=64, seed=3509),
        L.with_(name="edge_lightning_fused_40000", B=2, n=40000, k=300, hq=256,
                seq_lens=(40000, 23457), page=0, seed=3510),
        L.with_(name="edge_lightning_fused_k4096", B=2, n=30000, k=4096, hq=64,
                seq_lens=(29999, 4097), page=64, seed=3511),
        L.with_(name="edge_lightning_fused_k1", B=3, n=16385, k=1, hq=192,
                seq_lens=(16385, 1, 12289), page=0, seed=3512),
        # a request with no valid token: an all -1 selection, output 0,
        # log-sum-exp -inf (every kind; latent rows on both select paths)
        L.with_(name="edge_empty_lightning", B=2, n=500, k=64, seq_lens=(0, 500), page=64,
                seed=3513),
        L.with_(name="edge_empty_lightning_fused", B=2, n=13000, k=512, seq_lens=(13000, 0),
                page=64, seed=3514),
        Bk.with_(name="edge_empty_block", B=2, n=700, k=4, seq_lens=(0, 700), seed=3515),
        T.with_(name="edge_empty_dot", B=2, n=600, k=17, seq_lens=(600, 0), seed=3516),
        F.with_(name="edge_empty_fathom", B=2, n=3000, k=100, seq_lens=(0, 3000), seed=3517),
        # a zero bit budget: no plane is read, every score is the constant
        F.with_(name="edge_fathom_budget0", B=1, n=5000, k=100, budget=0, seq_lens=(4999,),
                seed=3518),
    ]


SHAPES = _shapes() + _edges()


@pytest.mark.parametrize("w", SHAPES, ids=[w.name for w in SHAPES])
def test_random_step_matches_oracle(w):
    print(f"[random] {w.name} B={w.B} n={w.n} k={w.k} seq={w.seq_lens} hq={w.hq} "
          f"page={w.page} budget={w.budget} idx_heads={w.idx_heads}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    arr = arrays(inp)
    ref = oracle_step(w, arr)
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    g = r.topk.cpu().numpy()
    s = r.index_scores().clone()
    torch.cuda.synchronize()
    sn = s.cpu().numpy()
    for b in range(w.B):
        v = valid_units(w, b)
        for h in range(g.shape[1]):
            ok, err, tau = C.scores_ok(sn[b, h], ref["scores"][b, h], w.k, v)
            assert ok, (b, h, "scores", err, tau)
            ok, why = C.selection_ok(g[b, h], ref["sel"][b, h], ref["scores"][b, h], w.k, v)
            assert ok, (b, h, why)
    # the standalone top-k, bit-exact on the GPU's own scores
    rows = s.shape[0] * s.shape[1]
    flat = s.view(rows, -1)
    vu = None
    if inp.get("seq_lens") is not None:
        vu = ((inp["seq_lens"] + w.block - 1) // w.block).to(torch.int32)
    idx = torch.empty((rows, w.k), dtype=torch.int32, device="cuda")
    ws = isa.workspace(isa.sparse_topk_workspace_size(rows, flat.shape[1], w.k))
    isa.sparse_topk(flat, w.k, idx, None, vu, s.shape[1], ws)
    torch.cuda.synchronize()
    sc = flat.cpu().numpy().astype(np.float64)
    gi = idx.cpu().numpy()
    for row in range(rows):
        exp = O.topk(sc[row], w.k, valid_units(w, row // s.shape[1]))
        assert np.array_equal(gi[row], exp), ("topk", row)
    # the step's own selection (select kernel, or the latent attention's fused
    # select) is the same exact top-k of the same scores
    assert np.array_equal(g.reshape(rows, -1), gi), "step selection"
    # attention over the GPU's own selection
    ref_g = oracle_step(w, arr, sel_in=g.astype(np.int64))
    outs = ref_g["layers"][0]["out"] if w.kind == "block" else ref_g["out"]
    ok, err = C.attn_ok(r.outs[0].cpu().numpy(), outs)
    assert ok, ("attention", err)
