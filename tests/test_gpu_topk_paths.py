"""GPU: the standalone top-k (sparse_topk) on each of its kernel paths.

Rows of at most 12288 units take the select kernel alone, which stages the
whole row and finds the boundary bin itself.  Longer rows of up to 64
histogram parts (4096 units each, so n_units <= 262144) take the fused
filter, which finds the boundary bin from the parts' coarse counts and
writes one candidate list per row; longer rows still take the bin /
per-chunk filter kernels.  Each case here is checked element by
element against the oracle's exact top-k (ties to the lower index, output
ascending, -1 padding past the valid units), on score patterns chosen to
stress the bin search and the per-part candidate offsets: heavy ties,
every winner in the last part, a single distinct value, signed zeros and
infinities, and ragged valid lengths.
"""
import numpy as np
import pytest
import torch

import indexer_top_sparse_amd as isa
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _scores(kind, rows, n, seed):
    g = np.random.default_rng(seed)
    if kind == "ties":  # few distinct values: long runs of equal keys
        s = np.round(g.normal(size=(rows, n)) * 4.0) / 4.0
    elif kind == "rising":  # the largest keys all sit in the last part
        s = np.tile(np.linspace(-3.0, 5.0, n), (rows, 1)) + g.normal(size=(rows, n)) * 1e-3
    elif kind == "constant":
        s = np.full((rows, n), 0.5)
    elif kind == "special":  # signed zeros (equal keys) and infinities
        s = g.choice(np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf]), size=(rows, n))
    else:
        s = g.normal(size=(rows, n))
    return s.astype(np.float32)


CASES = [
    # (pattern, rows, n_units, k, valid per row or None)
    ("ties", 2, 262144, 2048, [262144, 200001]),     # 64 parts: fused filter
    ("ties", 2, 262145, 2048, [262145, 200001]),     # 65 parts: bin + chunk filter
    ("rising", 3, 131072, 2048, None),
    ("rising", 2, 300000, 2048, None),
    ("constant", 2, 9000, 512, [9000, 100]),         # all tied; k > valid pads
    ("special", 2, 70000, 777, [70000, 12345]),
    ("normal", 4, 4096, 1, None),
    ("normal", 3, 5001, 5001, [5001, 4000, 0]),      # k = n; an empty row
    # rows of at most 12288 units take the select kernel alone
    ("ties", 3, 12288, 700, [12288, 12287, 600]),    # the longest such row
    ("ties", 2, 12289, 700, None),                   # one unit more: fused filter
    ("special", 2, 3000, 64, [3000, 17]),
    ("rising", 2, 1280, 32, None),
]


@pytest.mark.parametrize("pattern,rows,n,k,valid", CASES,
                         ids=[f"{c[0]}-{c[2]}-{c[3]}" for c in CASES])
def test_topk_paths_match_oracle(pattern, rows, n, k, valid):
    print(f"[topk] {pattern} rows={rows} n={n} k={k} valid={valid}", flush=True)
    s = _scores(pattern, rows, n, seed=n + k)
    scores = torch.from_numpy(s).cuda()
    vu = None if valid is None else torch.tensor(valid, dtype=torch.int32, device="cuda")
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    val = torch.empty((rows, k), dtype=torch.float32, device="cuda")
    ws = isa.workspace(isa.sparse_topk_workspace_size(rows, n, k))
    isa.sparse_topk(scores, k, idx, val, vu, 1, ws)
    torch.cuda.synchronize()
    gi, gv = idx.cpu().numpy(), val.cpu().numpy()
    for r in range(rows):
        v = n if valid is None else valid[r]
        exp = O.topk(s[r].astype(np.float64), k, v)
        assert np.array_equal(gi[r], exp), (r, np.nonzero(gi[r] != exp)[0][:8])
        take = exp >= 0
        got, want = gv[r][take], s[r][exp[take]]
        # equal keys: +0 and -0 map to the same key, so compare as values
        assert np.array_equal(got, want), r
        assert np.all(np.isneginf(gv[r][~take])), r


def test_topk_repeat_is_bit_identical():
    s = _scores("ties", 2, 262144, seed=3)
    scores = torch.from_numpy(s).cuda()
    ws = isa.workspace(isa.sparse_topk_workspace_size(2, 262144, 2048))
    outs = []
    for _ in range(2):
        idx = torch.empty((2, 2048), dtype=torch.int32, device="cuda")
        isa.sparse_topk(scores, 2048, idx, None, None, 1, ws)
        torch.cuda.synchronize()
        outs.append(idx.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
