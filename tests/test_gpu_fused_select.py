"""GPU: the fused step's selection on rows with many exactly tied scores.

In the fused step over latent rows the attention selects each request's top-k
itself, from the candidate list of the fused filter (every unit whose top 12
key bits are at or above the boundary bin).  How many candidates a row has
decides where they are kept: up to 4096 of them arrive with the count, up to
11264 are staged in LDS, and more are read from global memory on every pass.
Equal index keys give equal scores, so the number of candidates can be set
exactly: a seeded subset of the tokens shares one key and every other token
holds the zero key (score 0 below every ReLU sum of the subset's key).  The
exact top-k is then known without any score: the subset's k lowest token ids
(ties go to the lower index), followed by the lowest other ids when the
subset is short.  The selection must equal that list (the oracle's own
float64 scores tie only up to the rounding of its matrix product, so it is
held to the near-tie band rule), and the attention must match the oracle's
attention over it.
"""
import numpy as np
import pytest
import torch

import synth
from indexer_top_sparse_amd.runner import StepRunner
from oracle import compare as C
from oracle import oracle as O

from helpers import arrays, oracle_step

pytestmark = pytest.mark.gpu


def _expected(tied: np.ndarray, valid: int, k: int) -> np.ndarray:
    """Top-k of a row whose tokens in `tied` share the highest score and all
    others score lower and equal: ascending ids, -1 padded."""
    hi = tied[tied < valid]
    lo = np.setdiff1d(np.arange(valid), hi)
    k_eff = min(k, valid)
    take = np.concatenate([hi, lo])[:k_eff] if hi.size < k_eff else hi[:k_eff]
    out = np.full(k, -1, dtype=np.int64)
    out[:k_eff] = np.sort(take)
    return out


# (tied tokens per request, n): 3000 and 6000 candidates stay in LDS (the
# second past the 4096 loaded with the count), 15000 and all 20000 tokens
# exceed the 11264 staged and are read from global memory
@pytest.mark.parametrize("n_tied", [3000, 6000, 15000, 20000])
def test_fused_select_exact_ties(n_tied):
    n, k = 20000, 2048
    w = synth.get("lightning_small").with_(name=f"ties_{n_tied}", B=2, n=n, k=k,
                                           seq_lens=(n, 17001), page=64, seed=4100 + n_tied)
    print(f"[fused select] {n_tied} tied tokens of n={n}, k={k}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    g = np.random.default_rng(4200 + n_tied)
    tied = []
    for b in range(w.B):
        t = np.sort(g.choice(n, size=n_tied, replace=False))
        tied.append(t)
        mask = torch.zeros(n, dtype=torch.bool)
        mask[torch.from_numpy(t)] = True
        mask = mask.cuda()
        key0 = inp["k8"][b, t[0]].clone()
        s0 = inp["k_scale"][b, t[0]].clone()
        inp["k8"][b] = torch.where(mask[:, None], key0[None, :], torch.zeros_like(key0)[None, :])
        inp["k_scale"][b] = s0
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    gsel = r.topk.cpu().numpy()
    arr = arrays(inp)
    ref = oracle_step(w, arr)
    for b in range(w.B):
        valid = w.valid(b)
        # the tied score must be above the others, or the construction is void
        rest = np.setdiff1d(np.arange(valid), tied[b])
        if rest.size:
            assert ref["scores"][b, 0][tied[b][0]] > ref["scores"][b, 0][rest[0]]
        exp = _expected(tied[b], valid, k)
        assert np.array_equal(gsel[b, 0].astype(np.int64), exp), b
        # the oracle's float64 sums of equal rows differ in the last bits
        # (the library product rounds rows at different places of the
        # matrix differently), so its own top-k breaks the ties arbitrarily;
        # it still has to agree under the near-tie band rule
        ref_s = ref["scores"][b, 0]
        tv = tied[b][tied[b] < valid]
        assert np.ptp(ref_s[tv]) <= 1e-12 * abs(ref_s[tv[0]]), b
        ok, why = C.selection_ok(gsel[b, 0], O.topk(ref_s, k, valid), ref_s, k, valid)
        assert ok, (b, why)
    ref_g = oracle_step(w, arr, sel_in=gsel.astype(np.int64))
    ok, err = C.attn_ok(r.outs[0].cpu().numpy(), ref_g["out"])
    assert ok, err
