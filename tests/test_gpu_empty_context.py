"""GPU: a decode step over an empty context (n = 0).

With no cached token there is nothing to score or select and no row to
attend: every request's selection is all -1, every output row is 0 and every
log-sum-exp is -inf, as the oracle gives (softmax over an empty set).  The
KV tensors are empty, so their pointers reach the library as NULL, which it
accepts for n = 0 because no row is ever read (bf16 K/V rows with a value
cache are told from latent rows by a non-NULL v_cache, so that layout is not
among these cases).
"""
import numpy as np
import pytest
import torch

import synth
from indexer_top_sparse_amd.runner import StepRunner

from helpers import arrays, oracle_step

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("base,page", [("lightning_small", 64), ("lightning_small", 0),
                                       ("tiny_fp32_small", 0)])
def test_empty_context_step(base, page):
    w = synth.get(base).with_(name=f"{base}_n0", B=2, n=0, k=8, seq_lens=None, page=page,
                              seed=3540)
    print(f"[empty] {base} page={page}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    ref = oracle_step(w, arrays(inp))
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    assert np.all(r.topk.cpu().numpy() == -1)
    assert np.all(ref["sel"] == -1)
    for out, lse in zip(r.outs, r.lses):
        assert torch.count_nonzero(out).item() == 0
        assert bool(torch.all(torch.isneginf(lse)))
    assert np.all(ref["out"] == 0)
