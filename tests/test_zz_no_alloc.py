"""GPU: the no-allocation step (sparse_decode_step_noalloc) against the step
with a caller workspace (sparse_decode_step), called through the C ABI.

Two calls in a row on the fixed scratch, the second with a smaller input, so
that the second runs on scratch the first has filled; each must give the
same selection, outputs and log-sum-exp as the workspace step, bit for bit
(both run the same kernels in the same order), and the first call's input
is run once more at the end.  The workloads are the lightning indexer
(paged latent rows; also at a length where the attention makes the
selection itself) and the Fathom scan (per-KV-head selections).
"""
import pytest
import torch

import indexer_top_sparse_amd as isa
from indexer_top_sparse_amd.runner import StepRunner
import synth

pytestmark = pytest.mark.gpu


def _both(w):
    print(f"[noalloc] {w.name} B={w.B} n={w.n} k={w.k}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    r = StepRunner(inp)
    r.run()
    aa = r.layer_args[0][0]
    topk = torch.full_like(r.topk, -7)
    out = torch.full_like(r.outs[0], float("nan"))
    lse = torch.full_like(r.lses[0], float("nan"))
    isa.sparse_decode_step_noalloc(r.ia, aa, w.k, topk, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(topk, r.topk)
    assert torch.equal(out, r.outs[0])
    assert torch.equal(lse, r.lses[0])


def _workload(kind):
    if kind == "lightning_fused":
        # past the select-only size, so the attention makes the selection;
        # its half-size second call takes the select kernel instead
        return synth.get("lightning_small").with_(name=kind, n=20000, k=2048,
                                                  seq_lens=(20000, 17001, 300), seed=2102)
    return synth.get(f"{kind}_small")


@pytest.mark.parametrize("kind", ["lightning", "lightning_fused", "fathom"])
def test_noalloc_matches_workspace_step(kind):
    big = _workload(kind)
    small = big.with_(B=big.B - 1, n=big.n // 2, k=big.k // 2,
                      seq_lens=tuple(min(v, big.n // 2) - 7 * i
                                     for i, v in enumerate(big.seq_lens[:big.B - 1])),
                      seed=big.seed + 1)
    _both(big)
    _both(small)
    _both(big)


def test_noalloc_full_size_lightning_128k():
    """The 128K batch fits the fixed scratch (88.5 MiB of 128 MiB)."""
    _both(synth.get("lightning_128k"))
