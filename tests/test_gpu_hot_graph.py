"""GPU: hot-buffer miss fetch and HIP-graph replay of whole steps.

* With a 20 % or a 40 % miss rate the step fetches the missing selected rows
  from pinned host memory; its output must equal the oracle's attention, and
  be bit-identical to the same step with every selected row hot
  ("XM-Sparse" blog: fixed miss rates, misses fetched over PCIe into HBM).
* A captured step replayed several times, with eager work and
  synchronisation in between, must reproduce the eager result bit for bit
  on every replay (also for a latent step long enough that its attention
  makes the top-k selection itself).
"""
import numpy as np
import pytest
import torch

import synth
from synth.gen import build_hot_buffer
from indexer_top_sparse_amd.runner import StepRunner
from oracle import compare as C

from helpers import arrays, oracle_step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=[0.2, 0.4])
def hot_case(request):
    """The hot-buffer workload at the pages' two miss rates (20 % and 40 %)."""
    w = synth.get("hot_small").with_(miss_rate=request.param)
    print(f"[hot] workload={w.name} miss_rate={w.miss_rate}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    arr = arrays(inp)
    ref = oracle_step(w, arr)
    sel = torch.from_numpy(ref["sel"][:, 0].astype(np.int32)).cuda()
    hot_miss = build_hot_buffer(inp, sel, "cuda")
    hot_all = build_hot_buffer(dict(inp, workload=w.with_(miss_rate=0.0)), sel, "cuda")
    return w, inp, arr, ref, hot_miss, hot_all


def test_hot_buffer_misses_counted(hot_case):
    w, inp, arr, ref, hot_miss, hot_all = hot_case
    slot = hot_miss["hot_slot"].cpu().numpy()
    for b in range(w.B):
        s = ref["sel"][b, 0]
        s = s[s >= 0]
        missing = int((slot[b, s] < 0).sum())
        assert missing == hot_miss["n_miss"][b] == int(np.floor(w.miss_rate * s.size + 0.5))
    assert np.all(hot_all["n_miss"] == 0)


def test_hot_step_matches_oracle_and_no_miss_run(hot_case):
    w, inp, arr, ref, hot_miss, hot_all = hot_case
    r_miss = StepRunner(inp, hot=hot_miss)
    r_all = StepRunner(inp, hot=hot_all)
    r_miss.run()
    r_all.run()
    torch.cuda.synchronize()
    g = r_miss.topk.cpu().numpy().astype(np.int64)
    for b in range(w.B):
        ok, why = C.selection_ok(g[b, 0], ref["sel"][b, 0], ref["scores"][b, 0], w.k,
                                 w.valid(b))
        assert ok, why
    ref_g = oracle_step(w, arr, sel_in=g)
    ok, err = C.attn_ok(r_miss.outs[0].cpu().numpy(), ref_g["out"])
    assert ok, err
    assert torch.equal(r_miss.outs[0], r_all.outs[0])
    assert torch.equal(r_miss.lses[0], r_all.lses[0])


def _graph_workload(name):
    if name == "lightning_fused":
        # past the select-only size: the attention selects in its prologue
        return synth.get("lightning_small").with_(name=name, n=20000, k=2048,
                                                  seq_lens=(20000, 17001, 300))
    return synth.get(name)


@pytest.mark.parametrize("name", ["lightning_small", "lightning_fused", "block_sparse_small",
                                  "fathom_small"])
def test_graph_replays_match_eager(name):
    w = _graph_workload(name)
    print(f"[graph] workload={name}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in r.outs + r.lses + [r.topk]]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.run()
    for rep in range(4):
        for t in r.outs + r.lses + [r.topk]:
            t.fill_(7.0 if t.dtype.is_floating_point else 7)
        _ = torch.randn(1000, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        now = r.outs + r.lses + [r.topk]
        for a, b in zip(eager, now):
            assert torch.equal(a, b), (name, rep)
