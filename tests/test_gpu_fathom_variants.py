"""Fathom scan variants (GPU): a fixed read allocation given by the caller
in place of the reverse water-filling, and bit planes read in place from
pinned host memory (the offloaded index of the Fathom abstract).

Bars as in test_gpu_parity: scores within tau of the oracle, the selection
equal outside the near-tie band, attention within 2e-3 on the GPU's
selection; the host-planes run must equal the device-planes run bit for bit.
"""
import numpy as np
import pytest
import torch

import indexer_top_sparse_amd as isa
from indexer_top_sparse_amd.runner import StepRunner
import synth
from oracle import compare as C

from helpers import arrays, oracle_step

pytestmark = pytest.mark.gpu


def _check_against_oracle(w, inp, r):
    arr = arrays(inp)
    ref = oracle_step(w, arr)
    s = r.index_scores().cpu().numpy()
    g = r.topk.cpu().numpy()
    for b in range(w.B):
        v = w.valid(b)
        for h in range(w.hkv):
            ok, err, tau = C.scores_ok(s[b, h], ref["scores"][b, h], w.k, v)
            assert ok, (b, h, err, tau)
            ok, why = C.selection_ok(g[b, h], ref["sel"][b, h], ref["scores"][b, h], w.k, v)
            assert ok, (b, h, why)
    ref_g = oracle_step(w, arr, sel_in=g.astype(np.int64))
    ok, err = C.attn_ok(r.outs[0].cpu().numpy(), ref_g["out"])
    assert ok, err
    return ref


@pytest.mark.parametrize("kind", ["random", "bits136", "bits68", "none"])
def test_fixed_depth_matches_oracle(kind):
    w = synth.get("fathom_small")
    print(f"[fathom] fixed depth {kind}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    if kind == "random":
        inp["depth_in"] = synth.random_depths(w, "cuda")
    elif kind == "none":
        inp["depth_in"] = torch.zeros((w.B, w.hkv, w.d_qk), dtype=torch.int8, device="cuda")
    else:
        inp["depth_in"] = synth.fixed_depths(w, int(kind[4:]), "cuda")
    r = StepRunner(inp)
    r.run()
    torch.cuda.synchronize()
    ref = _check_against_oracle(w, inp, r)
    depth = torch.empty((w.B, w.hkv, w.d_qk), dtype=torch.int8, device="cuda")
    isa.sparse_read_depth(r.ia, depth)
    torch.cuda.synchronize()
    assert np.array_equal(depth.cpu().numpy().astype(np.int64), ref["depth"])
    assert np.array_equal(ref["depth"], np.clip(inp["depth_in"].cpu().numpy(), 0, 4))


def test_host_resident_planes_bit_identical():
    w = synth.get("fathom_small")
    print("[fathom] planes in pinned host memory", flush=True)
    inp = synth.make_inputs(w, "cuda")
    r_dev = StepRunner(inp)
    r_dev.run()
    s_dev = r_dev.index_scores().clone()
    torch.cuda.synchronize()
    inp_h = dict(inp, planes=synth.pinned_copy(inp["planes"]))
    r_host = StepRunner(inp_h)
    r_host.run()
    s_host = r_host.index_scores()
    torch.cuda.synchronize()
    assert torch.equal(s_dev, s_host)
    assert torch.equal(r_dev.topk, r_host.topk)
    assert torch.equal(r_dev.outs[0], r_host.outs[0])
    _check_against_oracle(w, inp, r_host)
