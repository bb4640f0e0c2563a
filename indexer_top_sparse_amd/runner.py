"""Map a decode-step input set onto the C-ABI calls (marshalling only).

``StepRunner(inputs)`` takes the tensors of one decode step (keys as in
``synth.make_inputs``: q_idx/head_w/k8/k_scale/kv_pool/page_table for the
lightning kind, q/k_cache/v_cache for the dot kind, q_idx/k_idx/layers for
the block kind, q/planes/chan_*/k_cache/v_cache (+ optional depth_in, and
planes may be pinned host memory) for the Fathom kind), builds
the argument structs, output buffers and workspace once, and ``run()``
enqueues one whole step: ``sparse_decode_step`` and, for workloads whose
later layers reuse the selection, ``sparse_gather_attn_decode`` per extra
layer.  It allocates nothing inside ``run()``.
"""
from __future__ import annotations

import torch

from . import (attn_args, bitplane_index_args, dot_index_args,
               lightning_index_args, sparse_decode_step,
               sparse_gather_attn_decode, sparse_index_score,
               sparse_workspace_size, workspace)


class StepRunner:
    def __init__(self, inp: dict, hot: dict | None = None, device="cuda"):
        w = inp["workload"]
        self.w = w
        self.inp = inp
        self.hot = hot
        B, n, k = w.B, w.n, w.k
        seq = inp.get("seq_lens")
        self.layer_args = []
        if w.kind == "dot":
            keys = inp["k_cache"][:, :, 0, :]
            self.ia = dot_index_args(inp["q"], keys, 1, seq)
            self.layer_args.append((attn_args(inp["q"], inp["k_cache"], inp["v_cache"],
                                              n=n, d_v=w.d_v, sm_scale=w.sm_scale,
                                              seq_lens=seq), inp["q"].shape[1]))
            self.unit, self.rows = 1, 1
        elif w.kind == "lightning":
            self.ia = lightning_index_args(inp["q_idx"], inp["head_w"], inp["k8"],
                                           inp["k_scale"], seq)
            if hot is not None:
                aa = attn_args(inp["q"], None, n=n, d_v=w.d_v, sm_scale=w.sm_scale,
                               seq_lens=seq,
                               hot_slot=hot["hot_slot"], hot_kv=hot["hot_kv"],
                               host_kv=hot["host_kv"])
            elif "kv_pool" in inp:
                aa = attn_args(inp["q"], inp["kv_pool"], n=n, d_v=w.d_v,
                               sm_scale=w.sm_scale, seq_lens=seq,
                               page_table=inp["page_table"], page_size=w.page)
            else:
                aa = attn_args(inp["q"], inp["kv"], n=n, d_v=w.d_v, sm_scale=w.sm_scale,
                               seq_lens=seq)
            self.layer_args.append((aa, w.hq))
            self.unit, self.rows = 1, 1
        elif w.kind == "block":
            self.ia = dot_index_args(inp["q_idx"], inp["k_idx"], w.block, seq)
            for layer in inp["layers"]:
                self.layer_args.append((attn_args(layer["q"], layer["k_cache"],
                                                  layer["v_cache"], n=n, d_v=w.d_v,
                                                  sm_scale=w.sm_scale, seq_lens=seq),
                                        w.hq))
            self.unit, self.rows = w.block, 1
        elif w.kind == "fathom":
            self.ia = bitplane_index_args(inp["q"], inp["planes"], inp["chan_zero"],
                                          inp["chan_scale"], inp["chan_var"], w.budget,
                                          n, seq, depth_in=inp.get("depth_in"))
            self.layer_args.append((attn_args(inp["q"], inp["k_cache"], inp["v_cache"],
                                              n=n, d_v=w.d_v, sm_scale=w.sm_scale,
                                              seq_lens=seq), w.hq))
            self.unit, self.rows = 1, w.hkv
        else:
            raise ValueError(w.kind)
        self.n_units = (n + self.unit - 1) // self.unit
        self.topk = torch.empty((B, self.rows, k), dtype=torch.int32, device=device)
        self.outs = [torch.empty((B, hq, w.d_v), dtype=torch.float32, device=device)
                     for _, hq in self.layer_args]
        self.lses = [torch.empty((B, hq), dtype=torch.float32, device=device)
                     for _, hq in self.layer_args]
        need = sparse_workspace_size(self.ia, self.layer_args[0][0], k)
        for aa, _ in self.layer_args[1:]:
            need = max(need, sparse_workspace_size(None, aa, k * self.unit))
        self.ws = workspace(need, device)
        self.scores = None

    def run(self, stream=None) -> None:
        k = self.w.k
        aa0 = self.layer_args[0][0]
        sparse_decode_step(self.ia, aa0, k, self.topk, self.outs[0], self.lses[0],
                           self.ws, stream)
        for i in range(1, len(self.layer_args)):
            sparse_gather_attn_decode(self.layer_args[i][0], self.topk, self.rows, k,
                                      self.unit, self.outs[i], self.lses[i], self.ws,
                                      stream)

    def index_scores(self, stream=None) -> torch.Tensor:
        """The index scores alone, [B][R][n_units] (sparse_index_score)."""
        if self.scores is None:
            self.scores = torch.empty((self.w.B, self.rows, self.n_units),
                                      dtype=torch.float32, device=self.topk.device)
        sparse_index_score(self.ia, self.scores, self.ws, stream)
        return self.scores
