"""GPU: least-recently-used hot-buffer replacement (sparse_hot_update) after
a step, against the oracle (oracle/hot.py), bit for bit.

* Attention-only steps (sparse_gather_attn_decode, which fetches the missed
  rows into the workspace) on a random hot-buffer state -- resident tokens,
  empty slots, stamps from -1 up -- then a sequence of updates with
  overlapping selections, padding entries and ragged valid lengths, at
  several buffer sizes, including buffers smaller than a selection (misses
  that stay out) and ties of stamps.  After every update the token -> slot
  map, the slot -> token map, the stamps and every hot row are compared with
  the oracle's.
* 64-token selection units (the tokens of the selected blocks), more misses
  than free slots.
* The fused step (sparse_decode_step, lightning indexer) on the small
  hot-buffer workload, then the update with the step's own selection.
* The buffer and selection sizes of the hot-buffer workloads (4096 slots,
  2048 selected tokens, 2048 prefetch candidates), beside small ones.
* The prefetch (sparse_hot_prefetch) after each update of a sequence:
  candidate lists that mix resident tokens, new tokens, padding and tokens
  past the valid length, more candidates than free slots, against the
  oracle's hot_prefetch.
"""
import numpy as np
import pytest
import torch

import indexer_top_sparse_amd as isa
import synth
from synth.gen import build_hot_buffer
from indexer_top_sparse_amd.runner import StepRunner
from oracle.hot import hot_prefetch, hot_update

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_all(hs, st, ss, hk, host, sel, valid, step):
    out = [np.empty_like(x) for x in (hs, st, ss, hk)]
    for b in range(hs.shape[0]):
        r = hot_update(hs[b], st[b], ss[b], hk[b], host[b], sel[b], valid[b], step)
        for o, x in zip(out, r):
            o[b] = x
    return out


def _check(state, ref, where):
    hs, st, ss, hk = state
    names = ("hot_slot", "slot_token", "slot_stamp", "hot_kv")
    got = (hs.cpu().numpy(), st.cpu().numpy(), ss.cpu().numpy(), _bits(hk))
    for name, g, r in zip(names, got, ref):
        bad = np.argwhere(g != r)
        assert bad.size == 0, (where, name, bad[:5].tolist())


CASES = [
    # (B, n, slots, k, steps, valid lengths)
    (3, 3000, 1024, 512, 4, [3000, 2500, 700]),
    (2, 5000, 300, 256, 3, None),       # a buffer a little larger than a selection
    (2, 2000, 64, 100, 5, [2000, 90]),  # fewer slots than selected: misses stay out
    # the measured sizes: 4096 slots and 2048 selected tokens, so the update
    # runs its multi-pass paths (miss compaction, eligible count, victim scan
    # over more slots and selections than one pass of its 1024 threads)
    (2, 16384, 4096, 2048, 3, [16384, 12000]),
]


@pytest.mark.parametrize("B,n,S,k,steps,valid", CASES,
                         ids=[f"S{c[2]}-k{c[3]}" for c in CASES])
def test_hot_update_sequence_matches_oracle(B, n, S, k, steps, valid):
    print(f"[hot-update] B={B} n={n} slots={S} k={k} steps={steps}", flush=True)
    g = np.random.default_rng(S + k + n)
    Hq, d = 64, 576
    vl = np.array(valid if valid is not None else [n] * B)
    host_f = g.normal(size=(B, n, d)).astype(np.float32)
    host = torch.from_numpy(host_f).to(torch.bfloat16).pin_memory()
    host_bits = host.view(torch.int16).numpy().view(np.uint16)
    # a random starting state: some resident tokens, some empty slots
    hs = np.full((B, n), -1, np.int32)
    st = np.full((B, S), -1, np.int32)
    ss = np.full((B, S), -1, np.int32)
    hk = np.zeros((B, S, d), np.uint16)
    for b in range(B):
        m = int(g.integers(0, min(S, vl[b]) + 1))
        toks = g.choice(vl[b], size=m, replace=False)
        slots = g.choice(S, size=m, replace=False)
        for t, s in zip(toks, slots):
            hs[b, t], st[b, s], ss[b, s] = s, t, int(g.integers(-1, 4))
            hk[b, s] = host_bits[b, t]
    dev = "cuda"
    hot_slot = torch.from_numpy(hs).to(dev)
    slot_token = torch.from_numpy(st).to(dev)
    slot_stamp = torch.from_numpy(ss).to(dev)
    hot_kv = torch.from_numpy(hk.view(np.int16)).to(dev).view(torch.bfloat16)
    q = torch.from_numpy(g.normal(size=(B, Hq, d)).astype(np.float32) * 0.1).to(torch.bfloat16).to(dev)
    seq = torch.from_numpy(vl.astype(np.int32)).to(dev)
    aa = isa.attn_args(q, None, n=n, d_v=512, sm_scale=d ** -0.5, seq_lens=seq,
                       hot_slot=hot_slot, hot_kv=hot_kv, host_kv=host)
    ws = isa.workspace(isa.sparse_workspace_size(None, aa, k))
    out = torch.empty((B, Hq, 512), dtype=torch.float32, device=dev)
    prev = [np.array([], dtype=np.int64) for _ in range(B)]
    state = [hs, st, ss, hk]
    for i in range(steps):
        step = 10 + i
        sel = np.full((B, k), -1, np.int32)
        for b in range(B):
            # half of the last selection again, the rest new
            keep = prev[b][: prev[b].size // 2]
            fresh = g.choice(n, size=k, replace=False)
            pick = np.unique(np.concatenate([keep, fresh]))[:k]
            pick = np.sort(g.permutation(pick)[: int(g.integers(k // 2, k + 1))])
            sel[b, : pick.size] = pick
            prev[b] = pick[pick < vl[b]]
        sel_t = torch.from_numpy(sel).to(dev)
        isa.sparse_gather_attn_decode(aa, sel_t, 1, k, 1, out, None, ws)
        isa.sparse_hot_update(None, aa, sel_t, k, 1, S, step, slot_token, slot_stamp, ws)
        torch.cuda.synchronize()
        state = _oracle_all(state[0], state[1], state[2], state[3], host_bits, sel, vl, step)
        _check((hot_slot, slot_token, slot_stamp, hot_kv), state, f"step {step}")


def test_hot_update_block_units():
    # 64-token selection units: the misses are the tokens of the selected
    # blocks (block order, then token order) that the buffer does not hold
    B, n, S, kb, unit, d, Hq = 2, 3000, 512, 12, 64, 576, 64
    print(f"[hot-update] block units B={B} n={n} slots={S} blocks={kb}", flush=True)
    g = np.random.default_rng(77)
    vl = np.array([3000, 1500])
    host = torch.from_numpy(g.normal(size=(B, n, d)).astype(np.float32)).to(torch.bfloat16).pin_memory()
    host_bits = host.view(torch.int16).numpy().view(np.uint16)
    hs = np.full((B, n), -1, np.int32)
    st = np.full((B, S), -1, np.int32)
    ss = np.full((B, S), -1, np.int32)
    hk = np.zeros((B, S, d), np.uint16)
    for b in range(B):
        toks = g.choice(vl[b], size=300, replace=False)
        for s_, t in enumerate(toks):
            hs[b, t], st[b, s_], ss[b, s_] = s_, t, int(g.integers(0, 5))
            hk[b, s_] = host_bits[b, t]
    dev = "cuda"
    hot_slot = torch.from_numpy(hs).to(dev)
    slot_token = torch.from_numpy(st).to(dev)
    slot_stamp = torch.from_numpy(ss).to(dev)
    hot_kv = torch.from_numpy(hk.view(np.int16)).to(dev).view(torch.bfloat16)
    q = torch.from_numpy(g.normal(size=(B, Hq, d)).astype(np.float32) * 0.1).to(torch.bfloat16).to(dev)
    seq = torch.from_numpy(vl.astype(np.int32)).to(dev)
    aa = isa.attn_args(q, None, n=n, d_v=512, sm_scale=d ** -0.5, seq_lens=seq,
                       hot_slot=hot_slot, hot_kv=hot_kv, host_kv=host)
    ws = isa.workspace(isa.sparse_workspace_size(None, aa, kb * unit))
    out = torch.empty((B, Hq, 512), dtype=torch.float32, device=dev)
    nblk = (n + unit - 1) // unit
    sel = np.full((B, kb), -1, np.int32)
    for b in range(B):
        sel[b, :10] = np.sort(g.choice(nblk, size=10, replace=False))
    sel_t = torch.from_numpy(sel).to(dev)
    isa.sparse_gather_attn_decode(aa, sel_t, 1, kb, unit, out, None, ws)
    isa.sparse_hot_update(None, aa, sel_t, kb, unit, S, 9, slot_token, slot_stamp, ws)
    torch.cuda.synchronize()
    toks = np.full((B, kb * unit), -1, np.int64)
    for b in range(B):
        for j in range(kb * unit):
            u = sel[b, j // unit]
            toks[b, j] = -1 if u < 0 else u * unit + j % unit
    ref = _oracle_all(hs, st, ss, hk, host_bits, toks, vl, 9)
    _check((hot_slot, slot_token, slot_stamp, hot_kv), ref, "block units")


def test_hot_update_after_fused_step():
    w = synth.get("hot_small")
    print(f"[hot-update] fused step on {w.name}", flush=True)
    inp = synth.make_inputs(w, "cuda")
    # start from the buffer the data generator builds for the workload's own
    # selection (index scores and top-k through the library), then let the
    # update evolve it over two steps
    ia = isa.lightning_index_args(inp["q_idx"], inp["head_w"], inp["k8"], inp["k_scale"],
                                  inp.get("seq_lens"))
    scores = torch.empty((w.B, w.n), dtype=torch.float32, device="cuda")
    ws0 = isa.workspace(max(isa.sparse_workspace_size(ia, None, w.k),
                            isa.sparse_topk_workspace_size(w.B, w.n, w.k)))
    isa.sparse_index_score(ia, scores, ws0)
    sel0 = torch.empty((w.B, w.k), dtype=torch.int32, device="cuda")
    isa.sparse_topk(scores, w.k, sel0, None, inp.get("seq_lens"), 1, ws0)
    torch.cuda.synchronize()
    hot = build_hot_buffer(inp, sel0, "cuda")
    r = StepRunner(inp, hot=hot)
    S = w.hot
    hs = hot["hot_slot"]
    slot_token = torch.full((w.B, S), -1, dtype=torch.int32, device="cuda")
    stt = slot_token.cpu().numpy()
    hsn = hs.cpu().numpy()
    for b in range(w.B):
        for t in np.nonzero(hsn[b] >= 0)[0]:
            stt[b, hsn[b, t]] = t
    slot_token.copy_(torch.from_numpy(stt))
    slot_stamp = torch.zeros((w.B, S), dtype=torch.int32, device="cuda")
    host_bits = hot["host_kv"].view(torch.int16).numpy().view(np.uint16)
    vl = np.array([w.valid(b) for b in range(w.B)])
    aa = r.layer_args[0][0]
    for step in (1, 2):
        state = (hs.cpu().numpy(), slot_token.cpu().numpy(), slot_stamp.cpu().numpy(),
                 _bits(hot["hot_kv"]))
        r.run()
        isa.sparse_hot_update(r.ia, aa, r.topk, w.k, 1, S, step, slot_token, slot_stamp, r.ws)
        torch.cuda.synchronize()
        sel = r.topk[:, 0].cpu().numpy()
        ref = _oracle_all(*state, host_bits, sel, vl, step)
        _check((hs, slot_token, slot_stamp, hot["hot_kv"]), ref, f"fused step {step}")
        # every selected token is resident after the update (the buffer holds more)
        for b in range(w.B):
            s = sel[b][(sel[b] >= 0) & (sel[b] < vl[b])]
            assert (ref[0][b, s] >= 0).all()


PF_CASES = [
    # (B, n, slots, k, candidates, steps, valid lengths)
    (3, 3000, 1024, 512, 300, 3, [3000, 2500, 700]),
    (2, 2000, 160, 100, 120, 3, [2000, 90]),  # more candidates than free slots
    # the measured sizes: 4096 slots, k = 2048 and 2048 candidates
    (2, 16384, 4096, 2048, 2048, 2, [16384, 9000]),
]


@pytest.mark.parametrize("B,n,S,k,m,steps,valid", PF_CASES,
                         ids=[f"S{c[2]}-m{c[4]}" for c in PF_CASES])
def test_hot_prefetch_matches_oracle(B, n, S, k, m, steps, valid):
    print(f"[hot-prefetch] B={B} n={n} slots={S} k={k} m={m} steps={steps}", flush=True)
    g = np.random.default_rng(S + m + n)
    Hq, d = 64, 576
    vl = np.array(valid)
    host = torch.from_numpy(g.normal(size=(B, n, d)).astype(np.float32)).to(torch.bfloat16).pin_memory()
    host_bits = host.view(torch.int16).numpy().view(np.uint16)
    hs = np.full((B, n), -1, np.int32)
    st = np.full((B, S), -1, np.int32)
    ss = np.full((B, S), -1, np.int32)
    hk = np.zeros((B, S, d), np.uint16)
    for b in range(B):
        cnt = int(g.integers(0, min(S, vl[b]) + 1))
        toks = g.choice(vl[b], size=cnt, replace=False)
        slots = g.choice(S, size=cnt, replace=False)
        for t, s_ in zip(toks, slots):
            hs[b, t], st[b, s_], ss[b, s_] = s_, t, int(g.integers(-1, 6))
            hk[b, s_] = host_bits[b, t]
    dev = "cuda"
    hot_slot = torch.from_numpy(hs).to(dev)
    slot_token = torch.from_numpy(st).to(dev)
    slot_stamp = torch.from_numpy(ss).to(dev)
    hot_kv = torch.from_numpy(hk.view(np.int16)).to(dev).view(torch.bfloat16)
    q = torch.from_numpy(g.normal(size=(B, Hq, d)).astype(np.float32) * 0.1).to(torch.bfloat16).to(dev)
    seq = torch.from_numpy(vl.astype(np.int32)).to(dev)
    aa = isa.attn_args(q, None, n=n, d_v=512, sm_scale=d ** -0.5, seq_lens=seq,
                       hot_slot=hot_slot, hot_kv=hot_kv, host_kv=host)
    ws = isa.workspace(isa.sparse_workspace_size(None, aa, k))
    out = torch.empty((B, Hq, 512), dtype=torch.float32, device=dev)
    state = [hs, st, ss, hk]
    for i in range(steps):
        step = 20 + i
        sel = np.full((B, k), -1, np.int32)
        cand = np.full((B, m), -1, np.int32)
        for b in range(B):
            pick = np.sort(g.choice(n, size=int(g.integers(k // 2, k + 1)), replace=False))
            sel[b, : pick.size] = pick
            # candidates: some of the selection, some held tokens, new tokens
            # (some past the valid length), in a random order, with padding
            held = np.nonzero(state[0][b] >= 0)[0]
            pool = np.unique(np.concatenate([
                g.choice(pick, size=min(pick.size, m // 4), replace=False),
                g.choice(held, size=min(held.size, m // 4), replace=False) if held.size else
                np.array([], dtype=np.int64),
                g.choice(n, size=m, replace=False)]))
            c = g.permutation(pool)[: int(g.integers(m // 2, m + 1))]
            cand[b, : c.size] = c
            cand[b][g.random(m) < 0.05] = -1
        sel_t = torch.from_numpy(sel).to(dev)
        cand_t = torch.from_numpy(cand).to(dev)
        isa.sparse_gather_attn_decode(aa, sel_t, 1, k, 1, out, None, ws)
        isa.sparse_hot_update(None, aa, sel_t, k, 1, S, step, slot_token, slot_stamp, ws)
        torch.cuda.synchronize()
        state = _oracle_all(state[0], state[1], state[2], state[3], host_bits, sel, vl, step)
        _check((hot_slot, slot_token, slot_stamp, hot_kv), state, f"update {step}")
        isa.sparse_hot_prefetch(aa, cand_t, m, S, step, slot_token, slot_stamp)
        torch.cuda.synchronize()
        ref = [np.empty_like(x) for x in state]
        for b in range(B):
            r = hot_prefetch(state[0][b], state[1][b], state[2][b], state[3][b], host_bits[b],
                             cand[b], vl[b], step)
            for o, x in zip(ref, r):
                o[b] = x
        _check((hot_slot, slot_token, slot_stamp, hot_kv), ref, f"prefetch {step}")
        state = ref
