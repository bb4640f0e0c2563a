"""Pins of the oracle's comparators and of its index -> KV address steps.

Each pin checks an oracle function against something that does not come
from the oracle: hand-made cases for the parity comparators, textbook dense
softmax attention over rows picked out of a contiguous copy of the KV, and
per-head brute force for grouped-query routing.  Each group also plants one
plausible mistake in a copy of the oracle function (on the CPU) and checks
that the same pin rejects it, with no tolerance changed:

* the latent page lookup with the page number and the row in the page
  swapped ("XM-Sparse" blog, opening paragraph: attention reads only the
  selected entries, so the address of each selected entry must be right);
* query heads routed to KV head h % Hkv instead of h // (Hq / Hkv) (grouped
  query attention of the Fathom workload, Fathom abstract);
* a selected 64-token block expanded to tokens 64b+1 .. 64b+64 instead of
  64b .. 64b+63 ("MiniMax-M3" PR, description: the top-k KV blocks).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import compare as C
from oracle import oracle as O
from oracle import step as S

RNG = np.random.default_rng(4242)


def _dense_textbook(q, K, V, scale):
    logits = scale * np.einsum("hd,md->hm", q, K)
    w = scipy.special.softmax(logits, axis=1)
    return w @ V, scipy.special.logsumexp(logits, axis=1)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ====================================================== parity comparators
def test_kth_tau_hand_example():
    s = np.array([3.0, -1.0, 7.5, 7.5, 0.25, -np.inf])
    # valid = 5: sorted 7.5 7.5 3 0.25 -1 -> 3rd largest is 3.0
    sk, tau = C.kth_tau(s, 3, 5)
    assert sk == 3.0 and tau == pytest.approx(1e-3 * 4.0, rel=1e-15)
    # k above the valid count: the smallest valid score
    sk, tau = C.kth_tau(s, 9, 5)
    assert sk == -1.0 and tau == pytest.approx(2e-3, rel=1e-15)
    sk, tau = C.kth_tau(s, 3, 0)
    assert sk == -np.inf and tau == 0.0


def test_selection_ok_band_rule():
    # k = 3; the 3rd largest is s_k = 5.004, tau = 1e-3 * 6.004; 5.0 and
    # 4.9985 lie within tau of it, 4.997 does not
    s = np.array([9.0, 5.0, 1.0, 5.004, 4.9985, 8.0, 4.997, 0.0])
    ref = O.topk(s, 3)  # 0, 3, 5
    assert list(ref) == [0, 3, 5]
    ok, _ = C.selection_ok(ref, ref, s, 3, 8)
    assert ok
    # swap 3 (5.004) for 1 (5.0) or 4 (4.9985): both inside the band
    for other in (1, 4):
        g = np.sort(np.array([0, other, 5]))
        ok, why = C.selection_ok(g, ref, s, 3, 8)
        assert ok, why
    # swap for 6 (4.997): outside the band
    ok, why = C.selection_ok(np.array([0, 5, 6]), ref, s, 3, 8)
    assert not ok and "outside the band" in why
    # a top score dropped for a band member fails too
    ok, _ = C.selection_ok(np.array([1, 3, 5]), ref, s, 3, 8)
    assert not ok
    # count, duplicates, order, range
    assert not C.selection_ok(np.array([0, 3, -1]), ref, s, 3, 8)[0]
    assert not C.selection_ok(np.array([0, 3, 3]), ref, s, 3, 8)[0]
    assert not C.selection_ok(np.array([5, 3, 0]), ref, s, 3, 8)[0]
    assert not C.selection_ok(np.array([0, 3, 8]), ref, s, 3, 8)[0]
    # padding on both sides when fewer than k are valid
    r2 = O.topk(s, 4, valid=2)
    assert C.selection_ok(r2, r2, s, 4, 2)[0]


def test_scores_ok_tolerance_edges():
    ref = np.array([2.0, -3.0, 10.0, 0.5])
    k = 2  # s_k = 2.0, tau = 3e-3
    tau = 3e-3
    ok, m, t = C.scores_ok(ref + 0.99 * tau, ref, k, 4)
    assert ok and t == pytest.approx(tau)
    g = ref.copy()
    g[1] += 1.01 * tau
    ok, m, _ = C.scores_ok(g, ref, k, 4)
    assert not ok and m == pytest.approx(1.01 * tau)
    # entries past the valid length are not compared
    g = ref.copy()
    g[3] = 99.0
    assert C.scores_ok(g, ref, k, 3)[0]
    # a NaN or an infinity at a valid unit fails
    for bad in (np.nan, np.inf, -np.inf):
        g = ref.copy()
        g[0] = bad
        assert not C.scores_ok(g, ref, k, 4)[0]


def test_attn_ok_tolerance_and_special_values():
    ref = RNG.standard_normal((3, 16))
    assert C.attn_ok(ref + 1.9e-3, ref)[0]
    g = ref.copy()
    g[2, 5] += 2.1e-3
    ok, m = C.attn_ok(g, ref)
    assert not ok and m == pytest.approx(2.1e-3, rel=1e-9)
    g = ref.copy()
    g[0, 0] = np.nan
    assert C.attn_ok(g, ref) == (False, float("inf"))
    assert not C.attn_ok(ref, g)[0]
    # lse of an empty selection: -inf on both sides passes, on one side fails
    lse = np.array([1.5, -np.inf, 0.25])
    assert C.attn_ok(lse.copy(), lse) == (True, 0.0)
    g = lse.copy()
    g[1] = -80.0
    assert not C.attn_ok(g, lse)[0]
    g = lse.copy()
    g[0] = np.inf
    assert not C.attn_ok(g, lse)[0]
    assert not C.attn_ok(ref[:2], ref)[0]


def test_attn_ok_sees_one_dropped_high_weight_row():
    # latent-shaped rows at k = 2048 with the query scaled so that the logits
    # spread over more than 8 (softmax far from uniform): dropping the row
    # of largest weight must move the output beyond the 2e-3 bar
    m, d_qk, d_v, H = 2048, 576, 512, 8
    rows = RNG.standard_normal((m, d_qk))
    q = RNG.standard_normal((H, d_qk)) * 3.0
    scale = 1.0 / math.sqrt(d_qk)
    out, _ = O.attention(q, rows, rows[:, :d_v], scale)
    logits = scale * q @ rows.T
    assert np.all(logits.max(1) - logits.min(1) > 8.0)
    drop = int(np.argmax(logits[0]))
    keep = np.ones(m, bool)
    keep[drop] = False
    out2, _ = O.attention(q, rows[keep], rows[keep][:, :d_v], scale)
    ok, err = C.attn_ok(out2, out)
    assert not ok and err > 1e-2
    # dropping the row of least weight stays inside the bar
    drop = int(np.argmin(logits.max(0)))
    keep = np.ones(m, bool)
    keep[drop] = False
    out3, _ = O.attention(q, rows[keep], rows[keep][:, :d_v], scale)
    assert C.attn_ok(out3, out)[0]


# ======================================================== latent paging
def _paged_latent(B=2, n=4096, page=64, hq=8, seed=0):
    """A contiguous latent KV [B][n][576] and the same rows scattered into a
    shuffled page pool shared by the requests (pages interleaved)."""
    rng = np.random.default_rng(seed)
    kv = _bf16_bits(rng.standard_normal((B, n, 576)))
    q = _bf16_bits(rng.standard_normal((B, hq, 576)))
    n_pages = n // page
    perm = rng.permutation(B * n_pages)
    pt = perm.reshape(B, n_pages).astype(np.int32)
    pool = np.zeros((B * n_pages, page, 576), dtype=np.uint16)
    for b in range(B):
        for j in range(n_pages):
            pool[pt[b, j]] = kv[b, j * page:(j + 1) * page]
    arr = {"q": q, "kv_pool": pool, "page_table": pt}
    p = {"n": n, "k": 0, "seq_lens": None, "page": page, "d_qk": 576, "d_v": 512}
    return arr, p, kv


def _latent_pins_hold(step_fn) -> bool:
    """True when lightning_step's attention over paged rows equals textbook
    attention over the contiguous copy for: a random subset of tokens, one
    token, and every token (k = n)."""
    arr, p, kv = _paged_latent()
    B, n = kv.shape[0], kv.shape[1]
    scale = 1.0 / math.sqrt(576)
    q = O.decode_bf16(arr["q"])
    rows_all = O.decode_bf16(kv)
    # a random subset of 300 tokens per request
    sel = np.stack([np.sort(RNG.choice(n, 300, replace=False)) for _ in range(B)])[:, None]
    r = step_fn(arr, dict(p, k=300), sel_in=sel)
    for b in range(B):
        ro, rl = _dense_textbook(q[b], rows_all[b, sel[b, 0]], rows_all[b, sel[b, 0], :512],
                                 scale)
        if not (np.allclose(r["out"][b], ro, rtol=1e-10, atol=1e-12)
                and np.allclose(r["lse"][b], rl, rtol=1e-12)):
            return False
    # one selected token: every head's output is exactly that row's first 512
    for t in (5, 64 * 17 + 63, n - 1):
        sel1 = np.full((B, 1, 4), -1, dtype=np.int64)
        sel1[:, 0, 0] = t
        r = step_fn(arr, dict(p, k=4), sel_in=sel1)
        for b in range(B):
            if not np.array_equal(r["out"][b], np.repeat(rows_all[b, t:t + 1, :512], 8, 0)):
                return False
    # every token selected: dense attention over the request's rows
    allsel = np.tile(np.arange(n), (B, 1))[:, None]
    r = step_fn(arr, dict(p, k=n), sel_in=allsel)
    for b in range(B):
        ro, _ = _dense_textbook(q[b], rows_all[b], rows_all[b, :, :512], scale)
        if not np.allclose(r["out"][b], ro, rtol=1e-10, atol=1e-12):
            return False
    return True


def test_latent_rows_paged_address():
    assert _latent_pins_hold(S.lightning_step)


def test_latent_rows_pin_rejects_swapped_page_lookup(monkeypatch):
    def bad_latent_rows(arr, p, b, toks):
        page = p["page"]
        pt = arr["page_table"][b]
        phys = pt[toks % page]            # planted: page and row swapped
        return O.decode_bf16(arr["kv_pool"][phys, toks // page])
    monkeypatch.setattr(S, "latent_rows", bad_latent_rows)
    assert not _latent_pins_hold(S.lightning_step)


def test_latent_rows_pin_rejects_request_ignored(monkeypatch):
    def bad_latent_rows(arr, p, b, toks):
        page = p["page"]
        pt = arr["page_table"][0]         # planted: request 0's page table
        return O.decode_bf16(arr["kv_pool"][pt[toks // page], toks % page])
    monkeypatch.setattr(S, "latent_rows", bad_latent_rows)
    assert not _latent_pins_hold(S.lightning_step)


# ============================================== grouped-query routing
def _fathom_routing_case():
    w = synth.get("fathom_small").with_(B=1, n=200, k=20, hq=4, hkv=2, seq_lens=None,
                                        budget=40)
    inp = synth.make_inputs(w)
    arr = {k: synth.host_view(v) for k, v in inp.items() if isinstance(v, torch.Tensor)}
    # full read depth: the plane-prefix score is the 4-bit dequantised dot
    arr["depth_in"] = np.full((1, 2, 128), 4, dtype=np.int8)
    p = {"n": w.n, "k": w.k, "budget": w.budget, "seq_lens": None}
    return w, arr, p


def _routing_pins_hold(step_fn) -> bool:
    w, arr, p = _fathom_routing_case()
    q = O.decode_bf16(arr["q"][0])  # [4][128]
    K = O.decode_bf16(arr["k_cache"][0])  # [n][2][128]
    V = O.decode_bf16(arr["v_cache"][0])
    G = 2
    # the two KV heads get different selections
    sel = np.stack([np.sort(RNG.choice(w.n, w.k, replace=False)) for _ in range(2)])[None]
    r = step_fn(arr, p, sel_in=sel)
    scale = 1.0 / math.sqrt(128)
    for h in range(4):
        kvh = h // G
        ro, rl = _dense_textbook(q[h:h + 1], K[sel[0, kvh], kvh], V[sel[0, kvh], kvh], scale)
        if not (np.allclose(r["out"][0, h], ro[0], rtol=1e-10, atol=1e-12)
                and np.allclose(r["lse"][0, h], rl[0], rtol=1e-12)):
            return False
    # each KV head's scores use the sum of its own consecutive query heads
    codes = arr["codes"][0].astype(np.float64)  # [2][n][128]
    for j in range(2):
        qbar = q[G * j] + q[G * j + 1]
        deq = arr["chan_zero"][0, j] + arr["chan_scale"][0, j] * (codes[j] + 0.5)
        if not np.allclose(r["scores"][0, j], deq @ qbar, rtol=1e-12, atol=1e-12):
            return False
    # without sel_in the selection is each KV head's own top-k
    r = step_fn(arr, p)
    for j in range(2):
        if not np.array_equal(r["sel"][0, j], O.topk(r["scores"][0, j], w.k)):
            return False
    if np.array_equal(r["sel"][0, 0], r["sel"][0, 1]):
        return False
    return True


def test_gqa_routing_and_own_selection():
    assert _routing_pins_hold(S.fathom_step)


def test_gqa_routing_pin_rejects_modulo_routing(monkeypatch):
    def bad_gqa(q, K_raw, V_raw, toks_per_kv_head, scale):
        Hq, hkv = q.shape[0], K_raw.shape[1]
        out = np.zeros((Hq, V_raw.shape[2]))
        lse = np.zeros(Hq)
        for h in range(Hq):
            kvh = h % hkv                  # planted: modulo routing
            toks = toks_per_kv_head[kvh]
            o, l = O.attention(q[h:h + 1], O.decode_bf16(K_raw[toks, kvh]),
                               O.decode_bf16(V_raw[toks, kvh]), scale)
            out[h], lse[h] = o[0], l[0]
        return out, lse
    monkeypatch.setattr(S, "gqa_attention", bad_gqa)
    assert not _routing_pins_hold(S.fathom_step)


def test_gqa_routing_pin_rejects_wrong_query_group(monkeypatch):
    def first_head_only(q_group):
        return q_group[0].copy()           # planted: q_bar = the group's first head
    monkeypatch.setattr(O, "fathom_group_query", first_head_only)
    assert not _routing_pins_hold(S.fathom_step)


# ================================================== block expansion
def test_expand_selection_blocks_by_hand():
    assert np.array_equal(O.expand_selection(np.array([2]), 64, 1000), np.arange(128, 192))
    assert np.array_equal(O.expand_selection(np.array([0, 2, -1]), 64, 150),
                          np.concatenate([np.arange(64), np.arange(128, 150)]))
    assert O.expand_selection(np.array([3, -1]), 64, 150).shape == (0,)
    assert np.array_equal(O.expand_selection(np.array([4, 7]), 1, 6), [4])


def _block_pins_hold(step_fn, expand) -> bool:
    w = synth.get("block_sparse_small").with_(B=2, n=700, k=11, seq_lens=(700, 650),
                                              layers=1)
    inp = synth.make_inputs(w)
    arr = {k: synth.host_view(v) for k, v in inp.items() if isinstance(v, torch.Tensor)}
    arr["layers"] = [{kk: synth.host_view(vv) for kk, vv in L.items()} for L in inp["layers"]]
    p = {"n": w.n, "k": w.k, "block": 64, "seq_lens": w.seq_lens}
    L0 = arr["layers"][0]
    scale = 1.0 / math.sqrt(128)
    # all 11 blocks selected: dense attention over the valid tokens
    r = step_fn(arr, p)
    for b in range(2):
        valid = w.seq_lens[b]
        if not np.array_equal(r["sel"][b, 0], np.arange(11)):
            return False
        q = O.decode_bf16(L0["q"][b])
        K = O.decode_bf16(L0["k_cache"][b, :valid])
        V = O.decode_bf16(L0["v_cache"][b, :valid])
        for h in range(8):
            hs = slice(8 * h, 8 * h + 8)
            ro, _ = _dense_textbook(q[hs], K[:, h], V[:, h], scale)
            if not np.allclose(r["layers"][0]["out"][b, hs], ro, rtol=1e-10, atol=1e-12):
                return False
    # two chosen blocks, the last one partial (tokens 640..649 of request 1)
    sel = np.array([[[3, 10] + [-1] * 9], [[0, 10] + [-1] * 9]])
    r = step_fn(arr, p, sel_in=sel)
    for b in range(2):
        valid = w.seq_lens[b]
        toks = np.concatenate([np.arange(64 * sel[b, 0, 0], 64 * sel[b, 0, 0] + 64),
                               np.arange(640, valid)])
        if not np.array_equal(expand(sel[b, 0], 64, valid), toks):
            return False
        q = O.decode_bf16(L0["q"][b])
        K = O.decode_bf16(L0["k_cache"][b, toks])
        V = O.decode_bf16(L0["v_cache"][b, toks])
        for h in range(8):
            hs = slice(8 * h, 8 * h + 8)
            ro, _ = _dense_textbook(q[hs], K[:, h], V[:, h], scale)
            if not np.allclose(r["layers"][0]["out"][b, hs], ro, rtol=1e-10, atol=1e-12):
                return False
    return True


def test_block_expansion_and_partial_block():
    assert _block_pins_hold(S.block_step, O.expand_selection)


def test_block_pin_rejects_shifted_expansion(monkeypatch):
    def shifted(sel, unit, valid):
        toks = [t for u in sel if u >= 0
                for t in range(u * unit + 1, (u + 1) * unit + 1) if t < valid]
        return np.array(toks, dtype=np.int64)   # planted: 64b+1 .. 64b+64
    monkeypatch.setattr(O, "expand_selection", shifted)
    assert not _block_pins_hold(S.block_step, O.expand_selection)
