"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks an oracle function against a closed form, a brute-force
enumeration on tiny inputs, an invariant of the mathematics, an independent
library routine, or a hand-derived fixture under tests/golden/.  They run on
the CPU (no GPU marker).
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import oracle as O
from oracle import step as S
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------- decoding
def test_e4m3fn_spec_values():
    # OCP 8-bit floating point spec (E4M3): bias 7, max 448, no inf,
    # S.1111.111 = NaN, subnormals m/8 * 2^-6.
    t = O.E4M3FN_TABLE
    assert t[0x7E] == 448.0
    assert t[0xFE] == -448.0
    assert t[0x38] == 1.0            # e=7, m=0
    assert t[0x08] == 2.0 ** -6      # smallest normal
    assert t[0x07] == 7 * 2.0 ** -9  # largest subnormal
    assert t[0x01] == 2.0 ** -9      # smallest subnormal
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)  # strictly increasing magnitudes


def test_e4m3fn_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.decode_e4m3fn(codes.numpy())
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.all(both_nan | (ref == mine))


def test_bf16_decode_matches_torch():
    x = torch.randn(10000) * torch.exp(torch.randn(10000) * 5)
    xb = x.to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.decode_bf16(bits), xb.to(torch.float64).numpy())


# ---------------------------------------------------------------- top-k
def _brute_topk(s, k, valid):
    items = sorted(range(valid), key=lambda i: (-s[i], i))[:k]
    out = sorted(items) + [-1] * (k - min(k, valid))
    return np.array(out)


@pytest.mark.parametrize("trial", range(40))
def test_topk_brute_force_with_ties(trial):
    rng = np.random.default_rng(trial)
    n = int(rng.integers(1, 40))
    k = int(rng.integers(1, 45))
    valid = int(rng.integers(0, n + 1))
    s = rng.integers(-3, 4, size=n).astype(np.float64)  # many exact ties
    got = O.topk(s, k, valid)
    assert np.array_equal(got, _brute_topk(s, k, valid))


def test_topk_all_equal_takes_first_k():
    s = np.full(100, 2.5)
    assert np.array_equal(O.topk(s, 7), np.arange(7))


def test_topk_ignores_invalid_tail_and_pads():
    s = np.array([0.0, 5.0, 1.0, 9.0, 9.0])
    assert np.array_equal(O.topk(s, 4, valid=3), [0, 1, 2, -1])


# ---------------------------------------------------------------- attention
def _dense_textbook(q, K, V, scale):
    logits = scale * np.einsum("hd,md->hm", q, K)
    w = scipy.special.softmax(logits, axis=1)
    return w @ V, scipy.special.logsumexp(logits, axis=1)


def test_attention_equals_dense_when_all_selected():
    q = RNG.standard_normal((5, 16))
    K = RNG.standard_normal((37, 16))
    V = RNG.standard_normal((37, 9))
    out, lse = O.attention(q, K, V, 0.25)
    ref_out, ref_lse = _dense_textbook(q, K, V, 0.25)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_attention_single_entry_and_equal_logits():
    q = RNG.standard_normal((3, 8))
    K = RNG.standard_normal((1, 8))
    V = RNG.standard_normal((1, 4))
    out, lse = O.attention(q, K, V, 0.5)
    np.testing.assert_array_equal(out, np.repeat(V, 3, axis=0))
    np.testing.assert_allclose(lse, 0.5 * (q @ K[0]), rtol=1e-15)
    # zero query: every logit is 0 -> out = mean of V, lse = log m
    K = RNG.standard_normal((11, 8))
    V = RNG.standard_normal((11, 4))
    out, lse = O.attention(np.zeros((2, 8)), K, V, 0.5)
    np.testing.assert_allclose(out, np.repeat(V.mean(0, keepdims=True), 2, 0),
                               rtol=1e-13)
    np.testing.assert_allclose(lse, math.log(11), rtol=1e-15)


def test_attention_permutation_invariant_and_empty():
    q = RNG.standard_normal((4, 8))
    K = RNG.standard_normal((20, 8))
    V = RNG.standard_normal((20, 6))
    perm = RNG.permutation(20)
    a = O.attention(q, K, V, 0.3)
    b = O.attention(q, K[perm], V[perm], 0.3)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13)
    out, lse = O.attention(q, K[:0], V[:0], 0.3)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- scores
def test_dot_headsum_brute_force():
    q = RNG.standard_normal((3, 5))
    K = RNG.standard_normal((7, 5))
    ref = [sum(q[h, d] * K[t, d] for h in range(3) for d in range(5))
           for t in range(7)]
    np.testing.assert_allclose(O.score_dot_headsum(q, K), ref, rtol=1e-12)


def test_lightning_reductions():
    q = RNG.standard_normal((4, 6))
    k8 = O.decode_e4m3fn(RNG.integers(0, 0x7E, size=(9, 6)).astype(np.uint8))
    sc = RNG.uniform(0.5, 2.0, size=9)
    # all weights 1 and every dot non-negative -> plain head-summed dot
    qp, kp = np.abs(q), np.abs(k8)
    np.testing.assert_allclose(O.score_lightning(qp, np.ones(4), kp, sc),
                               O.score_dot_headsum(qp, kp * sc[:, None]),
                               rtol=1e-12)
    # one head -> w * relu(q . sigma k)
    for t in range(9):
        d = float(q[0] @ (sc[t] * k8[t]))
        got = O.score_lightning(q[:1], np.array([0.7]), k8[t:t + 1],
                                sc[t:t + 1])[0]
        assert got == pytest.approx(0.7 * max(0.0, d), rel=1e-12, abs=0)
    # brute force over heads with explicit ReLU
    w = RNG.uniform(0, 1, 4)
    ref = [sum(w[h] * max(0.0, sum(q[h, d] * sc[t] * k8[t, d]
                                   for d in range(6))) for h in range(4))
           for t in range(9)]
    np.testing.assert_allclose(O.score_lightning(q, w, k8, sc), ref,
                               rtol=1e-12, atol=1e-12)


def test_block_max():
    s = RNG.standard_normal(10)
    np.testing.assert_array_equal(O.block_max(s, 1, 10), s)
    got = O.block_max(s, 4, 9)  # blocks [0,4) [4,8) [8,9)
    assert got[0] == s[:4].max() and got[1] == s[4:8].max() \
        and got[2] == s[8]
    assert np.isneginf(O.block_max(s, 4, 4)[1])


# ---------------------------------------------------------------- Fathom
def _fathom_data(n=300, D=7, seed=0):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((n, D), generator=g) * torch.linspace(0.1, 5, D)
    codes, zero, cell = synth.quantize_4bit(k)
    return (k.double().numpy(), codes.numpy(), zero.double().numpy(),
            cell.double().numpy())


def test_prefix_of_planes_is_the_tbit_quantizer():
    # Fathom abstract: reading the first t planes of a channel gives that
    # channel's t-bit quantizer, exactly
    x, codes, zero, cell = _fathom_data()
    for t in range(5):
        q_t = O.fathom_tbit_quantize(x, zero[None], cell[None], t)
        assert np.array_equal(codes.astype(np.int64) >> (4 - t), q_t), t


def test_every_code_prefix_identity():
    # exhaustive over codes: (c >> (4-t)) is the t-bit cell of any value in
    # the 4-bit cell c, for every code and depth
    for c in range(16):
        for t in range(5):
            for frac in (0.0, 0.5, 0.999):
                u = (c + frac) / 16.0  # position in [0, 1)
                assert math.floor(u * 2 ** t) == c >> (4 - t)


def test_reconstruction_is_cell_midpoint_and_within_half_cell():
    x, codes, zero, cell = _fathom_data(seed=3)
    for t in range(5):
        depth = np.full(codes.shape[1], t)
        xh = O.fathom_reconstruct(codes, zero, cell, depth)
        cell_t = cell * 2.0 ** (4 - t)
        q_t = O.fathom_tbit_quantize(x, zero[None], cell[None], t)
        np.testing.assert_allclose(xh, zero + cell_t * (q_t + 0.5),
                                   rtol=1e-14, atol=1e-14)
        # the stored fp32 cell can make 16 * cell fall short of (max - min)
        # by one fp32 rounding, so the top value may sit that far outside
        assert np.all(np.abs(x - xh) <= cell_t / 2 * (1 + 1e-5))


def test_planes_layout_matches_codes():
    w = synth.get("fathom_small").with_(n=100, B=1, hkv=2, hq=8,
                                        seq_lens=None)
    inp = synth.make_inputs(w)
    codes = inp["codes"].numpy()
    planes = inp["planes"].numpy().view(np.uint32)
    B, H, n, D = codes.shape
    for h in range(H):
        for c in range(0, D, 17):
            for j in range(4):
                for t in range(n):
                    bit = (int(planes[0, h, c, j, t // 32]) >> (t % 32)) & 1
                    assert bit == (int(codes[0, h, t, c]) >> (3 - j)) & 1
        # words past n are zero
        assert int(planes[0, h, 0, 0, -1]) >> (n % 32) == 0


def _read_golden_waterfill():
    cases = []
    with open(os.path.join(GOLDEN, "waterfill_hand.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            a, b, c = line.split(";")
            cases.append((np.array(a.split(), float), int(b),
                          np.array(c.split(), int)))
    return cases


@pytest.mark.parametrize("case", _read_golden_waterfill())
def test_waterfill_hand_examples(case):
    imp, budget, expect = case
    # imp = q_bar^2 * var with var = 1 and q_bar = sqrt(imp)
    t = O.fathom_read_depth(np.sqrt(imp), np.ones_like(imp), budget)
    assert np.array_equal(t, expect)


def _objective(imp, t):
    return float(np.sum(imp * 4.0 ** (-np.asarray(t, float))))


@pytest.mark.parametrize("trial", range(30))
def test_waterfill_brute_force_optimal(trial):
    rng = np.random.default_rng(100 + trial)
    D = int(rng.integers(1, 7))
    qb = rng.standard_normal(D)
    var = np.exp(rng.standard_normal(D))
    budget = int(rng.integers(0, 4 * D + 1))
    t = O.fathom_read_depth(qb, var, budget)
    imp = (qb * qb) * var
    assert t.sum() == budget and t.min() >= 0 and t.max() <= 4
    best = min(_objective(imp, a) for a in np.ndindex(*(5,) * D)
               if sum(a) == budget)
    assert _objective(imp, t) <= best * (1 + 1e-12) + 1e-300
    # monotone: more important channels never get fewer planes
    for c in range(D):
        for d in range(D):
            if imp[c] > imp[d]:
                assert t[c] >= t[d]


def test_waterfill_equal_importance_and_budget_92():
    t = O.fathom_read_depth(np.ones(128), np.ones(128), 92)
    assert np.array_equal(t, [1] * 92 + [0] * 36)
    t = O.fathom_read_depth(np.ones(10), np.ones(10), 23)
    assert np.array_equal(t, [3, 3, 3, 2, 2, 2, 2, 2, 2, 2])
    rng = np.random.default_rng(7)
    t = O.fathom_read_depth(rng.standard_normal(128),
                            np.exp(rng.standard_normal(128)), 92)
    assert t.sum() == 92


def test_fathom_full_depth_is_dequantised_dot_and_bits_agree():
    x, codes, zero, cell = _fathom_data(n=50, D=6, seed=5)
    qb = RNG.standard_normal(6)
    s = O.score_fathom(qb, codes, zero, cell, np.full(6, 4))
    # brute force from the bits of each code, full depth = 4-bit dequant
    ref = []
    for t in range(50):
        acc = 0.0
        for c in range(6):
            val = sum(((int(codes[t, c]) >> (3 - j)) & 1) * 2 ** (3 - j)
                      for j in range(4))
            acc += qb[c] * (zero[c] + cell[c] * (val + 0.5))
        ref.append(acc)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12)
    # partial depth from bits: sum_{j<t} b_j 2^(3-j) + 2^(3-t)
    depth = np.array([0, 1, 2, 3, 4, 2])
    s = O.score_fathom(qb, codes, zero, cell, depth)
    ref = []
    for t in range(50):
        acc = 0.0
        for c in range(6):
            val = sum(((int(codes[t, c]) >> (3 - j)) & 1) * 2 ** (3 - j)
                      for j in range(depth[c]))
            acc += qb[c] * (zero[c] + cell[c] * (val + 2.0 ** (3 - depth[c])))
        ref.append(acc)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12)
    # zero budget -> every score is the same constant -> first k selected
    s0 = O.score_fathom(qb, codes, zero, cell, np.zeros(6, int))
    assert np.all(s0 == s0[0])
    assert np.array_equal(O.topk(s0, 5), np.arange(5))


def test_fathom_full_budget_matches_exact_topk_of_dequantised_scores():
    # Fathom abstract: a per-token scan agrees with exact top-k decoding; at
    # full depth the plane scan is the 4-bit dequantised dot
    x, codes, zero, cell = _fathom_data(n=400, D=8, seed=9)
    qb = RNG.standard_normal(8)
    t = O.fathom_read_depth(qb, np.ones(8), 32)
    assert np.all(t == 4)
    deq = zero[None] + cell[None] * (codes + 0.5)
    assert np.array_equal(O.topk(O.score_fathom(qb, codes, zero, cell, t), 20),
                          O.topk(deq @ qb, 20))


def test_group_query_left_to_right():
    q = np.array([[1e16, 1.0], [1.0, 2.0], [-1e16, 3.0]])
    # ((1e16 + 1) + -1e16) = 0 in float64 (1 is lost), not 1
    assert O.fathom_group_query(q)[0] == 0.0
    assert O.fathom_group_query(q)[1] == 6.0


# ---------------------------------------------------------------- steps
def _arrays(inp):
    out = {}
    for k, v in inp.items():
        if isinstance(v, torch.Tensor):
            out[k] = synth.host_view(v)
        elif k == "layers":
            out[k] = [{kk: synth.host_view(vv) for kk, vv in L.items()}
                      for L in v]
    return out


def _params(w):
    return {"n": w.n, "k": w.k, "hq": w.hq, "hkv": w.hkv, "dtype": w.dtype,
            "seq_lens": w.seq_lens, "page": w.page, "block": w.block,
            "budget": w.budget, "d_qk": w.d_qk, "d_v": w.d_v}


def test_dot_step_select_all_is_dense_attention():
    w = synth.get("tiny_fp32_small").with_(n=300, k=300, seq_lens=None, B=1)
    arr = _arrays(synth.make_inputs(w))
    r = S.dot_step(arr, _params(w))
    q = arr["q"][0].astype(np.float64)
    K = arr["k_cache"][0, :, 0].astype(np.float64)
    V = arr["v_cache"][0, :, 0].astype(np.float64)
    ref_out, ref_lse = _dense_textbook(q, K, V, 1 / math.sqrt(128))
    np.testing.assert_allclose(r["out"][0], ref_out, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["lse"][0], ref_lse, rtol=1e-12)
    assert np.array_equal(r["sel"][0, 0], np.arange(300))


def test_block_step_block1_reduces_to_token_scores_and_reuse():
    w = synth.get("block_sparse_small").with_(B=1, n=640, k=4,
                                              seq_lens=(600,))
    arr = _arrays(synth.make_inputs(w))
    p = _params(w)
    r = S.block_step(arr, p)
    # block size 1: block scores are the token scores
    p1 = dict(p, block=1, k=40)
    r1 = S.block_step(arr, p1)
    q = O.decode_bf16(arr["q_idx"][0])
    keys = O.decode_bf16(arr["k_idx"][0, :600])
    np.testing.assert_allclose(r1["scores"][0, 0, :600],
                               O.score_dot_headsum(q, keys), rtol=1e-12)
    # reuse: later layers given layer 0's selection give the same outputs
    r2 = S.block_step(arr, p, sel_in=r["sel"])
    for a, b in zip(r["layers"], r2["layers"]):
        np.testing.assert_array_equal(a["out"], b["out"])
    # the last partial block (tokens 576..599) is scored over valid tokens
    assert np.isfinite(r["scores"][0, 0, 9]) and r["scores"].shape[2] == 10
