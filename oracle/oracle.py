"""Plain, slow CPU oracle for one decode step of indexer-driven sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` use it.  It shares no code with the HIP library or its Python
binding; the two meet only through the seeded inputs of ``synth``.

Every function works in float64 on plain numpy arrays and writes out the
definition of what it computes, with no blocking, fusion or reordering beyond
what that definition states.  Sources, cited by page title and passage:

* [XM]  "XM-Sparse: Pushing the Throughput Frontier of Sparse Attention with
  Netpreme X-Mem" -- opening paragraph (sparse attention reads only the
  selected KV entries; the indexer key cache sits in HBM), the modelling
  paragraphs (2,048 selected entries per layer per step, a 4,096-token hot KV
  buffer) and the KV-lifecycle list (fetch only the missing selected entries).
* [MM]  "MiniMax-M3: share the sparse index top-k across layers and reuse the
  decode top-k buffer" -- description (a lightning-indexer pass picks the
  top-k KV *blocks*; the first layer of a group stores the reduced top-k in a
  persistent int32 buffer, the rest reuse it) and its Correctness note.
* [FA]  "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
  Caches" -- abstract (4-bit K stored channel-major as bit planes, a prefix of
  t planes is the channel's t-bit quantizer, the bit budget is spent by
  reverse water-filling over variance-weighted channel importance).

Readings of points the pages leave open are listed in the module docstrings
of each function ("reading:").  Parity status: every function here is pinned
by the ``-m "not gpu"`` tests (closed forms, brute force, invariants, the OCP
FP8 table); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Input decoding (exact, to float64)
# ----------------------------------------------------------------------------


def _build_e4m3fn_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3 ("e4m3fn") byte, from the format definition.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field
    0 is subnormal (m/8 * 2^-6).  There are no infinities; S.1111.111 is NaN,
    so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            table[code] = np.nan
        elif exp == 0:
            table[code] = sign * (man / 8.0) * 2.0 ** (1 - 7)
        else:
            table[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return table


E4M3FN_TABLE = _build_e4m3fn_table()


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """uint8 OCP E4M3FN bytes -> float64 (table lookup, exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return E4M3FN_TABLE[codes]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (bit-widening, exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Index scores (step a2)
# ----------------------------------------------------------------------------


def score_dot_headsum(q: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """s_t = sum_h q_h . k_t  (head-summed dot product of every cached key).

    q: [H][D] float64, keys: [n][D] float64 -> [n].
    reading: one shared index key per token, summed over the index heads with
    no weights and no ReLU ([MM] description names only the pass; the tiny
    fp32 workload and the block-sparse workload both use this form).
    """
    dots = keys @ q.T  # [n][H]
    return dots.sum(axis=1)


def score_lightning(q: np.ndarray, w: np.ndarray, k8_vals: np.ndarray,
                    k_scale: np.ndarray) -> np.ndarray:
    """Lightning-indexer score over an fp8 K-index with a per-token scale.

    s_t = sum_h w_h * max(0, q_h . (sigma_t * k8_t)).
    q: [H][D], w: [H], k8_vals: [n][D] decoded e4m3 values, k_scale: [n].
    reading: the key is dequantised (sigma_t * k8_t) before the ReLU; this is
    the indexer pass the [XM] opening paragraph keeps in HBM and the [MM]
    description runs once per sparse layer.
    """
    keys = k8_vals * k_scale[:, None]
    dots = keys @ q.T  # [n][H]
    return np.maximum(dots, 0.0) @ w


def block_max(scores: np.ndarray, block: int, valid: int) -> np.ndarray:
    """Block score = max over the block's valid tokens ([MM]: KV *blocks*).

    scores: [n] token scores; tokens >= valid are excluded.  A block with no
    valid token scores -inf.  Returns [ceil(n / block)].
    """
    n = scores.shape[0]
    nb = (n + block - 1) // block
    out = np.full(nb, -np.inf)
    for b in range(nb):
        lo, hi = b * block, min((b + 1) * block, valid)
        if hi > lo:
            out[b] = scores[lo:hi].max()
    return out


# ----------------------------------------------------------------------------
# Fathom: read-depth allocation (step a1) and plane-prefix score (step a2)
# ----------------------------------------------------------------------------


def fathom_group_query(q_group: np.ndarray) -> np.ndarray:
    """q_bar_c = ((q_0 + q_1) + q_2) + ... for the query heads of one KV head.

    q_group: [G][D] float64.  The adds run left to right in explicit scalar
    order so that the float64 result is reproducible bit for bit.
    reading: the ranked score of a grouped-query KV head is sum_h q_h . k =
    q_bar . k, so allocation and scan use q_bar.
    """
    acc = q_group[0].copy()
    for g in range(1, q_group.shape[0]):
        acc = acc + q_group[g]
    return acc


def fathom_read_depth(q_bar: np.ndarray, var: np.ndarray, budget: int,
                      planes: int = 4) -> np.ndarray:
    """Per-channel read depth t_c in {0..planes} with sum_c t_c = budget.

    [FA] abstract: each query divides its per-key bit budget among the
    channels by reverse water-filling, with a channel's importance weighted
    by its variance.  Written out:
      importance  imp_c = (q_bar_c * q_bar_c) * var_c
      the distortion of channel c read to depth t is modelled as
      imp_c * 4^-t, so reading plane j of channel c lowers it by
      gain g_{c,j} = imp_c * 4^-(j+1) * 3, which is proportional to
      imp_c * 4^-j; the constant factor does not change the order, so the
      gains are taken as imp_c * 4^-j.
      Rank all gains by (gain descending, channel ascending, plane ascending)
      and take the first `budget`; t_c is how many were taken from channel c.
    Each channel's gains fall strictly with j when imp_c > 0 (and tie on
    equal c otherwise, broken by j), so the taken set is a prefix of every
    channel's planes.  Greedy is the exact minimiser of sum_c imp_c 4^-t_c
    under sum t_c = budget because the objective is separable and convex in
    t_c; it is the integer form of R_c = max(0, 1/2 log2(imp_c / theta)).
    """
    D = q_bar.shape[0]
    if not 0 <= budget <= planes * D:
        raise ValueError("budget out of range")
    imp = (q_bar * q_bar) * var
    gains, chans, plns = [], [], []
    for c in range(D):
        for j in range(planes):
            gains.append(imp[c] * (4.0 ** -j))
            chans.append(c)
            plns.append(j)
    gains = np.array(gains)
    chans = np.array(chans)
    plns = np.array(plns)
    # lexsort: last key is primary
    order = np.lexsort((plns, chans, -gains))
    t = np.zeros(D, dtype=np.int64)
    for idx in order[:budget]:
        t[chans[idx]] += 1
    return t


def fathom_reconstruct(codes: np.ndarray, zero: np.ndarray, cell: np.ndarray,
                       depth: np.ndarray) -> np.ndarray:
    """Cell-midpoint value of the t_c-bit prefix of each 4-bit code.

    codes: [n][D] ints 0..15, zero/cell: [D] (4-bit cell width), depth: [D].
    A t-bit prefix p = code >> (4 - t) names a cell of width cell * 2^(4-t)
    starting at zero + p * cell * 2^(4-t); its midpoint is
      x_hat = zero + cell * (p * 2^(4-t) + 2^(3-t)).
    t = 0 gives the constant zero + 8 * cell (the middle of the range).
    reading: [FA] says a t-plane prefix *is* the channel's t-bit quantizer;
    reconstructing at the middle of that quantizer's cell is the plainest
    estimate of the key it stands for.
    """
    codes = np.asarray(codes, dtype=np.int64)
    depth = np.asarray(depth, dtype=np.int64)
    shift = 4 - depth  # [D]
    prefix = codes >> shift[None, :]
    step = np.power(2.0, shift)[None, :]
    mid = np.power(2.0, 3 - depth.astype(np.float64))[None, :]
    return zero[None, :] + cell[None, :] * (prefix * step + mid)


def fathom_tbit_quantize(x: np.ndarray, zero: np.ndarray, cell: np.ndarray,
                         t: int) -> np.ndarray:
    """The channel's own t-bit quantizer: 2^t equal cells over [min, max].

    cell is the 4-bit cell width ((max - min) / 16); the t-bit cell is
    16 * cell / 2^t.  code_t = min(floor((x - zero) / cell_t), 2^t - 1).
    Used by the tests to pin the [FA] prefix identity.
    """
    cell_t = cell * (2.0 ** (4 - t))
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.floor((x - zero) / cell_t)
    u = np.where(cell_t > 0, u, 0.0)
    return np.minimum(u, 2 ** t - 1).astype(np.int64)


def score_fathom(q_bar: np.ndarray, codes: np.ndarray, zero: np.ndarray,
                 cell: np.ndarray, depth: np.ndarray) -> np.ndarray:
    """s_t = q_bar . x_hat_t with x_hat from the t_c-plane prefixes."""
    x_hat = fathom_reconstruct(codes, zero, cell, depth)
    return x_hat @ q_bar


# ----------------------------------------------------------------------------
# Top-k selection (step a3)
# ----------------------------------------------------------------------------


def topk(scores: np.ndarray, k: int, valid: int | None = None) -> np.ndarray:
    """Exact top-k with ties to the lower index; indices returned ascending.

    Units at index >= valid are never selected.  If fewer than k units are
    valid, the tail is padded with -1.  Sorting by (-score, index) is the
    definition; the ascending output order is the reading taken for a
    deterministic result (any order gives the same attention).
    """
    n = scores.shape[0]
    valid = n if valid is None else max(0, min(valid, n))
    s = scores[:valid]
    order = np.lexsort((np.arange(valid), -s))
    take = np.sort(order[: min(k, valid)])
    out = np.full(k, -1, dtype=np.int64)
    out[: take.shape[0]] = take
    return out


# ----------------------------------------------------------------------------
# Sparse attention (step a6)
# ----------------------------------------------------------------------------


def attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
              scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of the query heads over the given rows.

    q: [H][dqk], keys: [m][dqk], values: [m][dv] (all float64).
    logits_i = scale * q . k_i; out = sum_i softmax_i * v_i; lse = natural log
    of sum_i exp(logits_i).  With m = 0 the output is 0 and lse is -inf.
    [XM] opening paragraph: each step attends over only the selected entries.
    """
    H = q.shape[0]
    dv = values.shape[1]
    if keys.shape[0] == 0:
        return np.zeros((H, dv)), np.full(H, -np.inf)
    logits = scale * (q @ keys.T)  # [H][m]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    denom = p.sum(axis=1, keepdims=True)
    out = (p @ values) / denom
    lse = m[:, 0] + np.log(denom[:, 0])
    return out, lse


def expand_selection(sel: np.ndarray, unit: int, valid: int) -> np.ndarray:
    """Selected units -> token positions (unit 64 = a 64-token block).

    -1 entries are padding and dropped; tokens >= valid are dropped.
    """
    toks = []
    for u in sel:
        if u < 0:
            continue
        for t in range(u * unit, (u + 1) * unit):
            if t < valid:
                toks.append(t)
    return np.array(toks, dtype=np.int64)
