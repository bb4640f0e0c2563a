"""Parity comparators between a GPU result and the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/oracle.py).

Let s_k be the oracle's k-th largest valid score of a row and
tau = 1e-3 * (|s_k| + 1).  The band is {i : |s_i - s_k| <= tau}.
* Selection: the GPU set and the oracle set have the same size and agree
  outside the band (swaps among near-ties are allowed, nothing else).
* Scores: |s_gpu - s_oracle| <= tau for every valid unit.
* Attention: max-abs difference <= 2e-3.
"""
from __future__ import annotations

import numpy as np

ATTN_TOL = 2e-3


def kth_tau(oracle_scores: np.ndarray, k: int, valid: int):
    s = oracle_scores[:valid]
    if valid == 0:
        return -np.inf, 0.0
    kk = min(k, valid)
    sk = np.sort(s)[::-1][kk - 1]
    return sk, 1e-3 * (abs(sk) + 1.0)


def selection_ok(gpu_sel: np.ndarray, oracle_sel: np.ndarray,
                 oracle_scores: np.ndarray, k: int, valid: int) -> tuple[bool, str]:
    """Band rule on one row.  gpu_sel / oracle_sel: [k] (-1 padded)."""
    g = gpu_sel[gpu_sel >= 0]
    o = oracle_sel[oracle_sel >= 0]
    if g.shape[0] != o.shape[0]:
        return False, f"count {g.shape[0]} != {o.shape[0]}"
    if np.unique(g).shape[0] != g.shape[0]:
        return False, "duplicate indices"
    if g.shape[0] and (g.min() < 0 or g.max() >= valid):
        return False, "index out of range"
    if np.any(np.diff(g) <= 0):
        return False, "not ascending"
    if g.shape[0] == 0:
        return True, ""
    sk, tau = kth_tau(oracle_scores, k, valid)
    band = np.abs(oracle_scores - sk) <= tau
    gs, os_ = set(g.tolist()), set(o.tolist())
    diff = gs.symmetric_difference(os_)
    bad = [i for i in diff if not band[i]]
    if bad:
        return False, f"{len(bad)} swaps outside the band, e.g. {bad[:5]}"
    return True, ""


def scores_ok(gpu_scores: np.ndarray, oracle_scores: np.ndarray, k: int,
              valid: int) -> tuple[bool, float, float]:
    """Scores within tau on every valid unit; returns (ok, max_err, tau).
    A non-finite GPU score at a valid unit fails (error inf)."""
    _, tau = kth_tau(oracle_scores, k, valid)
    if valid == 0:
        return True, 0.0, tau
    g = np.asarray(gpu_scores[:valid], dtype=np.float64)
    if not np.all(np.isfinite(g)):
        return False, float("inf"), tau
    err = np.abs(g - oracle_scores[:valid])
    m = float(err.max())
    return m <= tau, m, tau


def attn_ok(gpu: np.ndarray, ref: np.ndarray, tol: float = ATTN_TOL):
    """Max-abs difference of outputs (or lse values) within tol.

    Non-finite entries must sit at the same positions with the same value on
    both sides (an empty selection gives lse = -inf in the oracle); a NaN on
    either side, or a shape mismatch, fails with error inf.  The maximum is
    then taken over the finite entries."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape or np.isnan(g).any() or np.isnan(r).any():
        return False, float("inf")
    gf, rf = np.isfinite(g), np.isfinite(r)
    if not np.array_equal(gf, rf) or not np.array_equal(g[~gf], r[~rf]):
        return False, float("inf")
    if not gf.any():
        return True, 0.0
    m = float(np.abs(g[gf] - r[rf]).max())
    return m <= tol, m
