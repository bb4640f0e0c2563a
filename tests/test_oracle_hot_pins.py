"""Pins of the hot-buffer replacement oracle (oracle/hot.py), CPU only.

* a worked example computed by hand from the rule;
* one token selected per step: the resident set equals a textbook LRU cache
  (an ordered dict that moves a hit to the end and evicts its front) over
  the same access sequence;
* on random states and selections: the token -> slot and slot -> token maps
  stay inverse, every selected token is resident afterwards when the buffer
  has room, moved rows are the host rows, and no evicted slot was more
  recently used (stamp, slot index) than a surviving slot that this step did
  not select.
"""
from collections import OrderedDict

import numpy as np

from oracle.hot import hot_update


def _state(S, n, d=3):
    return (np.full(n, -1, np.int64), np.full(S, -1, np.int64), np.full(S, -1, np.int64),
            np.zeros((S, d), np.int64))


def _host(n, d=3):
    return np.arange(n * d, dtype=np.int64).reshape(n, d) + 1000


def test_worked_example():
    n, S = 32, 4
    hs, st, ss, hk = _state(S, n)
    host = _host(n)
    for s, (t, stamp) in enumerate([(10, 0), (11, 2), (12, 1)]):
        hs[t], st[s], ss[s], hk[s] = s, t, stamp, host[t]
    # step 3 selects 11 and 12 (held in slots 1, 2) and misses 20, 21; the
    # slots not used this step are 0 (stamp 0) and 3 (empty, stamp -1), so
    # both are taken and, in slot order, 20 -> 0 (evicting 10) and 21 -> 3
    hs2, st2, ss2, hk2 = hot_update(hs, st, ss, hk, host, [11, 20, -1, 21, 12], n, 3)
    assert st2.tolist() == [20, 11, 12, 21]
    assert ss2.tolist() == [3, 3, 3, 3]
    assert hs2[10] == -1 and hs2[20] == 0 and hs2[21] == 3 and hs2[11] == 1 and hs2[12] == 2
    assert (hk2[0] == host[20]).all() and (hk2[3] == host[21]).all()
    assert (hk2[1] == host[11]).all()


def test_worked_example_full_buffer():
    # three misses, two slots free of this step: the least recently used two
    # (stamps 0 and 1 at slots 2 and 0) take the first two misses in slot order
    n, S = 16, 3
    hs, st, ss, hk = _state(S, n)
    host = _host(n)
    for s, (t, stamp) in enumerate([(1, 1), (2, 5), (3, 0)]):
        hs[t], st[s], ss[s], hk[s] = s, t, stamp, host[t]
    hs2, st2, ss2, _ = hot_update(hs, st, ss, hk, host, [2, 7, 8, 9], n, 6)
    assert st2.tolist() == [7, 2, 8]
    assert ss2.tolist() == [6, 6, 6]
    assert hs2[9] == -1 and hs2[1] == -1 and hs2[3] == -1


def test_one_token_per_step_is_lru():
    g = np.random.default_rng(5)
    n, S = 40, 7
    hs, st, ss, hk = _state(S, n)
    host = _host(n)
    lru = OrderedDict()
    for step in range(400):
        t = int(g.integers(0, n)) if g.random() < 0.5 else int(g.integers(0, 10))
        hs, st, ss, hk = hot_update(hs, st, ss, hk, host, [t], n, step)
        if t in lru:
            lru.move_to_end(t)
        else:
            if len(lru) == S:
                lru.popitem(last=False)
            lru[t] = True
        assert set(int(x) for x in st if x >= 0) == set(lru.keys()), step


def test_random_invariants():
    g = np.random.default_rng(11)
    for case in range(300):
        n = int(g.integers(8, 200))
        S = int(g.integers(1, 40))
        valid = int(g.integers(1, n + 1))
        hs, st, ss, hk = _state(S, n)
        host = _host(n)
        # a random resident set with random past stamps
        res = g.choice(n, size=int(g.integers(0, min(S, n) + 1)), replace=False)
        slots = g.choice(S, size=res.shape[0], replace=False)
        step = int(g.integers(1, 50))
        for t, s in zip(res, slots):
            hs[t], st[s], ss[s], hk[s] = s, t, int(g.integers(-1, step)), host[t]
        k = int(g.integers(1, 30))
        sel = np.sort(g.choice(n, size=min(k, n), replace=False))
        sel[g.random(sel.shape[0]) < 0.1] = -1
        hs2, st2, ss2, hk2 = hot_update(hs, st, ss, hk, host, sel, valid, step)
        # inverse maps
        for s in range(S):
            if st2[s] >= 0:
                assert hs2[st2[s]] == s
        for t in range(n):
            if hs2[t] >= 0:
                assert st2[hs2[t]] == t
        chosen = [int(t) for t in sel if 0 <= t < valid]
        # rows of resident tokens are their host rows
        for s in range(S):
            if st2[s] >= 0:
                assert (hk2[s] == host[st2[s]]).all()
        if len(chosen) <= S:
            assert all(hs2[t] >= 0 for t in chosen)
            assert all(ss2[hs2[t]] == step for t in chosen)
        # LRU: every replaced slot was not newer than any untouched survivor
        replaced = [s for s in range(S) if st2[s] != st[s]]
        untouched = [s for s in range(S) if st2[s] == st[s] and ss2[s] < step]
        for r in replaced:
            for u in untouched:
                assert (ss[r], r) < (ss[u], u)
