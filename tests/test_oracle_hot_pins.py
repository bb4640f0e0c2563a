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
* the prefetch: a worked example computed by hand from its rule, agreement
  with the update on every state where no candidate is resident (the two
  rules then coincide), and on random states the map invariants, resident
  candidates and this step's slots left alone, and the LRU order of the
  replaced slots.
"""
from collections import OrderedDict

import numpy as np

from oracle.hot import hot_prefetch, hot_update


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


def test_prefetch_worked_example():
    # slots: 0 holds 10 (stamped this step, 3), 1 holds 11 (stamp 1), 2 is
    # empty, 3 holds 12 (stamp 0), 4 holds 13 (stamp 2).  Candidates 11 and
    # 10 are resident (slot 1 is protected, slot 0 is this step's); 40 is
    # past the valid length.  The fills 20, 21, 22, 23 can use slots 2, 3, 4
    # only: in slot order 20 -> 2, 21 -> 3 (evicting 12), 22 -> 4 (evicting
    # 13), and 23 stays out.
    n, S, valid = 48, 5, 32
    hs, st, ss, hk = _state(S, n)
    host = _host(n)
    for s_, (t, stamp) in enumerate([(10, 3), (11, 1), (None, -1), (12, 0), (13, 2)]):
        if t is not None:
            hs[t], st[s_], hk[s_] = s_, t, host[t]
        ss[s_] = stamp
    hs2, st2, ss2, hk2 = hot_prefetch(hs, st, ss, hk, host, [11, 20, 21, 22, 23, -1, 40, 10],
                                      valid, 3)
    assert st2.tolist() == [10, 11, 20, 21, 22]
    assert ss2.tolist() == [3, 1, 3, 3, 3]
    assert hs2[12] == -1 and hs2[13] == -1 and hs2[23] == -1 and hs2[40] == -1
    assert hs2[11] == 1 and hs2[10] == 0
    assert hs2[20] == 2 and hs2[21] == 3 and hs2[22] == 4
    for s_ in (2, 3, 4):
        assert (hk2[s_] == host[st2[s_]]).all()


def _random_state(g, n, S, step):
    hs, st, ss, hk = _state(S, n)
    host = _host(n)
    res = g.choice(n, size=int(g.integers(0, min(S, n) + 1)), replace=False)
    slots = g.choice(S, size=res.shape[0], replace=False)
    for t, s in zip(res, slots):
        hs[t], st[s], hk[s] = s, t, host[t]
    # stamps from -1 up to step itself (a slot this step already used)
    ss[:] = g.integers(-1, step + 1, size=S)
    return hs, st, ss, hk, host


def test_prefetch_equals_update_without_resident_candidates():
    g = np.random.default_rng(23)
    for case in range(300):
        n = int(g.integers(8, 200))
        S = int(g.integers(1, 40))
        valid = int(g.integers(1, n + 1))
        step = int(g.integers(1, 30))
        hs, st, ss, hk, host = _random_state(g, n, S, step)
        free = np.nonzero(hs < 0)[0]
        cand = g.permutation(free)[: int(g.integers(0, free.shape[0] + 1))].copy()
        cand[g.random(cand.shape[0]) < 0.1] = -1
        a = hot_prefetch(hs, st, ss, hk, host, cand, valid, step)
        b = hot_update(hs, st, ss, hk, host, cand, valid, step)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), case


def test_prefetch_random_invariants():
    g = np.random.default_rng(29)
    for case in range(300):
        n = int(g.integers(8, 200))
        S = int(g.integers(1, 40))
        valid = int(g.integers(1, n + 1))
        step = int(g.integers(1, 30))
        hs, st, ss, hk, host = _random_state(g, n, S, step)
        cand = g.choice(n, size=int(g.integers(1, min(n, 40) + 1)), replace=False)
        cand[g.random(cand.shape[0]) < 0.1] = -1
        hs2, st2, ss2, hk2 = hot_prefetch(hs, st, ss, hk, host, cand, valid, step)
        for s in range(S):
            if st2[s] >= 0:
                assert hs2[st2[s]] == s
                assert (hk2[s] == host[st2[s]]).all()
        for t in range(n):
            if hs2[t] >= 0:
                assert st2[hs2[t]] == t
        chosen = [int(t) for t in cand if 0 <= t < valid]
        held = {int(hs[t]) for t in chosen if hs[t] >= 0}
        fills = [t for t in chosen if hs[t] < 0]
        # resident candidates and slots this step already used keep everything
        for s in held | {s for s in range(S) if ss[s] >= step}:
            assert st2[s] == st[s] and ss2[s] == ss[s] and (hk2[s] == hk[s]).all()
        eligible = [s for s in range(S) if ss[s] < step and s not in held]
        if len(fills) <= len(eligible):
            assert all(hs2[t] >= 0 and ss2[hs2[t]] == step for t in fills)
        replaced = [s for s in range(S) if st2[s] != st[s]]
        assert len(replaced) == min(len(fills), len(eligible))
        kept = [s for s in eligible if s not in replaced]
        for r in replaced:
            for u in kept:
                assert (ss[r], r) < (ss[u], u)
