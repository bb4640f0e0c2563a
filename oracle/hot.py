"""Plain CPU oracle of the hot-buffer replacement (test infrastructure only).

TEST INFRASTRUCTURE ONLY: nothing in the product path imports this module.

"XM-Sparse: Pushing the Throughput Frontier of Sparse Attention with Netpreme
X-Mem" (Figure 1 and the decode-path list) has decode GPUs keep a hot KV
buffer per request and layer in HBM and fetch only the missing selected rows;
it keeps HiSparse's cache management but measures fixed miss rates with
prefetch off, and states no replacement rule.  The rule taken here (least
recently used, the plainest cache policy) is, per request, after a
step that selected the tokens T (selection order, padding and tokens past the
valid length dropped):

1. every selected token held in a slot (a hit) stamps that slot with `step`;
2. the selected tokens not held (the misses, in selection order) go into the
   slots not stamped `step` that have the smallest (stamp, slot index) --
   least recently used first, an empty slot carrying stamp -1 -- taken in
   ascending slot order, one per miss; a slot's previous token loses its
   slot, the new token's row is copied into it and the slot is stamped;
3. misses beyond the slots available stay out.

Parity status: pinned by tests/test_oracle_hot_pins.py (worked examples
computed by hand from the rules, a textbook LRU cache when one token is
selected per step, the invariants of the maps and of the LRU order on random
states, and, for the prefetch, agreement with the update wherever no
candidate is resident).
"""
import numpy as np


def hot_update(hot_slot, slot_token, slot_stamp, hot_kv, host_kv, sel, valid, step):
    """One request.  hot_slot [n] (token -> slot or -1), slot_token [S]
    (slot -> token or -1), slot_stamp [S], hot_kv [S][d] and host_kv [n][d]
    (any dtype, rows copied as they are), sel [k] token ids (-1 = padding),
    valid = the request's valid tokens, step = the stamp of this update.
    Returns new arrays (hot_slot, slot_token, slot_stamp, hot_kv)."""
    hs = np.array(hot_slot, copy=True)
    st = np.array(slot_token, copy=True)
    ss = np.array(slot_stamp, copy=True)
    hk = np.array(hot_kv, copy=True)
    S = st.shape[0]
    misses = []
    for t in sel:
        t = int(t)
        if t < 0 or t >= valid:
            continue
        s = int(hs[t])
        if s >= 0:
            ss[s] = step
        else:
            misses.append(t)
    eligible = [s for s in range(S) if ss[s] < step]
    eligible.sort(key=lambda s: (int(ss[s]), s))
    victims = sorted(eligible[: len(misses)])
    for v, t in zip(victims, misses):
        u = int(st[v])
        if u >= 0:
            hs[u] = -1
        hk[v] = host_kv[t]
        hs[t] = v
        st[v] = t
        ss[v] = step
    return hs, st, ss, hk


def hot_prefetch(hot_slot, slot_token, slot_stamp, hot_kv, host_kv, cand, valid, step):
    """Prefetch into the hot buffer of one request, after the update of step
    `step`.  The pages keep HiSparse's prefetch mechanism without stating it
    (every measured run has it off), and CXL-SpecKV's abstract only names
    speculative preloading of the entries future tokens will use; the rule
    taken here is:

    1. candidates (cand, in list order; padding and tokens past the valid
       length dropped) that are resident stay where they are, keep their
       stamps and are not replaced by this call;
    2. the other candidates take the slots that are neither stamped `step`
       nor holding a resident candidate, smallest (stamp, slot index) first,
       in ascending slot order, one per candidate: the slot's previous token
       loses its slot, the candidate's host row is copied in and the slot is
       stamped `step`;
    3. candidates beyond the slots available stay out.

    Same arrays and return values as hot_update."""
    hs = np.array(hot_slot, copy=True)
    st = np.array(slot_token, copy=True)
    ss = np.array(slot_stamp, copy=True)
    hk = np.array(hot_kv, copy=True)
    S = st.shape[0]
    held = set()
    fills = []
    for t in cand:
        t = int(t)
        if t < 0 or t >= valid:
            continue
        s = int(hs[t])
        if s >= 0:
            held.add(s)
        else:
            fills.append(t)
    eligible = [s for s in range(S) if ss[s] < step and s not in held]
    eligible.sort(key=lambda s: (int(ss[s]), s))
    victims = sorted(eligible[: len(fills)])
    for v, t in zip(victims, fills):
        u = int(st[v])
        if u >= 0:
            hs[u] = -1
        hk[v] = host_kv[t]
        hs[t] = v
        st[v] = t
        ss[v] = step
    return hs, st, ss, hk
