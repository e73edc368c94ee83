"""Invariant checks shared by the oracle pins and the GPU parity tests."""
import numpy as np


def check_brim_invariants(b, idx, w, slot_expert, E, D):
    """Properties every correct SFD/EPD/BRIM build has (used for the oracle
    here and, in the GPU tests, for the HIP path too)."""
    T, k = idx.shape
    L = E // D
    S = b["S"]
    dev_of = np.empty(E, np.int64)
    loc_of = np.empty(E, np.int64)
    dev_of[slot_expert] = np.arange(E) // L
    loc_of[slot_expert] = np.arange(E) % L
    devsets = [set(dev_of[idx[t]].tolist()) for t in range(T)]
    # every (token, device) pair exactly once in SFD
    assert S == sum(len(s) for s in devsets)
    assert T <= S <= T * min(k, D) or T == 0
    b0 = b["brim0"]
    for t in range(T):
        assert set(np.nonzero(b0[:, t] >= 0)[0].tolist()) == devsets[t]
    vals = b0[b0 >= 0]
    assert np.array_equal(np.sort(vals), np.arange(S))
    for dv in range(D):
        row = b0[dv][b0[dv] >= 0]
        assert np.all(np.diff(row) > 0)
        if row.size:
            assert b["sfd_offset"][dv] <= row[0] and row[-1] < b["sfd_offset"][dv + 1]
    assert b["sfd_offset"][D] == S
    st = b["sfd_token"][:S]
    for dv in range(D):
        seg = st[b["sfd_offset"][dv]:b["sfd_offset"][dv + 1]]
        assert np.all(b0[dv, seg] == np.arange(b["sfd_offset"][dv], b["sfd_offset"][dv + 1]))
    # EPD holds exactly T*k rows; BRIM_1 entries are a permutation of them
    b1 = b["brim1"][:, :S]
    rv = b1[b1 >= 0]
    assert np.array_equal(np.sort(rv), np.arange(T * k))
    slot_of = np.argsort(slot_expert)  # inverse permutation: expert -> slot
    counts = np.bincount(slot_of[idx.ravel()], minlength=E)
    assert np.array_equal(np.diff(b["slot_offset"]), counts)
    for s in range(S):
        t = st[s]
        dv = int(np.searchsorted(b["sfd_offset"], s, side="right") - 1)
        want = sorted(loc_of[e] for e in idx[t] if dev_of[e] == dv)
        assert sorted(np.nonzero(b1[:, s] >= 0)[0].tolist()) == want
    et, es, ew = b["epd_token"], b["epd_sfd"], b["epd_w"]
    for r in range(T * k):
        g = int(np.searchsorted(b["slot_offset"], r, side="right") - 1)
        e = slot_expert[g]
        t = et[r]
        j = np.nonzero(idx[t] == e)[0]
        assert j.size == 1
        assert ew[r] == w[t, j[0]]
        assert es[r] == b0[g // L, t]
        assert b1[g % L, es[r]] == r
    for g in range(E):
        seg = et[b["slot_offset"][g]:b["slot_offset"][g + 1]]
        assert np.all(np.diff(seg) > 0)
