"""CPU oracle of the collaboration-aware MoE layer (Occult) -- TEST
INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path
(``expert_top_router_amd``) never imports it and shares no code with it; the
two meet only through the seeded inputs of ``workloads``.

The arithmetic lives in ``occ_oracle.c`` (plain single-threaded C, built with
``-O2 -fno-fast-math -ffp-contract=off``); this module only marshals numpy
arrays.  Steps and their sources (page and passage):

* routing (O1-O3) -- Expert Coupling in MoE Pretraining, Abstract (each token
  goes to k of E experts); softmax gate, logits as an in-order fp32 FMA chain.
* SFD/EPD layouts and BRIM_0/BRIM_1 (O4-O6) -- Occult, Figure 4 and Figure 5
  captions; Expert Coupling, Abstract (each token to each GPU once).
* expert networks (O8-O9) -- SwiGLU, the pages say only "expert networks".
* pre-reduction and scatter (O10-O11) -- Occult, Figure 4 caption.
* brute force without deduplication (O13) -- Occult, Abstract (exact results).
* co-activation counts (O12) and intra-collaboration share -- Occult,
  Abstract; greedy correlated placement (O-P) -- Expert Coupling, Abstract and
  Occult TL;DR (expert-placement rescheduling).  The greedy is a heuristic
  and no optimality is claimed; the output of the rule is pinned by
  properties, a hand-worked case and a planted-block case.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "occ_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

DT = {"f32": 0, "bf16": 1}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = C.CDLL(_LIB)
    return _lib


def round_dt(v, dtype):
    """The oracle's rounding of a double to the layer dtype (ties to even)."""
    f = lib().orc_round_dt
    f.restype = C.c_double
    f.argtypes = [C.c_double, C.c_int]
    return np.array([f(float(x), DT[dtype]) for x in np.ravel(v)]).reshape(np.shape(v))


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


# ---------------------------------------------------------------------------
def _dt_of(a):
    """Storage type of an array: float32, or bfloat16 kept as uint16 bits."""
    return {np.dtype(np.float32): 0, np.dtype(np.uint16): 1}[np.asarray(a).dtype]


def logits(x, wr, dtype=None):
    """O1: [T, E] float32 logits, each an in-order fmaf chain over d.  The
    storage types of x and wr come from their numpy dtypes."""
    T, d = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    _check(lib().orc_logits(T, d, E, _dt_of(x), _p(np.ascontiguousarray(x)), _dt_of(wr),
                            _p(np.ascontiguousarray(wr)), _p(out)), "logits")
    return out


def topk(lg, k, renorm=0):
    """O2-O3: indices [T, k] (logit desc, expert asc) and softmax weights."""
    lg = _f32(lg)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    _check(lib().orc_topk(T, E, k, int(renorm), _p(lg), _p(idx), _p(w)), "topk")
    return idx, w


def route(x, wr, k, renorm, dtype):
    lg = logits(x, wr, dtype)
    idx, w = topk(lg, k, renorm)
    return lg, idx, w


def prune(idx, w, slot_expert, E, D, budget, rescale):
    """O5': routing-score-based pruning to at most ``budget`` devices per
    token; dropped selections come back as idx -1, w 0."""
    T, k = idx.shape
    io = np.empty((T, k), np.int32)
    wo = np.empty((T, k), np.float32)
    _check(lib().orc_prune(T, k, E, D, _p(_i32(slot_expert)), int(budget), int(rescale),
                           _p(_i32(idx)), _p(_f32(w)), _p(io), _p(wo)), "prune")
    return io, wo


def brim(idx, w, slot_expert, E, D):
    """O4-O6: BRIM_0, BRIM_1 (ld = T*min(k, D)), offsets, SFD/EPD index arrays.
    idx entries of -1 (pairs dropped by pruning) are skipped; EPD then has
    R' = slot_offset[E] rows."""
    T, k = idx.shape
    L = E // D
    ld = T * min(k, D)
    R = T * k
    out = dict(
        brim0=np.empty((D, T), np.int32), brim1=np.empty((L, max(ld, 1)), np.int32),
        sfd_offset=np.empty(D + 1, np.int32), slot_offset=np.empty(E + 1, np.int32),
        sfd_token=np.empty(max(ld, 1), np.int32), epd_token=np.empty(max(R, 1), np.int32),
        epd_sfd=np.empty(max(R, 1), np.int32), epd_w=np.empty(max(R, 1), np.float32))
    S = np.zeros(1, np.int32)
    rc = lib().orc_brim(T, k, E, D, _p(_i32(idx)), _p(_f32(w)), _p(_i32(slot_expert)),
                        _p(out["brim0"]), _p(out["brim1"]), ld, _p(out["sfd_offset"]),
                        _p(out["slot_offset"]), _p(out["sfd_token"]), _p(out["epd_token"]),
                        _p(out["epd_sfd"]), _p(out["epd_w"]), _p(S))
    _check(rc, "brim")
    out["S"] = int(S[0])
    out["ld"] = ld
    Rp = int(out["slot_offset"][E])
    out["R"] = Rp
    out["epd_token"] = out["epd_token"][:Rp]
    out["epd_sfd"] = out["epd_sfd"][:Rp]
    out["epd_w"] = out["epd_w"][:Rp]
    return out


def gather(x, rows):
    """O7: bit copy of rows (SFD = X[sfd_token], EPD = SFD[epd_sfd])."""
    return np.ascontiguousarray(x[np.asarray(rows, dtype=np.int64)])


def expert_rows(x, tok, ex, wgu, wdn, dtype):
    """O8: round(FFN_ex(x[tok])) per row, float32 holding dtype values."""
    tok = _i32(tok)
    ex = _i32(ex)
    n = tok.size
    d = x.shape[1]
    I = wgu.shape[1] // 2
    out = np.empty((n, d), np.float32)
    _check(lib().orc_expert_rows(n, _p(tok), _p(ex), d, I, DT[dtype], _p(np.ascontiguousarray(x)),
                                 _p(np.ascontiguousarray(wgu)), _p(np.ascontiguousarray(wdn)),
                                 _p(out)), "expert_rows")
    return out


def shared_rows(x, tok, wgu_sh, wdn_sh, dtype):
    """O9: round(sum over shared experts of FFN(x[tok]))."""
    tok = _i32(tok)
    n = tok.size
    d = x.shape[1]
    nsh, twoI, _ = wgu_sh.shape
    out = np.empty((n, d), np.float32)
    _check(lib().orc_shared_rows(n, _p(tok), d, twoI // 2, nsh, DT[dtype],
                                 _p(np.ascontiguousarray(x)), _p(np.ascontiguousarray(wgu_sh)),
                                 _p(np.ascontiguousarray(wdn_sh)), _p(out)), "shared_rows")
    return out


def combine(tok, b, T, D, L, d, dtype, out_epd, epd_row=None, shared=None, want_sfd=False):
    """O10-O11 for the tokens ``tok``.  Returns (Y rows, out_SFD rows or None).
    out_SFD comes back as [S, d] (rows of tokens not requested stay NaN)."""
    tok = _i32(tok)
    n = tok.size
    y = np.empty((n, d), np.float32)
    osfd = None
    if want_sfd:
        osfd = np.full((max(b["S"], 1), d), np.nan, np.float32)
    rc = lib().orc_combine(n, _p(tok), T, D, L, b["ld"], d, DT[dtype], _p(b["brim0"]),
                           _p(b["brim1"]), _p(b["epd_w"]), _p(_f32(out_epd)),
                           _p(None if epd_row is None else _i32(epd_row)),
                           _p(None if shared is None else _f32(shared)), _p(osfd), None, _p(y))
    _check(rc, "combine")
    return y, osfd


def combine_direct(tok, b, T, D, L, d, dtype, out_epd, epd_row=None, shared=None):
    """O10': the conventional combine (no pre-reduction) for the tokens ``tok``."""
    tok = _i32(tok)
    n = tok.size
    y = np.empty((n, d), np.float32)
    rc = lib().orc_combine_direct(n, _p(tok), T, D, L, b["ld"], d, DT[dtype], _p(b["brim0"]),
                                  _p(b["brim1"]), _p(b["epd_w"]), _p(_f32(out_epd)),
                                  _p(None if epd_row is None else _i32(epd_row)),
                                  _p(None if shared is None else _f32(shared)), _p(y))
    _check(rc, "combine_direct")
    return y


def bruteforce(tok, x, idx, w, wgu, wdn, dtype, shared=None):
    """O13: the standard MoE layer with no SFD/EPD, for the tokens ``tok``."""
    tok = _i32(tok)
    n = tok.size
    d = x.shape[1]
    I = wgu.shape[1] // 2
    k = idx.shape[1]
    y = np.empty((n, d), np.float32)
    _check(lib().orc_bruteforce(n, _p(tok), d, I, k, DT[dtype], _p(np.ascontiguousarray(x)),
                                _p(_i32(idx)), _p(_f32(w)), _p(np.ascontiguousarray(wgu)),
                                _p(np.ascontiguousarray(wdn)),
                                _p(None if shared is None else _f32(shared)), _p(y)), "bruteforce")
    return y


def coactivation(idx, E, base=None):
    """O12: E x E counts of tokens selecting both experts (diag = n_e)."""
    idx = _i32(idx)
    T, k = idx.shape
    Cm = np.zeros((E, E), np.int32) if base is None else np.array(base, dtype=np.int32)
    _check(lib().orc_coactivation(T, k, E, _p(idx), _p(Cm), 0 if base is None else 1),
           "coactivation")
    return Cm


def cross_coactivation(idx1, E1, idx2, E2):
    """O12': E1 x E2 counts of tokens choosing i at one layer and j at the next."""
    idx1, idx2 = _i32(idx1), _i32(idx2)
    T, k1 = idx1.shape
    k2 = idx2.shape[1]
    A = np.empty((E1, E2), np.int32)
    _check(lib().orc_cross_coactivation(T, k1, E1, _p(idx1), k2, E2, _p(idx2), _p(A)),
           "cross_coactivation")
    return A


def home_device(idx1, E1, A, slot_expert2, D):
    """O12': predicted next-layer home device of every token."""
    idx1 = _i32(idx1)
    T, k1 = idx1.shape
    E2 = A.shape[1]
    home = np.empty(T, np.int32)
    _check(lib().orc_home_device(T, k1, E1, _p(idx1), E2, D, _p(_i32(slot_expert2)), _p(_i32(A)),
                                 _p(home)), "home_device")
    return home


def local_hits(idx2, E2, slot_expert2, D, home):
    """O12': number of next-layer assignments served on the token's home device."""
    idx2 = _i32(idx2)
    T, k2 = idx2.shape
    h = np.zeros(1, np.int64)
    _check(lib().orc_local_hits(T, k2, E2, _p(idx2), D, _p(_i32(slot_expert2)), _p(_i32(home)),
                                _p(h)), "local_hits")
    return int(h[0])


def greedy_placement(Cm, D):
    """O-P: slot_expert [E] from co-activation counts."""
    Cm = _i32(Cm)
    E = Cm.shape[0]
    se = np.empty(E, np.int32)
    _check(lib().orc_greedy_placement(E, D, _p(Cm), _p(se)), "greedy")
    return se


def intra_share(Cm, slot_expert, D):
    Cm = _i32(Cm)
    E = Cm.shape[0]
    a = C.c_longlong()
    b = C.c_longlong()
    _check(lib().orc_intra_share(E, D, _p(Cm), _p(_i32(slot_expert)), C.byref(a), C.byref(b)),
           "intra_share")
    return a.value, b.value


# ---------------------------------------------------------------------------
def layer(inp, tokens=None, with_bruteforce=False, budget=None, rescale=1):
    """Whole layer on the inputs of ``workloads.make_layer`` (duck-typed).

    Routing, BRIMs, gathers and co-activation always run on the full batch.
    The expert arithmetic runs for the tokens in ``tokens`` (default: all)
    and for every EPD row those tokens own."""
    cfg = inp.cfg
    T, d, E, k, D = cfg.T, cfg.d, cfg.E, cfg.k, cfg.D
    L = E // D
    lg, idx, w = route(inp.x, inp.w_router, k, cfg.renorm, cfg.dtype)
    res = dict(logits=lg, idx=idx, w=w, coact=coactivation(idx, E))
    if budget is not None:  # collaboration pruning: the layer runs on the kept pairs
        idx, w = prune(idx, w, inp.slot_expert, E, D, budget, rescale)
        res.update(idx_kept=idx, w_kept=w)
    b = brim(idx, w, inp.slot_expert, E, D)
    res.update(brim=b, S=b["S"])
    if inp.w_gate_up is None:
        return res
    tok = np.arange(T, dtype=np.int32) if tokens is None else _i32(tokens)
    # EPD rows owned by the requested tokens, found through BRIM_0 and BRIM_1
    rows = []
    for dv in range(D):
        s = b["brim0"][dv, tok]
        s = s[s >= 0]
        for l in range(L):
            r = b["brim1"][l, s]
            rows.append(r[r >= 0])
    rows = np.sort(np.concatenate(rows)) if rows else np.zeros(0, np.int64)
    ex_of_slot = np.repeat(np.asarray(inp.slot_expert), np.diff(b["slot_offset"]))
    epd_ex = ex_of_slot[rows] if rows.size else np.zeros(0, np.int32)
    out_rows = expert_rows(inp.x, b["epd_token"][rows], epd_ex, inp.w_gate_up, inp.w_down,
                           cfg.dtype)
    epd_row = np.full(T * k, -1, np.int32)
    epd_row[rows] = np.arange(rows.size, dtype=np.int32)
    shared = None
    if cfg.n_shared:
        shared = shared_rows(inp.x, tok, inp.w_gate_up_sh, inp.w_down_sh, cfg.dtype)
    y, osfd = combine(tok, b, T, D, L, d, cfg.dtype, out_rows, epd_row, shared, want_sfd=True)
    res.update(tokens=tok, epd_rows=rows, out_epd_rows=out_rows, shared=shared, y=y, out_sfd=osfd,
               y_direct=combine_direct(tok, b, T, D, L, d, cfg.dtype, out_rows, epd_row, shared))
    if with_bruteforce:
        res["y_bf"] = bruteforce(tok, inp.x, idx, w, inp.w_gate_up, inp.w_down, cfg.dtype, shared)
    return res
