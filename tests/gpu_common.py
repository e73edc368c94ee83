"""Helpers of the GPU parity tests: run the HIP layer through the C ABI and
the oracle on the same seeded inputs, then compare stage by stage."""
import concurrent.futures as cf
import os
import sys

import numpy as np

import workloads as W
from tests.checks import check_brim_invariants
from tests.tolerance import TOL, assert_close, assert_close_sum

_POOL = cf.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1)))


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def oracle_logits_parallel(orc, x, wr, dtype, parts=16):
    """The oracle's logits, computed on row blocks in threads (ctypes drops
    the GIL); each row is still one in-order fmaf chain per expert."""
    T = x.shape[0]
    bounds = np.linspace(0, T, parts + 1).astype(int)
    futs = [_POOL.submit(orc.logits, x[a:b], wr, dtype) for a, b in zip(bounds[:-1], bounds[1:])
            if b > a]
    return np.concatenate([f.result() for f in futs]) if futs else np.zeros((0, wr.shape[0]),
                                                                            np.float32)


def oracle_expert_rows_parallel(orc, x, tok, ex, wgu, wdn, dtype, parts=16):
    n = len(tok)
    bounds = np.linspace(0, n, parts + 1).astype(int)
    futs = [_POOL.submit(orc.expert_rows, x, tok[a:b], ex[a:b], wgu, wdn, dtype)
            for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    return np.concatenate([f.result() for f in futs]) if futs else np.zeros((0, x.shape[1]),
                                                                            np.float32)


def oracle_layer(orc, inp, tokens=None, budget=None, rescale=1, w_route=None):
    """Oracle results; routing, BRIMs and counts on the full batch, expert
    arithmetic for ``tokens`` (all by default) and their EPD rows.  With a
    budget the BRIMs are built from the pruned selections.  Pruning decides
    by fp32 sums of the routing weights, so ``w_route`` (the GPU's own
    weights, checked against the oracle's softmax separately) is what both
    sides prune from."""
    cfg = inp.cfg
    T, E, k, D = cfg.T, cfg.E, cfg.k, cfg.D
    L = E // D
    lg = oracle_logits_parallel(orc, inp.x, inp.w_router, cfg.dtype)
    idx, w = orc.topk(lg, k, cfg.renorm)
    res = dict(logits=lg, idx=idx, w=w, coact=orc.coactivation(idx, E), budget=budget)
    if budget is None:
        b = orc.brim(idx, w, inp.slot_expert, E, D)
    else:
        ik, wk = orc.prune(idx, w if w_route is None else w_route, inp.slot_expert, E, D,
                           budget, rescale)
        b = orc.brim(ik, wk, inp.slot_expert, E, D)
    res["brim"] = b
    if inp.w_gate_up is None:
        return res
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    rows = []
    for dv in range(D):
        s = b["brim0"][dv, tok]
        s = s[s >= 0]
        for l in range(L):
            r = b["brim1"][l, s]
            rows.append(r[r >= 0])
    rows = np.sort(np.concatenate(rows)).astype(np.int64) if rows else np.zeros(0, np.int64)
    ex_of_slot = np.repeat(np.asarray(inp.slot_expert), np.diff(b["slot_offset"]))
    out_rows = oracle_expert_rows_parallel(orc, inp.x, b["epd_token"][rows].astype(np.int32),
                                           ex_of_slot[rows].astype(np.int32), inp.w_gate_up,
                                           inp.w_down, cfg.dtype)
    epd_row = np.full(T * k, -1, np.int32)
    epd_row[rows] = np.arange(rows.size, dtype=np.int32)
    shared = None
    if cfg.n_shared:
        shared = orc.shared_rows(inp.x, tok, inp.w_gate_up_sh, inp.w_down_sh, cfg.dtype)
    y, osfd = orc.combine(tok, b, T, D, L, cfg.d, cfg.dtype, out_rows, epd_row, shared,
                          want_sfd=True)
    y_direct = orc.combine_direct(tok, b, T, D, L, cfg.d, cfg.dtype, out_rows, epd_row, shared)
    res.update(tokens=tok, epd_rows=rows, out_epd_rows=out_rows, shared=shared, y=y, out_sfd=osfd,
               y_direct=y_direct)
    return res


def gpu_layer(inp, runs=1, poison=True, budget=None, rescale=1):
    """Run the HIP layer (forward + co-activation) and fetch every buffer."""
    import torch
    from expert_top_router_amd.layer import MoELayer, upload_inputs
    cfg = inp.cfg
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert, with_logits=True, budget=budget,
                   rescale=rescale)
    outs = []
    for _ in range(runs):
        if poison:
            lay.poison()
        say(f"  gpu forward {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} D={cfg.D} "
            f"I={cfg.I} dtype={cfg.dtype}")
        lay.forward()
        lay.coactivation()
        torch.cuda.synchronize()
        names = ["logits", "topk_idx", "topk_w", "brim0", "brim1", "sfd_offset", "slot_offset",
                 "sfd_token", "epd_token", "epd_sfd", "epd_w", "S", "sfd", "epd", "out_epd",
                 "out_sfd", "y", "counts"] + (["shared_out"] if cfg.n_shared else [])
        out = {n: lay.host(n) for n in names}
        # the conventional strategy on the same BRIMs: EPD straight from ORI,
        # combine without pre-reduction
        for t in (lay.epd, lay.out_epd, lay.y):
            t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).fill_(-1)
        lay.dispatch_direct()
        lay.expert_ffn()
        lay.combine_direct()
        torch.cuda.synchronize()
        out["epd_direct"] = lay.host("epd")
        out["y_direct"] = lay.host("y")
        outs.append(out)
    del lay
    torch.cuda.empty_cache()
    return outs if runs > 1 else outs[0]


def as_f32(a, dtype):
    return W.to_f32(a, dtype)


def prune_decisions(idx, w_oracle, w_gpu, gpu_brim0, slot_expert, E, D, budget):
    """Tokens whose pruning decision lies within the weights' rounding.

    Pruning ranks a token's devices by the fp32 sum (pick order) of its
    routing weights there.  The oracle's weights (fp64 softmax, one rounding)
    and the GPU's (fp32 softmax) differ in the last bits, so where the
    budget-th and the next device score differ by less than what those
    differences can move a sum (delta = 2k * max |w_gpu - w_oracle| plus a
    few fp32 ulps), either decision is correct.  Returns (near, delta): the
    near-tie tokens, each certified here -- the GPU kept exactly `budget`
    devices, none scoring (oracle weights) more than delta below the
    oracle's budget-th score and none dropped more than delta above it."""
    T, k = idx.shape
    L = E // D
    slot_of = np.empty(E, np.int64)
    slot_of[np.asarray(slot_expert)] = np.arange(E)
    dev = slot_of[idx] // L
    maxdiff = float(np.max(np.abs(w_gpu.astype(np.float64) - w_oracle))) if T else 0.0
    delta = 2 * k * maxdiff + 8 * k * float(np.finfo(np.float32).eps)
    near = []
    for t in range(T):
        sc = {}
        for j in range(k):  # fp32 sums in pick order, as the pruning rule states
            dv = int(dev[t, j])
            sc[dv] = np.float32(sc.get(dv, np.float32(0)) + np.float32(w_oracle[t, j]))
        if len(sc) <= budget:
            continue
        order = sorted(sc, key=lambda dv: (-float(sc[dv]), dv))
        sb, snext = float(sc[order[budget - 1]]), float(sc[order[budget]])
        if sb - snext > delta:
            continue
        kept = {dv for dv in sc if gpu_brim0[dv, t] >= 0}
        assert len(kept) == budget, (t, kept)
        for dv in sc:
            if dv in kept:
                assert float(sc[dv]) >= sb - delta, (t, dv, sc, kept)
            else:
                assert float(sc[dv]) <= sb + delta, (t, dv, sc, kept)
        near.append(t)
    return np.array(near, dtype=np.int64), delta


def compare(g, o, inp, full=True, pruned_w_exact=True):
    """Stage-by-stage comparison; integer work bit-exact, floats by TOL.
    pruned_w_exact: pruned layers' rescaled weights bit for bit (both sides
    pruned from the same fp32 weights), else within the fp32 tolerance."""
    cfg = inp.cfg
    dt = cfg.dtype
    T, k, D, E = cfg.T, cfg.k, cfg.D, cfg.E
    # routing: logits and indices bit-exact (same fp32 FMA chain), weights by 1e-4
    assert np.array_equal(g["logits"].view(np.uint32), o["logits"].view(np.uint32)), "logits"
    assert np.array_equal(g["topk_idx"], o["idx"]), "topk_idx"
    assert_close(g["topk_w"], o["w"], "f32", "topk_w")
    b = o["brim"]
    S, Rp = b["S"], b["R"]
    pruned = o.get("budget") is not None
    assert int(g["S"][0]) == S, ("S", int(g["S"][0]), S)
    for name in ("brim0", "sfd_offset", "slot_offset"):
        assert np.array_equal(g[name], b[name]), name
    assert np.array_equal(g["brim1"][:, :S], b["brim1"][:, :S]), "brim1"
    assert np.array_equal(g["sfd_token"][:S], b["sfd_token"][:S]), "sfd_token"
    assert np.array_equal(g["epd_token"][:Rp], b["epd_token"]), "epd_token"
    assert np.array_equal(g["epd_sfd"][:Rp], b["epd_sfd"]), "epd_sfd"
    if pruned and pruned_w_exact:
        # the same fp32 scores and rescaling on both sides: bit for bit
        assert np.array_equal(g["epd_w"][:Rp].view(np.uint32), b["epd_w"].view(np.uint32)), \
            "epd_w (pruned)"
    elif pruned:
        assert_close(g["epd_w"][:Rp], b["epd_w"], "f32", "epd_w (pruned, own weights)")
    else:
        # epd_w is a copy of the GPU's own routing weights
        assert np.array_equal(g["epd_w"], g["topk_w"].reshape(-1)[
            _flat_pos(g["topk_idx"], b, inp.slot_expert, k)]), "epd_w copy"
    assert np.array_equal(g["counts"], o["coact"]), "coactivation"
    # dispatch: bit copies
    xs = inp.x
    assert np.array_equal(g["sfd"][:S], xs[b["sfd_token"][:S]]), "sfd"
    assert np.array_equal(g["epd"][:Rp], xs[b["epd_token"]]), "epd"
    gb = dict(brim0=g["brim0"], brim1=g["brim1"], sfd_offset=g["sfd_offset"],
              slot_offset=g["slot_offset"], sfd_token=g["sfd_token"], epd_token=g["epd_token"],
              epd_sfd=g["epd_sfd"], epd_w=g["epd_w"], S=S)
    if full and not pruned:
        check_brim_invariants(gb, g["topk_idx"], g["topk_w"], inp.slot_expert, E, D)
    if "y" not in o:
        return
    rows = o["epd_rows"]
    g_rows = as_f32(g["out_epd"][rows], dt)
    assert_close(g_rows, o["out_epd_rows"], dt, "out_epd")
    tok = o["tokens"]
    g_sh = None
    if cfg.n_shared:
        g_sh = as_f32(g["shared_out"][tok], dt)
        assert_close(g_sh, o["shared"], dt, "shared_out")
    srows = np.unique(b["brim0"][:, tok][b["brim0"][:, tok] >= 0])
    # the combine's own arithmetic: the oracle's pre-reduction and scatter of
    # the GPU's expert outputs
    import oracle as orc
    L = E // D
    epd_row = np.full(max(Rp, 1), -1, np.int32)
    epd_row[rows] = np.arange(rows.size, dtype=np.int32)
    y_s, osfd_s = orc.combine(tok, b, T, D, L, cfg.d, dt, g_rows, epd_row, g_sh, want_sfd=True)
    assert_close(as_f32(g["out_sfd"][srows], dt), osfd_s[srows], dt, "out_sfd (combine alone)")
    assert_close(as_f32(g["y"][tok], dt), y_s, dt, "y (combine alone)")
    # end to end, each element against the size of its summands
    mag_sfd, mag_y = summand_magnitudes(o, b, srows, cfg.d)
    assert_close_sum(as_f32(g["out_sfd"][srows], dt), o["out_sfd"][srows], mag_sfd, dt, "out_sfd")
    assert_close_sum(as_f32(g["y"][tok], dt), o["y"], mag_y, dt, "y")
    if "y_direct" in g:
        assert np.array_equal(g["epd_direct"][:Rp], xs[b["epd_token"]]), "epd (direct dispatch)"
        yd_s = orc.combine_direct(tok, b, T, D, L, cfg.d, dt, g_rows, epd_row, g_sh)
        assert_close(as_f32(g["y_direct"][tok], dt), yd_s, dt, "y (direct combine alone)")
        assert_close_sum(as_f32(g["y_direct"][tok], dt), o["y_direct"], mag_y, dt,
                         "y (direct combine)")


def summand_magnitudes(o, b, srows, d):
    """Per element: sum over an SFD row's EPD rows of |w * out_epd| (for the
    rows srows), and over a token's EPD rows plus |shared_out| (for the
    oracle's tokens), from the oracle's values."""
    rows = o["epd_rows"]
    term = (np.abs(o["out_epd_rows"].astype(np.float64))
            * np.abs(b["epd_w"][rows].astype(np.float64))[:, None])
    mag_sfd = np.zeros((len(srows), d))
    pos_s = np.searchsorted(srows, b["epd_sfd"][rows])
    np.add.at(mag_sfd, pos_s, term)
    tok = o["tokens"]
    mag_y = np.zeros((len(tok), d))
    np.add.at(mag_y, np.searchsorted(tok, b["epd_token"][rows]), term)
    if o.get("shared") is not None:
        mag_y += np.abs(o["shared"].astype(np.float64))
    return mag_sfd, mag_y


def _flat_pos(idx, b, slot_expert, k):
    """Position t*k + j of each EPD row's (token, choice) in topk arrays."""
    slot_of_row = np.repeat(np.arange(len(slot_expert)), np.diff(b["slot_offset"]))
    t = b["epd_token"].astype(np.int64)
    e = np.asarray(slot_expert)[slot_of_row]
    j = np.argmax(idx[t] == e[:, None], axis=1) if t.size else np.zeros(0, np.int64)
    return t * k + j
