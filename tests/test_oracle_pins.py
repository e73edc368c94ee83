"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks one oracle step against what the pages and the mathematics
fix: a hand-worked example (tests/golden/), closed forms, library routines on
special cases, invariants the Occult layouts must satisfy, and brute force on
tiny inputs.  Together they fail on a dropped term, a wrong sign or index or a
transposed operand anywhere in the oracle.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import workloads as W
from tests.checks import check_brim_invariants
from tests.tolerance import rel_err

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(v):
    return W.from_f64(np.asarray(v, np.float64), "bf16")


def _f32(v):
    return np.asarray(v, np.float32)


# ---------------------------------------------------------------------------
# O1 logits: in-order fp32 FMA chain
# ---------------------------------------------------------------------------
def test_logits_integer_inputs_are_exact(orc):
    """Small integers: every partial sum is exact in fp32, so the chain equals
    the integer matrix product X W^T (pins indices and the transpose)."""
    rng = np.random.default_rng(1)
    T, d, E = 9, 37, 5
    x = rng.integers(-4, 5, size=(T, d))
    w = rng.integers(-3, 4, size=(E, d))
    lg = orc.logits(_f32(x), _f32(w), "f32")
    assert np.array_equal(lg.astype(np.int64), x @ w.T)
    lgb = orc.logits(_bf16(x), _bf16(w), "bf16")  # same values as bf16 storage
    assert np.array_equal(lgb.astype(np.int64), x @ w.T)


def test_logits_one_hot_token_reads_router_column(orc):
    rng = np.random.default_rng(2)
    d, E = 16, 6
    w = _f32(rng.standard_normal((E, d)))
    x = np.eye(d, dtype=np.float32)
    lg = orc.logits(x, w, "f32")
    assert np.array_equal(lg, w.T)  # logits[t = j][e] = w[e][j]


def test_logits_chain_order_and_single_rounding(orc):
    """Order: 2^24 + 1 - 2^24 in that order is 0 in fp32 (the middle sum
    ties to even), though the exact sum is 1.  Fusion: fma(1+2^-12,
    1+2^-12, -1) keeps the 2^-24 term that a separate product would drop."""
    x = _f32([[1.0, 1.0, 1.0], [-1.0, 1.0 + 2.0 ** -12, 0.0]])
    w = _f32([[2.0 ** 24, 1.0, -(2.0 ** 24)], [1.0, 1.0 + 2.0 ** -12, 0.0]])
    lg = orc.logits(x, w, "f32")
    assert lg[0, 0] == 0.0
    assert lg[1, 1] == np.float32(2.0 ** -11 + 2.0 ** -24)
    assert lg[0, 1] == np.float32(2.0 + 2.0 ** -12)  # x0 . w1 = 1 + (1+2^-12) + 0, exact


def test_logits_within_textbook_error_bound(orc):
    """|chain - exact| <= gamma_d * sum |x_j w_j| (Higham, recursive sums with
    one rounding per step), exact taken in float64 from bf16 inputs."""
    cfg = W.CONFIGS["olmoe_bf16"]
    x = W.make_tokens(cfg, T=64)
    wr = W.make_router(cfg)
    lg = orc.logits(x, wr, "bf16").astype(np.float64)
    xf = W.to_f32(x, "bf16").astype(np.float64)
    wf = W.to_f32(wr, "bf16").astype(np.float64)
    exact = xf @ wf.T
    d = cfg.d
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    bound = gamma * (np.abs(xf) @ np.abs(wf).T)
    assert np.all(np.abs(lg - exact) <= bound)
    # and not trivially: the chain is not the exact value everywhere
    assert np.any(lg != exact)


# ---------------------------------------------------------------------------
# O2-O3 top-k and weights
# ---------------------------------------------------------------------------
def test_topk_matches_stable_argsort(orc):
    rng = np.random.default_rng(3)
    for E, k in [(8, 2), (64, 8), (128, 6), (5, 5)]:
        lg = _f32(rng.standard_normal((200, E)))
        lg[:50] = np.round(lg[:50] * 2) / 2  # many exact ties
        idx, _ = orc.topk(lg, k)
        ref = np.argsort(-lg, axis=1, kind="stable")[:, :k]
        assert np.array_equal(idx, ref)


def test_topk_ties_go_to_lower_index_and_nan_is_minus_inf(orc):
    lg = _f32([[1.0, 3.0, 3.0, 2.0],
               [np.nan, 0.5, 0.5, -np.inf],
               [0.0, -0.0, 0.0, -1.0]])
    idx, _ = orc.topk(lg, 3)
    assert idx[0].tolist() == [1, 2, 3]
    assert idx[1].tolist() == [1, 2, 0]  # NaN ranks with -inf; lower index first
    assert idx[2].tolist() == [0, 1, 2]  # -0 == +0


def test_softmax_weights_closed_form_and_library(orc):
    from scipy.special import softmax
    lg = _f32([[1.0, 3.0, 3.0, 2.0]])
    idx, w = orc.topk(lg, 2, renorm=0)
    z = math.exp(-2) + 1 + 1 + math.exp(-1)
    assert abs(w[0, 0] - 1 / z) < 1e-7 and abs(w[0, 1] - 1 / z) < 1e-7
    _, wr = orc.topk(lg, 2, renorm=1)
    assert np.allclose(wr, 0.5, atol=1e-7)
    # two experts: w_0 = 1 / (1 + e^{-(l0 - l1)})
    lg2 = _f32([[0.75, -0.5]])
    _, w2 = orc.topk(lg2, 2)
    assert abs(w2[0, 0] - 1 / (1 + math.exp(-1.25))) < 1e-7
    rng = np.random.default_rng(4)
    lgr = _f32(rng.standard_normal((100, 64)) * 2)
    idx, w = orc.topk(lgr, 8)
    p = softmax(lgr.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(p, idx, 1), rtol=1e-6, atol=0)
    _, wn = orc.topk(lgr, 8, renorm=1)
    assert np.allclose(wn.sum(1), 1.0, atol=1e-6)


# ---------------------------------------------------------------------------
# O4-O6 BRIMs: hand-worked example and invariants
# ---------------------------------------------------------------------------
def _golden():
    with open(os.path.join(GOLD, "brim_two_devices.json")) as f:
        return json.load(f)


def test_brim_hand_worked_two_devices(orc):
    g = _golden()
    idx = np.array(g["idx"], np.int32)
    w = np.array(g["w"], np.float32)
    b = orc.brim(idx, w, np.array(g["slot_expert"], np.int32), g["E"], g["D"])
    assert b["S"] == g["S"]
    assert b["sfd_offset"].tolist() == g["sfd_offset"]
    assert b["sfd_token"][:b["S"]].tolist() == g["sfd_token"]
    assert b["brim0"].tolist() == g["brim0"]
    assert b["brim1"][:, :b["S"]].tolist() == g["brim1_valid_columns"]
    assert b["slot_offset"].tolist() == g["slot_offset"]
    assert b["epd_token"].tolist() == g["epd_token"]
    assert b["epd_sfd"].tolist() == g["epd_sfd"]
    assert b["epd_w"].tolist() == g["epd_w"]
    C = orc.coactivation(idx, g["E"])
    assert C.tolist() == g["coactivation"]
    se = orc.greedy_placement(C, g["D"])
    assert se.tolist() == g["greedy_slot_expert"]
    assert orc.intra_share(C, se, g["D"]) == (g["intra_pairs"], g["total_pairs"])


def _random_routing(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k,D", [(50, 8, 2, 2), (64, 16, 4, 4), (33, 12, 3, 3), (40, 8, 8, 8)])
def test_brim_invariants_random(orc, T, E, k, D):
    rng = np.random.default_rng(T * 7 + E)
    idx = _random_routing(rng, T, E, k)
    w = _f32(rng.random((T, k)))
    for se in [np.arange(E, dtype=np.int32), rng.permutation(E).astype(np.int32)]:
        b = orc.brim(idx, w, se, E, D)
        check_brim_invariants(b, idx, w, se, E, D)


def test_brim_one_device_is_identity(orc):
    rng = np.random.default_rng(5)
    T, E, k = 40, 8, 3
    idx = _random_routing(rng, T, E, k)
    b = orc.brim(idx, _f32(rng.random((T, k))), np.arange(E, dtype=np.int32), E, 1)
    assert b["S"] == T
    assert np.array_equal(b["brim0"][0], np.arange(T))
    assert np.array_equal(b["sfd_token"][:T], np.arange(T))


def test_brim_one_expert_per_device_is_textbook_permutation(orc):
    """L = 1 (D = E): no deduplication is possible, S = T*k, and the EPD order
    is the stable argsort of the flattened slot keys (the usual MoE permute)."""
    rng = np.random.default_rng(6)
    T, E, k = 37, 8, 3
    idx = _random_routing(rng, T, E, k)
    se = rng.permutation(E).astype(np.int32)
    b = orc.brim(idx, _f32(rng.random((T, k))), se, E, E)
    assert b["S"] == T * k
    slot_of = np.argsort(se)
    order = np.argsort(slot_of[idx.ravel()], kind="stable")
    assert np.array_equal(b["epd_token"], order // k)


def test_sparse_matrix_reading_and_round_trip(orc):
    """SFD = P0 X and EPD = P1 SFD with 0/1 selection matrices; the inverse
    gather through sfd_token gives back X (every token has a device)."""
    rng = np.random.default_rng(7)
    T, E, k, D, d = 30, 8, 2, 4, 5
    idx = _random_routing(rng, T, E, k)
    w = _f32(rng.random((T, k)))
    b = orc.brim(idx, w, np.arange(E, dtype=np.int32), E, D)
    S = b["S"]
    X = rng.standard_normal((T, d))
    P0 = np.zeros((S, T))
    P0[np.arange(S), b["sfd_token"][:S]] = 1
    P1 = np.zeros((T * k, S))
    P1[np.arange(T * k), b["epd_sfd"]] = 1
    sfd = orc.gather(X, b["sfd_token"][:S])
    epd = orc.gather(sfd, b["epd_sfd"])
    assert np.array_equal(P0 @ X, sfd)
    assert np.array_equal(P1 @ sfd, epd)
    assert np.array_equal(epd, X[b["epd_token"]])
    back = np.full_like(X, np.nan)
    back[b["sfd_token"][:S]] = sfd
    assert np.array_equal(back, X)
    # BRIM_0 gathers the other way: X[t] = SFD[BRIM_0[d][t]] wherever >= 0
    for dv in range(D):
        ok = b["brim0"][dv] >= 0
        assert np.array_equal(sfd[b["brim0"][dv][ok]], X[ok])


# ---------------------------------------------------------------------------
# O8-O9 expert networks
# ---------------------------------------------------------------------------
def _swiglu_np(xf, wg, wu, wd, dtype):
    """numpy float64 matrix products on a whole expert at once."""
    a = xf @ wg.T
    b = xf @ wu.T
    h = a / (1.0 + np.exp(-a)) * b
    h = W.to_f32(W.from_f64(h, dtype), dtype).astype(np.float64) if dtype == "bf16" else \
        h.astype(np.float32).astype(np.float64)
    return h @ wd.T


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_expert_rows_against_numpy_matmul(orc, dtype):
    rng = np.random.default_rng(8)
    E, I, d, n = 3, 24, 16, 20
    wgu = W.from_f64(rng.standard_normal((E, 2 * I, d)) / 4, dtype)
    wdn = W.from_f64(rng.standard_normal((E, d, I)) / 4, dtype)
    x = W.from_f64(rng.standard_normal((10, d)), dtype)
    tok = rng.integers(0, 10, n).astype(np.int32)
    ex = rng.integers(0, E, n).astype(np.int32)
    out = orc.expert_rows(x, tok, ex, wgu, wdn, dtype)
    xf = W.to_f32(x, dtype).astype(np.float64)
    g = W.to_f32(wgu, dtype).astype(np.float64)
    dn = W.to_f32(wdn, dtype).astype(np.float64)
    for r in range(n):
        ref = _swiglu_np(xf[tok[r]][None], g[ex[r], :I], g[ex[r], I:], dn[ex[r]], dtype)[0]
        assert rel_err(out[r], ref) <= (1e-6 if dtype == "f32" else 1e-2)


def test_expert_rows_scalar_closed_form(orc):
    """d = I = 1: y = wd * silu(x wg) * (x wu) with silu(2) = 2/(1+e^-2)."""
    x = _f32([[2.0]])
    wgu = _f32([[[1.0], [1.5]]])
    wdn = _f32([[[0.5]]])
    out = orc.expert_rows(x, [0], [0], wgu, wdn, "f32")
    h = np.float32(2.0 / (1 + math.exp(-2.0)) * 3.0)
    assert out[0, 0] == np.float32(float(h) * 0.5)


def test_two_shared_experts_equal_one_concatenated(orc):
    """sum_s W_down_s h_s = [W_down_0 | W_down_1] [h_0; h_1]: exact identity."""
    rng = np.random.default_rng(9)
    d, I, n = 8, 6, 7
    wgu = _f32(rng.standard_normal((2, 2 * I, d)) / 3)
    wdn = _f32(rng.standard_normal((2, d, I)) / 3)
    x = _f32(rng.standard_normal((n, d)))
    tok = np.arange(n, dtype=np.int32)
    two = orc.shared_rows(x, tok, wgu, wdn, "f32")
    cat_gu = np.concatenate([wgu[0, :I], wgu[1, :I], wgu[0, I:], wgu[1, I:]])[None]
    cat_dn = np.concatenate([wdn[0], wdn[1]], axis=1)[None]
    one = orc.shared_rows(x, tok, cat_gu, cat_dn, "f32")
    assert np.array_equal(two, one)


# ---------------------------------------------------------------------------
# O10-O13 combine
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_fp32"])
def test_layer_matches_bruteforce(orc, name):
    cfg = W.CONFIGS[name]
    inp = W.make_layer(cfg)
    r = orc.layer(inp, with_bruteforce=True)
    assert rel_err(r["y"], r["y_bf"]) <= 1e-6


def test_layer_matches_bruteforce_bf16_with_shared_experts(orc):
    cfg = W.CONFIGS["dsv2lite_bf16"].replace(T=64, d=64, E=16, I=32, I_shared=32, D=4, k=6)
    inp = W.make_layer(cfg)
    r = orc.layer(inp, with_bruteforce=True)
    assert rel_err(r["y"], r["y_bf"]) <= 2e-2
    assert r["S"] < cfg.R  # deduplication happened


@pytest.mark.parametrize("renorm", [0, 1])
def test_identity_expert_combine(orc, renorm):
    """With out_EPD := EPD the combine returns (sum_j w_j) X, and X itself
    under renormalised weights (fp32 rounding only)."""
    rng = np.random.default_rng(10)
    T, E, k, D, d = 64, 16, 4, 4, 12
    x = _f32(rng.standard_normal((T, d)))
    wr = _f32(rng.standard_normal((E, d)))
    _, idx, w = orc.route(x, wr, k, renorm, "f32")
    b = orc.brim(idx, w, np.arange(E, dtype=np.int32), E, D)
    epd = orc.gather(orc.gather(x, b["sfd_token"][:b["S"]]), b["epd_sfd"])
    y, _ = orc.combine(np.arange(T), b, T, D, E // D, d, "f32", epd)
    yd = orc.combine_direct(np.arange(T), b, T, D, E // D, d, "f32", epd)
    want = x.astype(np.float64) * w.sum(1, dtype=np.float64)[:, None]
    assert rel_err(y, want) <= 1e-6
    assert rel_err(yd, want) <= 1e-6
    if renorm:
        assert rel_err(y, x) <= 1e-6
        assert rel_err(yd, x) <= 1e-6


def test_combine_invariant_under_placement(orc):
    cfg = W.CONFIGS["olmoe_bf16"].replace(T=128, d=64, E=16, I=32, D=4, k=4, dtype="f32")
    inp = W.make_layer(cfg)
    base = orc.layer(inp)
    inp.slot_expert = orc.greedy_placement(base["coact"], cfg.D)
    moved = orc.layer(inp)
    assert np.array_equal(moved["idx"], base["idx"])
    assert rel_err(moved["y"], base["y"]) <= 1e-6


# ---------------------------------------------------------------------------
# O10' the conventional strategy (one row per (token, expert) pair, Occult
# Figure 2 caption): EPD straight from ORI, combine without pre-reduction
# ---------------------------------------------------------------------------
def test_direct_dispatch_is_the_two_stage_gather(orc):
    """x[epd_token] is bit for bit the ORI -> SFD -> EPD result."""
    rng = np.random.default_rng(20)
    T, E, k, D, d = 70, 12, 3, 3, 10
    x = _f32(rng.standard_normal((T, d)))
    _, idx, w = orc.route(x, _f32(rng.standard_normal((E, d))), k, 0, "f32")
    b = orc.brim(idx, w, rng.permutation(E).astype(np.int32), E, D)
    two = orc.gather(orc.gather(x, b["sfd_token"][:b["S"]]), b["epd_sfd"])
    one = orc.gather(x, b["epd_token"])
    assert np.array_equal(one.view(np.uint32), two.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_direct_combine_matches_bruteforce(orc, dtype):
    """The conventional combine is the standard layer itself: both round one
    fp64 sum of the same exact products (fp32 weight x dtype output), only
    the order differs."""
    cfg = W.CONFIGS["olmoe_bf16"].replace(T=96, d=64, E=16, I=32, D=4, k=4, dtype=dtype)
    inp = W.make_layer(cfg)
    r = orc.layer(inp, with_bruteforce=True)
    if dtype == "bf16":
        assert np.array_equal(r["y_direct"], r["y_bf"])
    else:
        assert rel_err(r["y_direct"], r["y_bf"]) <= 1e-6
    assert r["S"] < cfg.R  # the Occult path deduplicated; the direct one did not need to


def test_direct_combine_drops_no_row(orc):
    """With out_EPD = 1 in every element and shared = 0, y_direct = sum of
    the token's k weights (and with renormalised weights exactly 1)."""
    rng = np.random.default_rng(21)
    T, E, k, D, d = 40, 8, 3, 2, 4
    x = _f32(rng.standard_normal((T, d)))
    for renorm in (0, 1):
        _, idx, w = orc.route(x, _f32(rng.standard_normal((E, d))), k, renorm, "f32")
        b = orc.brim(idx, w, np.arange(E, dtype=np.int32), E, D)
        ones = np.ones((T * k, d), np.float32)
        y = orc.combine_direct(np.arange(T), b, T, D, E // D, d, "f32", ones)
        want = np.repeat(w.sum(1, dtype=np.float64)[:, None], d, 1)
        assert rel_err(y, want) <= 1e-6
        if renorm:
            assert np.allclose(y, 1.0, rtol=0, atol=4e-7)


# ---------------------------------------------------------------------------
# O5' routing-score-based collaboration pruning (Occult TL;DR, budget C_T)
# ---------------------------------------------------------------------------
def test_prune_hand_worked(orc):
    from fractions import Fraction
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "prune_budget.json")))
    idx = np.array(g["idx"], np.int32)
    w = np.array(g["w"], np.float32)
    se = np.array(g["slot_expert"], np.int32)
    for case in g["cases"]:
        io, wo = orc.prune(idx, w, se, g["E"], g["D"], case["budget"], case["rescale"])
        assert np.array_equal(io, np.array(case["idx"], np.int32)), case
        want = np.array([[float(Fraction(v)) for v in row] for row in case["w"]])
        assert np.allclose(wo, want, rtol=1e-6, atol=0), case
        b = orc.brim(io, wo, se, g["E"], g["D"])
        assert b["S"] == case["S"] and b["R"] == case["R"], case
        check_brim_invariants_pruned(b, io, g["D"], g["E"], se)


def check_brim_invariants_pruned(b, io, D, E, se):
    """Every kept (token, device) pair has one SFD row and every kept
    (token, expert) pair one EPD row; dropped pairs have none."""
    T, k = io.shape
    L = E // D
    dev_of = np.empty(E, np.int64)
    dev_of[se] = np.arange(E) // L
    for t in range(T):
        kept = io[t][io[t] >= 0]
        devs = set(dev_of[kept].tolist())
        for dv in range(D):
            assert (b["brim0"][dv, t] >= 0) == (dv in devs)
    pairs = sorted((int(t), int(e)) for t in range(T) for e in io[t] if e >= 0)
    ex_of_row = np.repeat(se, np.diff(b["slot_offset"]))
    got = sorted(zip(b["epd_token"].tolist(), ex_of_row.tolist()))
    assert got == pairs


def test_prune_keeps_the_heaviest_devices_brute_force(orc):
    """The kept devices carry the largest summed weight of any device subset
    of the budget's size (checked over all subsets), and rescaling keeps the
    token's total weight."""
    rng = np.random.default_rng(30)
    for E, D, k, budget in [(8, 4, 3, 1), (12, 4, 4, 2), (16, 8, 6, 3), (6, 3, 3, 2)]:
        T = 60
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        w = _f32(rng.dirichlet(np.ones(k), size=T))
        se = rng.permutation(E).astype(np.int32)
        io, wo = orc.prune(idx, w, se, E, D, budget, 1)
        L = E // D
        dev_of = np.empty(E, np.int64)
        dev_of[se] = np.arange(E) // L
        for t in range(T):
            sums = {}
            for e, wt in zip(idx[t], w[t].astype(np.float64)):
                sums[int(dev_of[e])] = sums.get(int(dev_of[e]), 0.0) + wt
            m = min(budget, len(sums))
            best = max(sum(sums[dv] for dv in c) for c in itertools.combinations(sums, m))
            kept = {int(dev_of[e]) for e in io[t] if e >= 0}
            assert len(kept) == m
            assert abs(sum(sums[dv] for dv in kept) - best) <= 1e-6
            assert abs(float(wo[t].sum(dtype=np.float64)) - float(w[t].sum(dtype=np.float64))) <= 1e-6
            assert np.all(wo[t][io[t] < 0] == 0)
        # a budget of D changes nothing
        io_d, wo_d = orc.prune(idx, w, se, E, D, D, 1)
        assert np.array_equal(io_d, idx) and np.array_equal(wo_d, w)


def test_pruned_layer_is_the_standard_layer_on_the_kept_pairs(orc):
    cfg = W.CONFIGS["olmoe_bf16"].replace(T=96, d=64, E=16, I=32, D=4, k=4, dtype="f32")
    inp = W.make_layer(cfg)
    full = orc.layer(inp)
    for budget in (1, 2, 3):
        r = orc.layer(inp, with_bruteforce=True, budget=budget)
        assert rel_err(r["y"], r["y_bf"]) <= 1e-6
        assert rel_err(r["y_direct"], r["y_bf"]) <= 1e-6
        assert r["S"] <= budget * cfg.T and r["S"] <= full["S"]
        assert r["brim"]["R"] < cfg.R
        assert (r["brim"]["brim0"] >= 0).sum(0).max() <= budget


# ---------------------------------------------------------------------------
# O12 co-activation and placement
# ---------------------------------------------------------------------------
def test_coactivation_brute_force_and_sums(orc):
    rng = np.random.default_rng(11)
    for T, E, k in [(50, 8, 2), (80, 16, 6)]:
        idx = _random_routing(rng, T, E, k)
        C = orc.coactivation(idx, E)
        ref = np.zeros((E, E), np.int64)
        for t in range(T):
            for a, b in itertools.product(idx[t], idx[t]):
                ref[a, b] += 1
        assert np.array_equal(C, ref)
        assert np.array_equal(C, C.T)
        assert np.trace(C) == T * k
        assert C.sum() - np.trace(C) == T * k * (k - 1)
        assert np.array_equal(C.sum(1) - np.diag(C), (k - 1) * np.diag(C))
        C2 = orc.coactivation(idx, E, base=C)
        assert np.array_equal(C2, 2 * C)


def test_k2_closed_form_for_sfd_rows(orc):
    """For k = 2: S = 2T - sum of counts of pairs that share a device."""
    rng = np.random.default_rng(12)
    T, E, D = 200, 8, 4
    idx = _random_routing(rng, T, E, 2)
    C = orc.coactivation(idx, E)
    se = rng.permutation(E).astype(np.int32)
    b = orc.brim(idx, _f32(rng.random((T, 2))), se, E, D)
    intra, _ = orc.intra_share(C, se, D)
    assert b["S"] == 2 * T - intra


def _onehot(idx, E):
    oh = np.zeros((idx.shape[0], E), np.int64)
    for q in range(idx.shape[1]):
        oh[np.arange(idx.shape[0]), idx[:, q]] += 1
    return oh


def test_cross_layer_counts_are_a_one_hot_product(orc):
    rng = np.random.default_rng(40)
    for T, E1, k1, E2, k2 in [(50, 8, 2, 8, 2), (120, 16, 4, 12, 3), (64, 64, 8, 32, 6)]:
        idx1 = np.stack([rng.permutation(E1)[:k1] for _ in range(T)]).astype(np.int32)
        idx2 = np.stack([rng.permutation(E2)[:k2] for _ in range(T)]).astype(np.int32)
        A = orc.cross_coactivation(idx1, E1, idx2, E2)
        assert np.array_equal(A, _onehot(idx1, E1).T @ _onehot(idx2, E2))
        assert A.sum() == T * k1 * k2
    # one layer against itself is the plain co-activation
    assert np.array_equal(orc.cross_coactivation(idx1, E1, idx1, E1), orc.coactivation(idx1, E1))


def test_home_device_and_local_hits(orc):
    rng = np.random.default_rng(41)
    T, E1, k1, E2, k2, D = 200, 16, 4, 16, 3, 4
    L = E2 // D
    idx1 = np.stack([rng.permutation(E1)[:k1] for _ in range(T)]).astype(np.int32)
    idx2 = np.stack([rng.permutation(E2)[:k2] for _ in range(T)]).astype(np.int32)
    A = rng.integers(0, 50, size=(E1, E2)).astype(np.int32)
    A[3, :] = 7  # equal sums on every device for tokens that only see expert 3's row
    se2 = rng.permutation(E2).astype(np.int32)
    member = np.zeros((E2, D), np.int64)
    member[se2, np.arange(E2) // L] = 1
    scores = _onehot(idx1, E1) @ A.astype(np.int64) @ member
    home = orc.home_device(idx1, E1, A, se2, D)
    assert np.array_equal(home, np.argmax(scores, axis=1))  # argmax: first (lowest) on ties
    dev2 = np.empty(E2, np.int64)
    dev2[se2] = np.arange(E2) // L
    assert orc.local_hits(idx2, E2, se2, D, home) == int((dev2[idx2] == home[:, None]).sum())
    # the best possible home (knowing the next layer) serves at least as many
    best = np.argmax(_onehot(dev2[idx2], D), axis=1)
    assert orc.local_hits(idx2, E2, se2, D, best) >= orc.local_hits(idx2, E2, se2, D, home)


def test_planted_affinity_is_served_locally(orc):
    """Next-layer choice = a fixed permutation of this layer's (k = 1): the
    affinity is that permutation and every assignment lands on its home."""
    rng = np.random.default_rng(42)
    T, E, D = 300, 16, 4
    perm = rng.permutation(E).astype(np.int32)
    idx1 = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    idx2 = perm[idx1]
    A = orc.cross_coactivation(idx1, E, idx2, E)
    se2 = rng.permutation(E).astype(np.int32)
    home = orc.home_device(idx1, E, A, se2, D)
    assert orc.local_hits(idx2, E, se2, D, home) == T
    shard = (np.arange(T) * D // T).astype(np.int32)
    assert orc.local_hits(idx2, E, se2, D, shard) < T


def test_greedy_recovers_planted_blocks(orc):
    rng = np.random.default_rng(13)
    E, D = 32, 8
    L = E // D
    perm = rng.permutation(E)
    blocks = perm.reshape(D, L)
    C = rng.integers(0, 5, size=(E, E))
    C = C + C.T
    for blk in blocks:
        for a in blk:
            for b in blk:
                C[a, b] += 100
    np.fill_diagonal(C, rng.integers(200, 300, E))
    se = orc.greedy_placement(C.astype(np.int32), D)
    assert sorted(se.tolist()) == list(range(E))
    got = {frozenset(se[dv * L:(dv + 1) * L].tolist()) for dv in range(D)}
    assert got == {frozenset(b.tolist()) for b in blocks}
    assert np.array_equal(orc.greedy_placement(C.astype(np.int32), D), se)


# ---------------------------------------------------------------------------
# rounding and the input generator
# ---------------------------------------------------------------------------
def test_bf16_rounding_brute_force(orc):
    rng = np.random.default_rng(14)
    vals = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-30, 30, 300),
                           [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2.0 ** -130 * 1.5]])
    got = orc.round_dt(vals, "bf16")
    for v, g in zip(vals, got):
        f = np.float32(g)
        assert float(f) == g and (f.view(np.uint32) & 0xFFFF) == 0
        u = np.float32(v).view(np.uint32) & np.uint32(0xFFFF0000)
        lo = float(np.uint32(u).view(np.float32))
        step = float((np.uint32(u) + np.uint32(0x10000)).view(np.float32)) - lo
        hi = lo + step
        cands = sorted([lo, hi], key=lambda c: (abs(c - v),
                       (np.float32(c).view(np.uint32) >> 16) & 1))
        assert g == cands[0], (v, g, cands)


def test_generator_bf16_matches_torch_rounding():
    import torch
    v = np.random.default_rng(15).standard_normal(10000).astype(np.float32)
    ours = W.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generator_is_deterministic_and_keyed():
    cfg = W.CONFIGS["olmoe_bf16"]
    a = W.make_tokens(cfg, T=128)
    b = W.make_tokens(cfg, T=128)
    assert np.array_equal(a, b)
    c = W.make_tokens(cfg, T=128, token_seed=1)
    assert not np.array_equal(a, c)
    n = W.normal(0, "x", (3, 5))
    assert abs(W.normal(0, "x", (20000,)).std() - 1.0) < 0.03
    assert n.shape == (3, 5)
