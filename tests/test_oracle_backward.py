"""Pins of the backward oracle (oracle/backward.py) on the CPU.

The gradients through the BRIMs (fp64, no rounding) are checked against
central finite differences of the standard layer written plainly (no SFD,
no EPD, selections held fixed), and that plain forward against the C
oracle's forward.  A structural pin: with renormalised weights, a dy that
gives every expert output the same value has zero routing gradient.
"""
import numpy as np
import pytest

import workloads as W
from tests.tolerance import rel_err


def _ob():
    import oracle.backward as ob
    return ob


def _layer(seed=0, renorm=0, T=24, d=16, E=8, I=12, k=3, D=2):
    cfg = W.LayerConfig("bwd_tiny", T=T, d=d, E=E, I=I, k=k, D=D, dtype="f32", renorm=renorm,
                        clusters=3)
    return cfg, W.make_layer(cfg, seed=seed)


def fwd64(x, wr, wgu, wdn, idx, renorm):
    """The standard MoE layer in fp64 with the selections idx held fixed:
    y[t] = sum_j w_j FFN_{idx[t][j]}(x_t), w = softmax over all experts."""
    lg = x @ wr.T
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    T, k = idx.shape
    I = wgu.shape[1] // 2
    y = np.zeros_like(x)
    for t in range(T):
        wsel = p[t, idx[t]]
        if renorm:
            wsel = wsel / wsel.sum()
        for j in range(k):
            e = idx[t, j]
            a = wgu[e, :I] @ x[t]
            u = wgu[e, I:] @ x[t]
            h = a / (1.0 + np.exp(-a)) * u
            y[t] += wsel[j] * (wdn[e] @ h)
    return y


@pytest.mark.parametrize("renorm", [0, 1])
def test_gradients_match_finite_differences(orc, renorm):
    ob = _ob()
    cfg, inp = _layer(renorm=renorm)
    x, wr, wgu, wdn = (np.asarray(a, np.float64) for a in (inp.x, inp.w_router, inp.w_gate_up,
                                                           inp.w_down))
    lg, idx, w = orc.route(inp.x, inp.w_router, cfg.k, renorm, "f32")
    b = orc.brim(idx, w, inp.slot_expert, cfg.E, cfg.D)
    # the plain fp64 forward agrees with the C oracle's layer (fp32 storage)
    y_c = orc.layer(inp)["y"]
    y64 = fwd64(x, wr, wgu, wdn, idx, renorm)
    assert rel_err(y_c, y64) <= 1e-5
    rng = np.random.default_rng(3)
    dy = rng.standard_normal(y64.shape)
    g = ob.full(x, wr, wgu, wdn, lg, idx, w, renorm, b, inp.slot_expert, dy, cfg.D, "f64")

    def loss(x_, wr_, wgu_, wdn_):
        return float(np.sum(dy * fwd64(x_, wr_, wgu_, wdn_, idx, renorm)))

    eps = 1e-6
    for name, arr, grad in [("x", x, g["dx"]), ("w_router", wr, g["dW_router"]),
                            ("w_gate_up", wgu, g["dW_gate_up"]), ("w_down", wdn, g["dW_down"])]:
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            if name == "w_gate_up" or name == "w_down":
                pos = (int(idx[rng.integers(0, cfg.T), 0]),) + pos[1:]  # a used expert
            args = {"x": x, "w_router": wr, "w_gate_up": wgu, "w_down": wdn}
            plus = {k_: v.copy() for k_, v in args.items()}
            minus = {k_: v.copy() for k_, v in args.items()}
            plus[name][pos] += eps
            minus[name][pos] -= eps
            fd = (loss(plus["x"], plus["w_router"], plus["w_gate_up"], plus["w_down"]) -
                  loss(minus["x"], minus["w_router"], minus["w_gate_up"], minus["w_down"])) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def test_renormalised_routing_gradient_cancels(orc):
    """With renormalised weights and identical expert outputs along dy, the
    weights' gradients are equal within a token, so dp and dlogits vanish."""
    ob = _ob()
    cfg, inp = _layer(renorm=1, seed=2)
    lg, idx, w = orc.route(inp.x, inp.w_router, cfg.k, 1, "f32")
    dw_equal = lambda t, j: 0.37 * (t + 1)  # same for every pick of a token
    dl = ob.router_grads(lg, idx, w, 1, dw_equal, np.arange(cfg.T))
    assert np.abs(dl).max() <= 1e-12
    # without renormalisation the same dw moves the logits
    dl0 = ob.router_grads(lg, idx, w, 0, dw_equal, np.arange(cfg.T))
    assert np.abs(dl0).max() > 1e-3


def test_rounded_backward_stays_close_to_exact(orc):
    """bf16 rounding at the storage points changes the gradients by about
    the bf16 precision (median), and by a few per cent where a sum cancels
    (dh = d_out W_down of rounded inputs feeds dG, dU and the weight
    gradients)."""
    ob = _ob()
    cfg = W.LayerConfig("bwd_b", T=40, d=64, E=8, I=64, k=2, D=2, dtype="bf16", clusters=3)
    inp = W.make_layer(cfg, seed=1)
    lg, idx, w = orc.route(inp.x, inp.w_router, cfg.k, 0, "bf16")
    b = orc.brim(idx, w, inp.slot_expert, cfg.E, cfg.D)
    dy = W.to_f32(W.from_f64(np.random.default_rng(4).standard_normal((cfg.T, cfg.d)), "bf16"),
                  "bf16")
    args = (W.to_f32(inp.x, "bf16"), W.to_f32(inp.w_router, "bf16"),
            W.to_f32(inp.w_gate_up, "bf16"), W.to_f32(inp.w_down, "bf16"))
    g16 = ob.full(*args, lg, idx, w, 0, b, inp.slot_expert, dy, cfg.D, "bf16")
    g64 = ob.full(*args, lg, idx, w, 0, b, inp.slot_expert, dy, cfg.D, "f64")
    for name in ("dx", "dW_gate_up", "dW_down", "dW_router"):
        o = g64[name]
        rel = np.abs(g16[name] - o) / np.maximum(np.abs(o), np.sqrt(np.mean(o * o)))
        assert np.median(rel) <= 2e-3 and rel.max() <= 6e-2, (name, np.median(rel), rel.max())


def fwd_kept64(x, wgu, wdn, idx, w):
    """The layer with fixed picks and fixed weights (no router): y[t] = sum
    over the picks j with idx >= 0 of w[t][j] FFN_{idx[t][j]}(x_t)."""
    T, k = idx.shape
    I = wgu.shape[1] // 2
    y = np.zeros_like(x)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if e < 0:
                continue
            a = wgu[e, :I] @ x[t]
            u = wgu[e, I:] @ x[t]
            y[t] += w[t, j] * (wdn[e] @ (a / (1.0 + np.exp(-a)) * u))
    return y


@pytest.mark.parametrize("rescale", [0, 1])
def test_pruned_expert_gradients_match_finite_differences(orc, rescale):
    """Collaboration pruning (budget 1 of 2 devices): the BRIMs of the kept
    picks with their stored weights give the exact weight gradients of the
    layer those picks and weights define, and dropped picks get no routing
    weight gradient."""
    ob = _ob()
    cfg, inp = _layer(seed=5, k=4, E=8, D=2)
    x, wr, wgu, wdn = (np.asarray(a, np.float64) for a in (inp.x, inp.w_router, inp.w_gate_up,
                                                           inp.w_down))
    lg, idx, w = orc.route(inp.x, inp.w_router, cfg.k, 0, "f32")
    ik, wk = orc.prune(idx, w, inp.slot_expert, cfg.E, cfg.D, 1, rescale)
    assert np.any(ik < 0)  # something was dropped
    b = orc.brim(ik, wk, inp.slot_expert, cfg.E, cfg.D)
    rng = np.random.default_rng(6)
    dy = rng.standard_normal(x.shape)
    g = ob.full(x, wr, wgu, wdn, lg, idx, w, 0, b, inp.slot_expert, dy, cfg.D, "f64")
    wk64 = wk.astype(np.float64)

    def loss(wgu_, wdn_):
        return float(np.sum(dy * fwd_kept64(x, wgu_, wdn_, ik, wk64)))

    eps = 1e-6
    for name, arr, grad in [("w_gate_up", wgu, g["dW_gate_up"]), ("w_down", wdn, g["dW_down"])]:
        for _ in range(6):
            t0 = rng.integers(0, cfg.T)
            j0 = int(np.flatnonzero(ik[t0] >= 0)[0])
            pos = (int(ik[t0, j0]),) + tuple(rng.integers(0, s) for s in arr.shape[1:])
            plus, minus = wgu.copy(), wgu.copy()
            if name == "w_down":
                plus, minus = wdn.copy(), wdn.copy()
            plus[pos] += eps
            minus[pos] -= eps
            fd = ((loss(plus, wdn) - loss(minus, wdn)) if name == "w_gate_up" else
                  (loss(wgu, plus) - loss(wgu, minus))) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])
    # routing: dropped picks carry no weight gradient
    dw_zero_dropped = lambda t, j: 0.0 if ik[t, j] < 0 else 1.0  # noqa: E731
    dl = ob.router_grads(lg, idx, w, 0, dw_zero_dropped, np.arange(cfg.T))
    full_pick = lambda t, j: 1.0  # noqa: E731
    dl_all = ob.router_grads(lg, idx, w, 0, full_pick, np.arange(cfg.T))
    dropped_tokens = np.flatnonzero(np.any(ik < 0, axis=1))
    assert not np.allclose(dl[dropped_tokens], dl_all[dropped_tokens])


@pytest.mark.parametrize("renorm", [0, 1])
def test_pruned_routing_gradient_matches_finite_differences(orc, renorm):
    """Collaboration pruning without rescaling (budget 1 of 2 devices): a
    kept pick's weight is its routing weight, a dropped pick contributes
    nothing, so with the picks and the pruning decision held fixed the
    routing gradient through the pruned BRIMs is the exact derivative of
    that layer: dW_router and dx against central finite differences of the
    plain forward over the kept picks (with renormalisation the weights are
    still normalised over all k picks, dropped ones included)."""
    ob = _ob()
    cfg, inp = _layer(seed=7, renorm=renorm, k=4, E=8, D=2)
    x, wr, wgu, wdn = (np.asarray(a, np.float64) for a in (inp.x, inp.w_router, inp.w_gate_up,
                                                           inp.w_down))
    lg, idx, w = orc.route(inp.x, inp.w_router, cfg.k, renorm, "f32")
    ik, wk = orc.prune(idx, w, inp.slot_expert, cfg.E, cfg.D, 1, 0)
    assert np.any(ik < 0) and np.all((ik < 0) | (ik == idx))
    b = orc.brim(ik, wk, inp.slot_expert, cfg.E, cfg.D)
    rng = np.random.default_rng(8)
    dy = rng.standard_normal(x.shape)
    g = ob.full(x, wr, wgu, wdn, lg, idx, w, renorm, b, inp.slot_expert, dy, cfg.D, "f64")

    def kept_weights(x_, wr_):
        lg_ = x_ @ wr_.T
        p = np.exp(lg_ - lg_.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ws = np.take_along_axis(p, idx, axis=1)
        if renorm:
            ws = ws / ws.sum(axis=1, keepdims=True)
        return np.where(ik >= 0, ws, 0.0)

    # the weights at the base point are the oracle's stored ones
    assert np.allclose(kept_weights(x, wr), np.where(ik >= 0, wk, 0.0), rtol=1e-5, atol=1e-7)

    def loss(x_, wr_):
        return float(np.sum(dy * fwd_kept64(x_, wgu, wdn, ik, kept_weights(x_, wr_))))

    eps = 1e-6
    for name, arr, grad in [("w_router", wr, g["dW_router"]), ("x", x, g["dx"])]:
        for _ in range(8):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            if name == "x":  # a token that lost a device
                pos = (int(rng.choice(np.flatnonzero(np.any(ik < 0, axis=1)))), pos[1])
            plus, minus = arr.copy(), arr.copy()
            plus[pos] += eps
            minus[pos] -= eps
            if name == "w_router":
                fd = (loss(x, plus) - loss(x, minus)) / (2 * eps)
            else:
                fd = (loss(plus, wr) - loss(minus, wr)) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])



@pytest.mark.parametrize("renorm", [0, 1])
def test_rescaled_pruned_routing_gradient_matches_finite_differences(orc, renorm):
    """Collaboration pruning with rescaling (budget 1 of 2 devices): the
    routing gradient passes each kept pick's stored-weight gradient through
    the softmax backward unchanged (the rescaling factor is ignored there).
    That is the exact derivative of the layer whose kept weights are the
    routing weights plus constants that make them equal the stored rescaled
    weights at the base point: dW_router and dx against central finite
    differences of that layer (the expert part uses the stored weights)."""
    ob = _ob()
    cfg, inp = _layer(seed=7, renorm=renorm, k=4, E=8, D=2)
    x, wr, wgu, wdn = (np.asarray(a, np.float64) for a in (inp.x, inp.w_router, inp.w_gate_up,
                                                           inp.w_down))
    lg, idx, w = orc.route(inp.x, inp.w_router, cfg.k, renorm, "f32")
    ik, wk = orc.prune(idx, w, inp.slot_expert, cfg.E, cfg.D, 1, 1)
    assert np.any(ik < 0) and np.all((ik < 0) | (ik == idx))
    b = orc.brim(ik, wk, inp.slot_expert, cfg.E, cfg.D)
    rng = np.random.default_rng(9)
    dy = rng.standard_normal(x.shape)
    g = ob.full(x, wr, wgu, wdn, lg, idx, w, renorm, b, inp.slot_expert, dy, cfg.D, "f64")

    def routing_weights(x_, wr_):
        lg_ = x_ @ wr_.T
        p = np.exp(lg_ - lg_.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ws = np.take_along_axis(p, idx, axis=1)
        if renorm:
            ws = ws / ws.sum(axis=1, keepdims=True)
        return np.where(ik >= 0, ws, 0.0)

    # the constants: stored (rescaled) weight minus routing weight at the base
    shift = np.where(ik >= 0, np.asarray(wk, np.float64), 0.0) - routing_weights(x, wr)
    assert np.abs(shift).max() > 1e-3  # rescaling moved the kept weights

    def loss(x_, wr_):
        return float(np.sum(dy * fwd_kept64(x_, wgu, wdn, ik, routing_weights(x_, wr_) + shift)))

    eps = 1e-6
    for name, arr, grad in [("w_router", wr, g["dW_router"]), ("x", x, g["dx"])]:
        for _ in range(8):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            if name == "x":  # a token that lost a device
                pos = (int(rng.choice(np.flatnonzero(np.any(ik < 0, axis=1)))), pos[1])
            plus, minus = arr.copy(), arr.copy()
            plus[pos] += eps
            minus[pos] -= eps
            if name == "w_router":
                fd = (loss(x, plus) - loss(x, minus)) / (2 * eps)
            else:
                fd = (loss(plus, wr) - loss(minus, wr)) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])

def test_slot_weight_grads_pinned(orc):
    """slot_weight_grads (the reference for the weight gradients of sampled
    slots at full size) under a non-identity placement: for every slot it
    equals the slice of full() for the slot's expert, and for two slots it
    matches central finite differences of the plain fp64 layer in the
    weights of that slot's expert (a slot/expert mix-up, a wrong row set or
    a transposed product fails here)."""
    ob = _ob()
    cfg, inp = _layer(seed=7, T=40, d=16, E=8, I=12, k=3, D=4)
    se = np.array([5, 2, 7, 0, 3, 6, 1, 4], dtype=np.int32)
    x, wr, wgu, wdn = (np.asarray(a, np.float64) for a in (inp.x, inp.w_router, inp.w_gate_up,
                                                           inp.w_down))
    lg, idx, w = orc.route(inp.x, inp.w_router, cfg.k, 0, "f32")
    b = orc.brim(idx, w, se, cfg.E, cfg.D)
    rng = np.random.default_rng(8)
    dy = rng.standard_normal(x.shape)
    g = ob.full(x, wr, wgu, wdn, lg, idx, w, 0, b, se, dy, cfg.D, "f64")
    counts = np.diff(b["slot_offset"])
    for slot in range(cfg.E):
        dgu, ddn = ob.slot_weight_grads(x, wgu, wdn, b, se, dy, slot, "f64")
        e = se[slot]
        assert np.allclose(dgu, g["dW_gate_up"][e], rtol=1e-12, atol=1e-12), slot
        assert np.allclose(ddn, g["dW_down"][e], rtol=1e-12, atol=1e-12), slot
        if counts[slot] == 0:
            assert not dgu.any() and not ddn.any()

    def loss(wgu_, wdn_):
        return float(np.sum(dy * fwd64(x, wr, wgu_, wdn_, idx, 0)))

    eps = 1e-6
    busy = [int(s) for s in np.argsort(-counts, kind="stable")[:2]]
    for slot in busy:
        dgu, ddn = ob.slot_weight_grads(x, wgu, wdn, b, se, dy, slot, "f64")
        e = int(se[slot])
        for _ in range(5):
            # a gate row, an up row, and a down entry of this slot's expert
            for name, arr, grad in [("w_gate_up", wgu, dgu), ("w_down", wdn, ddn)]:
                pos = tuple(int(rng.integers(0, s)) for s in arr.shape[1:])
                plus, minus = arr.copy(), arr.copy()
                plus[(e,) + pos] += eps
                minus[(e,) + pos] -= eps
                if name == "w_gate_up":
                    fd = (loss(plus, wdn) - loss(minus, wdn)) / (2 * eps)
                else:
                    fd = (loss(wgu, plus) - loss(wgu, minus)) / (2 * eps)
                assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (slot, name, pos, fd,
                                                                          grad[pos])


def shared64(x, wgu_sh, wdn_sh):
    """The shared experts' output in fp64: sum over them of W_d (silu(W_g x) * W_u x)."""
    Is = wgu_sh.shape[1] // 2
    y = np.zeros_like(x)
    for sg in range(wgu_sh.shape[0]):
        a = x @ wgu_sh[sg, :Is].T
        u = x @ wgu_sh[sg, Is:].T
        y += (a / (1.0 + np.exp(-a)) * u) @ wdn_sh[sg].T
    return y


def test_shared_expert_gradients_match_finite_differences(orc):
    """A layer with two shared experts (weight 1, on every token): the
    input gradient (routed, router and shared paths together) and the
    shared experts' weight gradients against central finite differences of
    the plain fp64 layer with the selections held fixed."""
    ob = _ob()
    cfg = W.LayerConfig("bwd_shared", T=20, d=16, E=8, I=12, k=2, D=2, dtype="f32",
                        n_shared=2, I_shared=8, clusters=3)
    inp = W.make_layer(cfg, seed=9)
    x, wr, wgu, wdn, wgs, wds = (np.asarray(a, np.float64) for a in (
        inp.x, inp.w_router, inp.w_gate_up, inp.w_down, inp.w_gate_up_sh, inp.w_down_sh))
    lg, idx, w = orc.route(inp.x, inp.w_router, cfg.k, 0, "f32")
    b = orc.brim(idx, w, inp.slot_expert, cfg.E, cfg.D)
    # the plain fp64 forward with shared experts agrees with the C oracle's layer
    y_c = orc.layer(inp)["y"]
    assert rel_err(y_c, fwd64(x, wr, wgu, wdn, idx, 0) + shared64(x, wgs, wds)) <= 1e-5
    rng = np.random.default_rng(10)
    dy = rng.standard_normal(x.shape)
    g = ob.full(x, wr, wgu, wdn, lg, idx, w, 0, b, inp.slot_expert, dy, cfg.D, "f64",
                shared=(wgs, wds))

    def loss(x_, wgs_, wds_):
        return float(np.sum(dy * (fwd64(x_, wr, wgu, wdn, idx, 0) + shared64(x_, wgs_, wds_))))

    eps = 1e-6
    for name, arr, grad in [("x", x, g["dx"]), ("w_gate_up_sh", wgs, g["dW_gate_up_sh"]),
                            ("w_down_sh", wds, g["dW_down_sh"])]:
        for _ in range(8):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            args = {"x": x, "w_gate_up_sh": wgs, "w_down_sh": wds}
            plus = {k_: v.copy() for k_, v in args.items()}
            minus = {k_: v.copy() for k_, v in args.items()}
            plus[name][pos] += eps
            minus[name][pos] -= eps
            fd = (loss(plus["x"], plus["w_gate_up_sh"], plus["w_down_sh"]) -
                  loss(minus["x"], minus["w_gate_up_sh"], minus["w_down_sh"])) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def test_two_shared_experts_backward_equal_one_concatenated(orc):
    """Two shared SwiGLU experts are one with their intermediate rows
    concatenated (an exact identity of the forward); so are their gradients:
    the concatenated expert's weight gradients are the two experts' side by
    side, and the input gradients agree (rounded, bf16)."""
    ob = _ob()
    rng = np.random.default_rng(11)
    T, d, Is = 24, 32, 16
    x = W.from_f64(rng.standard_normal((T, d)), "bf16")
    wgs = W.from_f64(rng.standard_normal((2, 2 * Is, d)) / np.sqrt(d), "bf16")
    wds = W.from_f64(rng.standard_normal((2, d, Is)) / np.sqrt(d), "bf16")
    dy = W.from_f64(rng.standard_normal((T, d)), "bf16")
    tok = np.arange(T)
    two = ob.shared_backward(x, wgs, wds, dy, tok, "bf16")
    # one expert of intermediate 2 Is: gate rows of both, then up rows of both
    wg1 = np.concatenate([wgs[0, :Is], wgs[1, :Is], wgs[0, Is:], wgs[1, Is:]], axis=0)[None]
    wd1 = np.concatenate([wds[0], wds[1]], axis=1)[None]
    one = ob.shared_backward(x, wg1, wd1, dy, tok, "bf16")
    dWg = one["dW_gate_up_sh"][0]
    same = lambda u, v: np.allclose(u, v, rtol=1e-12, atol=1e-12)  # noqa: E731
    assert same(dWg[:Is], two["dW_gate_up_sh"][0, :Is])
    assert same(dWg[Is:2 * Is], two["dW_gate_up_sh"][1, :Is])
    assert same(dWg[2 * Is:3 * Is], two["dW_gate_up_sh"][0, Is:])
    assert same(dWg[3 * Is:], two["dW_gate_up_sh"][1, Is:])
    assert same(one["dW_down_sh"][0], np.concatenate([two["dW_down_sh"][0],
                                                      two["dW_down_sh"][1]], axis=1))
    # the input gradient is one rounded sum either way (summation order only)
    assert rel_err(one["dx_shared"], two["dx_shared"]) <= 1e-2


def test_shared_weight_grad_columns_are_slices_of_the_full_gradient():
    """The column-restricted shared weight gradients (the reference for
    full-size layers) equal the slices of shared_backward's full result."""
    ob = _ob()
    rng = np.random.default_rng(12)
    T, d, Is = 40, 32, 24
    x = W.from_f64(rng.standard_normal((T, d)), "bf16")
    wgs = W.from_f64(rng.standard_normal((2, 2 * Is, d)) / np.sqrt(d), "bf16")
    wds = W.from_f64(rng.standard_normal((2, d, Is)) / np.sqrt(d), "bf16")
    dy = W.from_f64(rng.standard_normal((T, d)), "bf16")
    full = ob.shared_backward(x, wgs, wds, dy, np.arange(T), "bf16")
    for s in range(2):
        cols = np.array([0, 5, Is - 1])
        gr, ur, dc = ob.shared_weight_grad_columns(x, wgs, wds, dy, s, cols, "bf16")
        same = lambda u, v: np.allclose(u, v, rtol=1e-12, atol=1e-12)  # noqa: E731
        assert same(gr, full["dW_gate_up_sh"][s][cols])
        assert same(ur, full["dW_gate_up_sh"][s][Is + cols])
        assert same(dc, full["dW_down_sh"][s][:, cols])
