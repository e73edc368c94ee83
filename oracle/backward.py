"""Backward pass of the collaboration-aware MoE layer -- part of the CPU
oracle, TEST INFRASTRUCTURE ONLY (same rules as the rest of ``oracle``).

Sources: Expert Coupling in MoE Pretraining, Abstract (every MoE layer runs
its all-to-alls in the forward and the backward pass); Occult, Figure 4
caption (the token states ORI, SFD, EPD and their moves guided by the BRIMs,
walked here in the opposite direction).  The chain rule of the forward
definition, in numpy fp64, with the layer dtype's rounding (``round_array``,
the oracle's own rounding) at the points where the layer stores a tensor:

  grad-combine   d_out_epd[r] = round(w[r] dy[t]),  dw[r] = <dy[t], out_epd[r]>
  experts        G, U = round(EPD W_g^T), round(EPD W_u^T)   (recomputed)
                 dh = d_out_epd W_d;  s = sigmoid(G)
                 dG = round(dh U s (1 + G (1 - s))),  dU = round(dh G s)
                 d_epd = round(dG W_g + dU W_u)
                 dW_g = dG^T EPD,  dW_u = dU^T EPD,  dW_d = d_out_epd^T h
  grad-dispatch  d_sfd[s] = round(sum over the SFD row's EPD rows of d_epd)
                 dx[t] = round(dx_router[t] + dx_shared[t] + sum over its SFD rows
                 of d_sfd)
  shared experts G, U = round(X W_g^T), round(X W_u^T); dh = dY W_d (weight 1);
                 dG, dU as above; dx_shared = round(sum over them of dG W_g + dU W_u);
                 dW_g = dG^T X, dW_u = dU^T X, dW_d = dY^T h
  router         dp from dw (through the renormalisation), then
                 dlogit = p (dp - <p, dp>);  dx_router = dlogit W_r,
                 dW_r = dlogit^T X
Top-k selection is a constant of the backward.  dtype "f64" skips every
rounding (used by the finite-difference pins).  Under collaboration pruning
the BRIMs hold only the kept picks with their stored (rescaled) weights: the
expert part is the exact gradient of that layer, and in the routing gradient
a kept pick carries its stored weight's gradient and a dropped one none (the
pruning decision is held constant and the rescaling factor is ignored: the
exact derivative of the layer whose kept weights are the routing weights
plus constants equal to the rescaling's change at the evaluation point).
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import DT, _p, lib

ROUND = {"f32": 0, "bf16": 1, "f64": 2}


def round_array(a, dtype):
    """The oracle's rounding (ties to even) of every element; "f64": none."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty_like(a)
    f = lib().orc_round_array
    f.argtypes = [C.c_long, C.c_int, C.c_void_p, C.c_void_p]
    rc = f(a.size, ROUND[dtype], a.ctypes.data, out.ctypes.data)
    assert rc == 0
    return out


def _f64(a, dtype):
    """Stored tensor (float32 holding dtype values, or bf16 bits) as fp64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def expert_rows(x, wgu, wdn, b, slot_expert, dy, rows, dtype):
    """Forward and backward of the EPD rows ``rows`` (any subset).  Returns
    per-row arrays (in the order of ``rows``): a, bu (fp64 pre-activations),
    h, out_epd, d_out_epd, dw, G, U, dG, dU, d_epd."""
    rows = np.asarray(rows, dtype=np.int64)
    I = wgu.shape[1] // 2
    so = b["slot_offset"]
    slot = np.searchsorted(so, rows, side="right") - 1
    ex = np.asarray(slot_expert)[slot]
    tok = b["epd_token"][rows]
    A = _f64(x, dtype)[tok]                       # EPD rows
    W = _f64(wgu, dtype)
    Wd = _f64(wdn, dtype)
    n, d = A.shape
    res = {k: np.empty((n, m)) for k, m in [("a", I), ("bu", I), ("h", I), ("out_epd", d),
                                            ("d_out_epd", d), ("G", I), ("U", I), ("dG", I),
                                            ("dU", I), ("d_epd", d)]}
    res["dw"] = np.empty(n)
    w = b["epd_w"][rows].astype(np.float64)
    g_dy = _f64(dy, dtype)[tok]
    for e in np.unique(ex):
        q = np.nonzero(ex == e)[0]
        Ae = A[q]
        a = Ae @ W[e, :I].T
        bu = Ae @ W[e, I:].T
        h = round_array(_silu(a) * bu, dtype)
        out = round_array(h @ Wd[e].T, dtype)
        dout = round_array(w[q, None] * g_dy[q], dtype)
        dw = np.sum(g_dy[q] * out, axis=1)
        G = round_array(a, dtype)
        U = round_array(bu, dtype)
        dh = dout @ Wd[e]
        s = 1.0 / (1.0 + np.exp(-G))
        dG = round_array(dh * U * s * (1.0 + G * (1.0 - s)), dtype)
        dU = round_array(dh * G * s, dtype)
        d_epd = round_array(dG @ W[e, :I] + dU @ W[e, I:], dtype)
        for k_, v in [("a", a), ("bu", bu), ("h", h), ("out_epd", out), ("d_out_epd", dout),
                      ("G", G), ("U", U), ("dG", dG), ("dU", dU), ("d_epd", d_epd)]:
            res[k_][q] = v
        res["dw"][q] = dw
    return res


def slot_weight_grads(x, wgu, wdn, b, slot_expert, dy, g, dtype):
    """Weight gradients of the expert of slot g: (dW_gate_up [2I][d], dW_down [d][I])."""
    so = b["slot_offset"]
    rows = np.arange(so[g], so[g + 1])
    I = wgu.shape[1] // 2
    d = wgu.shape[2]
    if rows.size == 0:
        return np.zeros((2 * I, d)), np.zeros((d, I))
    r = expert_rows(x, wgu, wdn, b, slot_expert, dy, rows, dtype)
    A = _f64(x, dtype)[b["epd_token"][rows]]
    dWgu = np.concatenate([r["dG"].T @ A, r["dU"].T @ A], axis=0)
    dWd = r["d_out_epd"].T @ r["h"]
    return dWgu, dWd


def shared_backward(x, wgu_sh, wdn_sh, dy, tokens, dtype):
    """Backward of the shared experts (always active, weight 1, on the ORI
    rows; their outputs enter Y unweighted) for the ORI rows ``tokens``.
    Per shared expert s, with the forward's pre-activations a = X Wg^T and
    b = X Wu^T (fp64) and its stored h = round(silu(a) b):
        G, U  = round(a), round(b)              (recomputed, stored)
        dh    = dY Wd[s]                         (the shared output's gradient is dY)
        dG    = round(dh U silu'(G)),  dU = round(dh G sigmoid(G))
        dW_gate_up_sh[s] = [dG | dU]^T X,  dW_down_sh[s] = dY^T h
    and dx_shared = round(sum over s of dG Wg[s] + dU Wu[s]).  Returns
    dx_shared [n][d], the per-expert G, U, dG, dU, h ([n_sh][n][I_sh]) and the
    weight gradients summed over the given rows (the exact ones when tokens
    covers every row)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    X = _f64(x, dtype)[tokens]
    Wgu = _f64(wgu_sh, dtype)
    Wd = _f64(wdn_sh, dtype)
    n_sh, two_i, d = Wgu.shape
    Is = two_i // 2
    g_dy = _f64(dy, dtype)[tokens]
    out = {k_: np.empty((n_sh, len(tokens), Is)) for k_ in ("G", "U", "dG", "dU", "h")}
    dxs = np.zeros((len(tokens), d))
    dWgu = np.zeros((n_sh, two_i, d))
    dWd = np.zeros((n_sh, d, Is))
    for sg in range(n_sh):
        a = X @ Wgu[sg, :Is].T
        bu = X @ Wgu[sg, Is:].T
        h = round_array(_silu(a) * bu, dtype)
        G = round_array(a, dtype)
        U = round_array(bu, dtype)
        dh = g_dy @ Wd[sg]
        sig = 1.0 / (1.0 + np.exp(-G))
        dG = round_array(dh * U * sig * (1.0 + G * (1.0 - sig)), dtype)
        dU = round_array(dh * G * sig, dtype)
        dxs += dG @ Wgu[sg, :Is] + dU @ Wgu[sg, Is:]
        dWgu[sg] = np.concatenate([dG.T @ X, dU.T @ X], axis=0)
        dWd[sg] = g_dy.T @ h
        for k_, v in (("G", G), ("U", U), ("dG", dG), ("dU", dU), ("h", h)):
            out[k_][sg] = v
    out.update(dx_shared=round_array(dxs, dtype), dW_gate_up_sh=dWgu, dW_down_sh=dWd)
    return out


def shared_weight_grad_columns(x, wgu_sh, wdn_sh, dy, s, cols, dtype):
    """The shared expert s's weight gradients at the intermediate columns
    ``cols`` (every ORI row): the gate rows dW_gate_up_sh[s][cols], the up
    rows dW_gate_up_sh[s][I_sh + cols] and the columns dW_down_sh[s][:, cols].
    Each intermediate column's G, U, dh, dG, dU and h depend on that column
    alone, so this is shared_backward's formula restricted to those columns.
    Returns (gate rows [n][d], up rows [n][d], down columns [d][n])."""
    cols = np.asarray(cols, dtype=np.int64)
    X = _f64(x, dtype)
    Wgu = _f64(wgu_sh, dtype)[s]
    Wd = _f64(wdn_sh, dtype)[s]
    Is = Wgu.shape[0] // 2
    g_dy = _f64(dy, dtype)
    a = X @ Wgu[cols].T
    bu = X @ Wgu[Is + cols].T
    h = round_array(_silu(a) * bu, dtype)
    G = round_array(a, dtype)
    U = round_array(bu, dtype)
    dh = g_dy @ Wd[:, cols]
    sig = 1.0 / (1.0 + np.exp(-G))
    dG = round_array(dh * U * sig * (1.0 + G * (1.0 - sig)), dtype)
    dU = round_array(dh * G * sig, dtype)
    return dG.T @ X, dU.T @ X, g_dy.T @ h


def grad_dispatch(b, d_epd_of, tokens, T, D, L, d, dtype, dx_router=None, dx_shared=None):
    """d_sfd for the tokens' SFD rows and dx for the tokens; d_epd_of maps an
    EPD row to its d_epd (fp64 [d]); dx_router (fp32) and dx_shared (the
    shared experts' stored input gradient) are rows of the tokens, added into
    dx with the SFD rows.  Returns (dx [n][d], {s: d_sfd[s]})."""
    dx = np.zeros((len(tokens), d))
    dsfd = {}
    for q, t in enumerate(tokens):
        acc_t = np.zeros(d) if dx_router is None else np.array(dx_router[q], dtype=np.float64)
        if dx_shared is not None:
            acc_t = acc_t + np.asarray(dx_shared[q], dtype=np.float64)
        for dv in range(D):
            s = b["brim0"][dv, t]
            if s < 0:
                continue
            acc = np.zeros(d)
            for l in range(L):
                r = b["brim1"][l, s]
                if r >= 0:
                    acc += d_epd_of(r)
            v = round_array(acc, dtype)
            dsfd[int(s)] = v
            acc_t += v
        dx[q] = round_array(acc_t, dtype)
    return dx, dsfd


def router_grads(logits, idx, w, renorm, dw_of, tokens):
    """dlogits for the tokens (fp64 [n][E]); dw_of(t, j) is the gradient of
    the weight of the token's pick j."""
    lg = np.asarray(logits, np.float64)[tokens]
    k = idx.shape[1]
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    out = np.empty_like(p)
    for q, t in enumerate(tokens):
        e = idx[t]
        g = np.array([dw_of(t, j) for j in range(k)])
        if renorm:
            P = p[q, e].sum()
            ww = p[q, e] / P
            dpj = (g - np.dot(g, ww)) / P
        else:
            dpj = g
        dp = np.zeros(p.shape[1])
        dp[e] = dpj
        out[q] = p[q] * (dp - np.dot(p[q], dp))
    return out


def full(x, wr, wgu, wdn, logits, idx, w, renorm, b, slot_expert, dy, D, dtype, shared=None):
    """The whole backward for every token and expert (small layers).
    shared: (w_gate_up_sh, w_down_sh) of the shared experts, or None.
    Returns dict: d_out_epd, dw, dG, dU, G, U, d_epd (per EPD row), dW_gate_up
    [E][2I][d], dW_down [E][d][I], dlogits [T][E], dx_router [T][d],
    dW_router [E][d], d_sfd {s: row}, dx [T][d]; with shared experts also
    dx_shared [T][d], dW_gate_up_sh, dW_down_sh and their G, U, dG, dU, h."""
    T, k = idx.shape
    E = wgu.shape[0]
    d = x.shape[1]
    L = E // D
    R = int(b["slot_offset"][E])
    rows = np.arange(R)
    r = expert_rows(x, wgu, wdn, b, slot_expert, dy, rows, dtype)
    dWgu = np.zeros((E, wgu.shape[1], d))
    dWd = np.zeros((E, d, wgu.shape[1] // 2))
    A = _f64(x, dtype)[b["epd_token"]]
    so = b["slot_offset"]
    for g in range(E):
        e = slot_expert[g]
        q = np.arange(so[g], so[g + 1])
        dWgu[e] = np.concatenate([r["dG"][q].T @ A[q], r["dU"][q].T @ A[q]], axis=0)
        dWd[e] = r["d_out_epd"][q].T @ r["h"][q]
    # the EPD row of each (token, pick)
    slot_of = np.empty(E, np.int64)
    slot_of[np.asarray(slot_expert)] = np.arange(E)

    def row_of(t, j):
        # -1 when the pick has no EPD row (dropped by collaboration pruning)
        gsl = slot_of[idx[t, j]]
        s = b["brim0"][gsl // L, t]
        return b["brim1"][gsl % L, s] if s >= 0 else -1

    def dw_of(t, j):
        # a dropped pick's weight gets no gradient; a kept pick's is that of
        # its stored (possibly rescaled) weight
        rr = row_of(t, j)
        return r["dw"][rr] if rr >= 0 else 0.0

    tokens = np.arange(T)
    dl = router_grads(logits, idx, w, renorm, dw_of, tokens)
    X = _f64(x, dtype)
    dxr = dl @ np.asarray(wr, np.float64)
    dWr = dl.T @ X
    sh = None
    if shared is not None:
        sh = shared_backward(x, shared[0], shared[1], dy, tokens, dtype)
    dx, dsfd = grad_dispatch(b, lambda rr: r["d_epd"][rr], tokens, T, D, L, d, dtype, dxr,
                             None if sh is None else sh["dx_shared"])
    out = {k_: r[k_] for k_ in ("d_out_epd", "dw", "dG", "dU", "G", "U", "d_epd", "out_epd", "h")}
    out.update(dW_gate_up=dWgu, dW_down=dWd, dlogits=dl, dx_router=dxr, dW_router=dWr,
               d_sfd=dsfd, dx=dx)
    if sh is not None:
        out.update({k_ + "_sh": sh[k_] for k_ in ("G", "U", "dG", "dU", "h")})
        out.update(dx_shared=sh["dx_shared"], dW_gate_up_sh=sh["dW_gate_up_sh"],
                   dW_down_sh=sh["dW_down_sh"])
    return out
