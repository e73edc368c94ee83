"""GPU parity of the backward pass through the BRIMs against the backward
oracle (oracle/backward.py).  Small bf16 layers are compared in full (every
EPD row, every expert's weight gradient, the router gradients); the
OLMoE-shaped layer on sampled tokens (their EPD rows) and two slots' weight
gradients.  Each stage is checked on the inputs the GPU stored for it (its
routing weights, its out_EPD for dw, its dw for the router, its d_epd for
the dispatch gradient): those inputs match the oracle's own only to the
forward's bf16 tolerance, and a stage's own arithmetic is held to a tighter
bound.  The expert backward itself (recomputed G and U, dG, dU, d_epd and
the weight gradients) is compared with the oracle's chain end to end."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_common import oracle_logits_parallel, say
from tests.tolerance import assert_close
from tests.tolerance import rel_err

pytestmark = pytest.mark.gpu

SMALL = {
    "bf16_ragged": W.LayerConfig("bf16_ragged", T=300, d=128, E=16, I=128, k=4, D=4,
                                 dtype="bf16", clusters=4),
    "bf16_renorm": W.LayerConfig("bf16_renorm", T=200, d=128, E=8, I=64, k=2, D=2,
                                 dtype="bf16", renorm=1),
    "bf16_e128_pairs": W.LayerConfig("bf16_e128_pairs", T=513, d=64, E=128, I=64, k=6, D=16,
                                     dtype="bf16", clusters=8),
    "bf16_one_expert_per_device": W.LayerConfig("bf16_one_expert_per_device", T=150, d=128,
                                                E=8, I=64, k=2, D=8, dtype="bf16"),
    # the largest device count and picks per token the library takes
    "bf16_max_devices_and_k": W.LayerConfig("bf16_max_devices_and_k", T=200, d=64, E=64, I=64,
                                            k=16, D=32, dtype="bf16", clusters=4),
    # an expert count that is not a multiple of 4 and a ragged token count:
    # the router gradient's products take their element-wise operand loads
    "bf16_e6": W.LayerConfig("bf16_e6", T=131, d=64, E=6, I=64, k=2, D=2, dtype="bf16"),
}


def _run_gpu(cfg, inp, dy_bits):
    import torch
    from expert_top_router_amd.layer import MoELayer, to_device, upload_inputs
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert, with_logits=True)
    lay.prepare_backward()
    say(f"  gpu forward+backward {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} D={cfg.D}")
    lay.forward()
    lay.dy.copy_(to_device(dy_bits))
    lay.grad_combine()
    lay.expert_backward()
    torch.cuda.synchronize()
    # [G | U] and [dG | dU] sit in the workspace (each part 256-byte aligned)
    # until the router gradient reuses it for its partial sums
    R, I = cfg.R, cfg.I
    ws = lay.bwd_ws.view(torch.int16)
    half = -(-R * 2 * I * 2 // 256) * 256 // 2  # int16 elements before [dG | dU]
    gu = ws[:R * 2 * I].cpu().numpy().view(np.uint16).reshape(R, 2 * I)
    dgu = ws[half:half + R * 2 * I].cpu().numpy().view(np.uint16).reshape(R, 2 * I)
    lay.router_backward()
    lay.grad_dispatch()
    torch.cuda.synchronize()
    names = ["topk_idx", "topk_w", "logits", "brim0", "brim1", "slot_offset", "epd_token",
             "epd_sfd", "epd_w", "S", "d_out_epd", "dw_epd", "d_epd", "dw_gate_up", "dw_down",
             "dlogits", "dx_router", "dw_router", "d_sfd", "d_out_sfd", "dx", "out_epd"]
    g = {n: lay.host(n) for n in names}
    g["gu"], g["dgu"] = gu, dgu
    del lay
    torch.cuda.empty_cache()
    return g


def _bf(a):
    return W.to_f32(a, "bf16").astype(np.float64)


def _row_of(b, idx, slot_expert, cfg):
    """EPD row of (token t, pick j), through BRIM_0 and BRIM_1."""
    L = cfg.E // cfg.D
    slot_of = np.empty(cfg.E, np.int64)
    slot_of[np.asarray(slot_expert)] = np.arange(cfg.E)

    def row_of(t, j):
        gs = slot_of[idx[t, j]]
        return int(b["brim1"][gs % L, b["brim0"][gs // L, t]])
    return row_of


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_backward_parity(orc, name):
    import oracle.backward as ob
    cfg = SMALL[name]
    say(f"case backward {name}")
    inp = W.make_layer(cfg, seed=9)
    dy = W.from_f64(np.random.default_rng(9).standard_normal((cfg.T, cfg.d)), "bf16")
    g = _run_gpu(cfg, inp, dy)
    lg = oracle_logits_parallel(orc, inp.x, inp.w_router, "bf16")
    assert np.array_equal(g["logits"].view(np.uint32), lg.view(np.uint32))
    idx = g["topk_idx"]
    b = orc.brim(idx, g["topk_w"], inp.slot_expert, cfg.E, cfg.D)
    assert np.array_equal(g["epd_token"], b["epd_token"])
    o = ob.full(_bf(inp.x), _bf(inp.w_router), _bf(inp.w_gate_up), _bf(inp.w_down), lg, idx,
                g["topk_w"], cfg.renorm, b, inp.slot_expert, _bf(dy), cfg.D, "bf16")
    I = cfg.I
    S = b["S"]
    g_out_epd = g["out_epd"]
    # the send buffer is a bit copy of dy
    assert np.array_equal(g["d_out_sfd"][:S], dy[b["sfd_token"][:S]]), "d_out_sfd"
    assert_close(_bf(g["d_out_epd"]), o["d_out_epd"], "bf16", "d_out_epd")
    # dw = <dy, out_EPD> on the GPU's stored out_EPD
    t_of = b["epd_token"]
    dw_ref = np.sum(_bf(dy)[t_of] * _bf(g_out_epd), axis=1)
    assert rel_err(g["dw_epd"], dw_ref) <= 1e-4, "dw_epd"
    assert_close(g["dw_epd"], o["dw"], "bf16", "dw_epd (oracle chain)")
    assert_close(_bf(g["gu"][:, :I]), o["G"], "bf16", "G (recomputed)")
    assert_close(_bf(g["gu"][:, I:]), o["U"], "bf16", "U (recomputed)")
    assert_close(_bf(g["dgu"][:, :I]), o["dG"], "bf16", "dG")
    assert_close(_bf(g["dgu"][:, I:]), o["dU"], "bf16", "dU")
    assert_close(_bf(g["d_epd"]), o["d_epd"], "bf16", "d_epd")
    assert_close(g["dw_gate_up"], o["dW_gate_up"], "bf16", "dW_gate_up")
    assert_close(g["dw_down"], o["dW_down"], "bf16", "dW_down")
    # router gradient on the GPU's dw
    row_of = _row_of(b, idx, inp.slot_expert, cfg)
    dl = ob.router_grads(lg, idx, g["topk_w"], cfg.renorm,
                         lambda t, j: float(g["dw_epd"][row_of(t, j)]), np.arange(cfg.T))
    assert rel_err(g["dlogits"], dl) <= 1e-4, "dlogits"
    assert rel_err(g["dx_router"], dl @ _bf(inp.w_router)) <= 1e-4, "dx_router"
    assert rel_err(g["dw_router"], dl.T @ _bf(inp.x)) <= 1e-4, "dw_router"
    assert_close(g["dlogits"], o["dlogits"], "bf16", "dlogits (oracle chain)")
    # dispatch gradient on the GPU's d_epd and dx_router
    dx, dsfd = ob.grad_dispatch(b, lambda r: _bf(g["d_epd"][r]), np.arange(cfg.T), cfg.T, cfg.D,
                                cfg.E // cfg.D, cfg.d, "bf16", g["dx_router"])
    srows = np.array(sorted(dsfd), dtype=np.int64)
    assert_close(_bf(g["d_sfd"][srows]), np.stack([dsfd[s] for s in srows]), "bf16", "d_sfd")
    assert_close(_bf(g["dx"]), dx, "bf16", "dx")
    assert_close(_bf(g["dx"]), o["dx"], "bf16", "dx (oracle chain)")


def test_full_size_backward_parity(orc):
    """OLMoE-shaped layer: sampled tokens' EPD rows, their dx, and the weight
    gradients of two slots (the least and the most loaded)."""
    import oracle.backward as ob
    cfg = W.CONFIGS["olmoe_bf16"]
    say("case backward full olmoe_bf16: generating inputs")
    inp = W.make_layer(cfg, seed=0)
    dy = W.from_f64(np.random.default_rng(10).standard_normal((cfg.T, cfg.d)), "bf16")
    g = _run_gpu(cfg, inp, dy)
    idx = g["topk_idx"]
    b = orc.brim(idx, g["topk_w"], inp.slot_expert, cfg.E, cfg.D)
    assert np.array_equal(g["epd_token"], b["epd_token"])
    X, WR, WGU, WD, DY = (_bf(a) for a in (inp.x, inp.w_router, inp.w_gate_up, inp.w_down, dy))
    rng = np.random.default_rng(11)
    tok = np.sort(rng.choice(cfg.T, size=24, replace=False))
    L = cfg.E // cfg.D
    rows = []
    for t in tok:
        for dv in range(cfg.D):
            s = b["brim0"][dv, t]
            if s >= 0:
                rows += [r for r in b["brim1"][:, s] if r >= 0]
    rows = np.array(sorted(rows), dtype=np.int64)
    say(f"  oracle on {tok.size} tokens, {rows.size} EPD rows")
    o = ob.expert_rows(X, WGU, WD, b, inp.slot_expert, DY, rows, "bf16")
    I = cfg.I
    assert_close(_bf(g["d_out_epd"][rows]), o["d_out_epd"], "bf16", "d_out_epd")
    dw_ref = np.sum(DY[b["epd_token"][rows]] * _bf(g["out_epd"][rows]), axis=1)
    assert rel_err(g["dw_epd"][rows], dw_ref) <= 1e-4, "dw_epd"
    assert_close(_bf(g["dgu"][rows, :I]), o["dG"], "bf16", "dG")
    assert_close(_bf(g["dgu"][rows, I:]), o["dU"], "bf16", "dU")
    assert_close(_bf(g["d_epd"][rows]), o["d_epd"], "bf16", "d_epd")
    row_of = _row_of(b, idx, inp.slot_expert, cfg)
    lg = g["logits"]
    dl = ob.router_grads(lg, idx, g["topk_w"], cfg.renorm,
                         lambda t, j: float(g["dw_epd"][row_of(t, j)]), tok)
    assert rel_err(g["dlogits"][tok], dl) <= 1e-4, "dlogits"
    dxr = dl @ WR
    assert rel_err(g["dx_router"][tok], dxr) <= 1e-4, "dx_router"
    dx, _ = ob.grad_dispatch(b, lambda r: _bf(g["d_epd"][r]), tok, cfg.T, cfg.D, L, cfg.d, "bf16",
                             g["dx_router"][tok])
    assert_close(_bf(g["dx"][tok]), dx, "bf16", "dx")
    cnt = np.diff(b["slot_offset"])
    for gs in (int(np.argmin(np.where(cnt > 0, cnt, cnt.max() + 1))), int(np.argmax(cnt))):
        say(f"  weight gradients of slot {gs} ({cnt[gs]} rows)")
        dWgu, dWd = ob.slot_weight_grads(X, WGU, WD, b, inp.slot_expert, DY, gs, "bf16")
        e = inp.slot_expert[gs]
        assert_close(g["dw_gate_up"][e], dWgu, "bf16", f"dW_gate_up[{e}]")
        assert_close(g["dw_down"][e], dWd, "bf16", f"dW_down[{e}]")


def test_empty_batch_backward():
    """T = 0: every call is a no-op on the rows, and the weight gradients
    (sums over no rows) are written as zeros over poisoned buffers."""
    import torch
    from expert_top_router_amd.layer import MoELayer, upload_inputs
    cfg = W.LayerConfig("bf16_empty", T=0, d=64, E=8, I=64, k=2, D=2, dtype="bf16")
    inp = W.make_layer(cfg, seed=3)
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert, with_logits=True)
    lay.prepare_backward()
    say("  gpu forward+backward bf16_empty T=0")
    for name in ("dw_gate_up", "dw_down", "dw_router"):
        getattr(lay, name).fill_(float("nan"))
    lay.forward()
    lay.backward()
    torch.cuda.synchronize()
    for name in ("dw_gate_up", "dw_down", "dw_router"):
        g = lay.host(name)
        assert g.size > 0 and np.all(g == 0.0), name


@pytest.mark.parametrize("budget,rescale", [(1, 1), (2, 0)])
def test_pruned_layer_backward_parity(orc, budget, rescale):
    """The backward under collaboration pruning: the BRIMs hold the kept
    picks with their stored weights; the expert backward, the dispatch
    gradient and the routing gradient (no gradient for dropped picks)
    against the backward oracle on the same BRIMs."""
    import torch
    import oracle.backward as ob
    from expert_top_router_amd.layer import MoELayer, to_device, upload_inputs
    cfg = SMALL["bf16_ragged"]
    say(f"case pruned backward budget={budget} rescale={rescale}")
    inp = W.make_layer(cfg, seed=21)
    dy = W.from_f64(np.random.default_rng(21).standard_normal((cfg.T, cfg.d)), "bf16")
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert, with_logits=True, budget=budget,
                   rescale=rescale)
    lay.prepare_backward()
    lay.forward()
    lay.dy.copy_(to_device(dy))
    lay.grad_combine()
    lay.expert_backward()
    torch.cuda.synchronize()
    R, I = int(lay.host("slot_offset")[cfg.E]), cfg.I
    Rmax = cfg.R
    ws = lay.bwd_ws.view(torch.int16)
    half = -(-Rmax * 2 * I * 2 // 256) * 256 // 2
    gu = ws[:Rmax * 2 * I].cpu().numpy().view(np.uint16).reshape(Rmax, 2 * I)[:R]
    dgu = ws[half:half + Rmax * 2 * I].cpu().numpy().view(np.uint16).reshape(Rmax, 2 * I)[:R]
    lay.router_backward()
    lay.grad_dispatch()
    torch.cuda.synchronize()
    g = {n: lay.host(n) for n in ("topk_idx", "topk_w", "logits", "epd_token", "dw_epd", "d_epd",
                                  "dw_gate_up", "dw_down", "dlogits", "dx", "dx_router")}
    del lay
    torch.cuda.empty_cache()
    idx, w = g["topk_idx"], g["topk_w"]
    ik, wk = orc.prune(idx, w, inp.slot_expert, cfg.E, cfg.D, budget, rescale)
    assert np.any(ik < 0)
    b = orc.brim(ik, wk, inp.slot_expert, cfg.E, cfg.D)
    assert b["R"] == R and np.array_equal(g["epd_token"][:R], b["epd_token"])
    o = ob.full(_bf(inp.x), _bf(inp.w_router), _bf(inp.w_gate_up), _bf(inp.w_down), g["logits"],
                idx, w, cfg.renorm, b, inp.slot_expert, _bf(dy), cfg.D, "bf16")
    assert_close(_bf(gu[:, :I]), o["G"], "bf16", "G (recomputed)")
    assert_close(_bf(gu[:, I:]), o["U"], "bf16", "U (recomputed)")
    assert_close(_bf(dgu[:, :I]), o["dG"], "bf16", "dG")
    assert_close(_bf(dgu[:, I:]), o["dU"], "bf16", "dU")
    assert_close(_bf(g["d_epd"][:R]), o["d_epd"], "bf16", "d_epd")
    assert_close(g["dw_gate_up"], o["dW_gate_up"], "bf16", "dW_gate_up")
    assert_close(g["dw_down"], o["dW_down"], "bf16", "dW_down")
    assert_close(g["dw_epd"][:R], o["dw"], "bf16", "dw_epd")
    # routing gradient on the GPU's own dw: dropped picks carry none
    row_of = _row_of(b, idx, inp.slot_expert, cfg)
    L = cfg.E // cfg.D
    slot_of = np.empty(cfg.E, np.int64)
    slot_of[np.asarray(inp.slot_expert)] = np.arange(cfg.E)

    def dw_of(t, j):
        gs = slot_of[idx[t, j]]
        if b["brim0"][gs // L, t] < 0:
            return 0.0
        return float(g["dw_epd"][row_of(t, j)])
    dl = ob.router_grads(g["logits"], idx, w, cfg.renorm, dw_of, np.arange(cfg.T))
    assert rel_err(g["dlogits"], dl) <= 1e-4, "dlogits"
    assert rel_err(g["dx_router"], dl @ _bf(inp.w_router)) <= 1e-4, "dx_router"
    dx, _ = ob.grad_dispatch(b, lambda r: _bf(g["d_epd"][r]), np.arange(cfg.T), cfg.T, cfg.D,
                             L, cfg.d, "bf16", g["dx_router"])
    assert_close(_bf(g["dx"]), dx, "bf16", "dx")


@pytest.mark.parametrize("name", ["bf16_ragged", "olmoe_bf16"])
def test_kept_preactivations_match_recompute(name):
    """occ_expert_ffn_keep + occ_expert_backward_kept against occ_expert_ffn +
    occ_expert_backward: the kept [G | U] equals the backward's recomputed
    one, and every output and gradient is the same, bit for bit."""
    import torch
    from expert_top_router_amd.layer import MoELayer, to_device, upload_inputs
    from tests.test_gpu_parity import SMALL

    cfg = SMALL[name] if name in SMALL else W.CONFIGS[name]
    say(f"case kept [G | U] {name}")
    inp = W.make_layer(cfg, seed=23)
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert, with_logits=True)
    lay.prepare_backward()
    dy = W.from_f64(np.random.default_rng(23).standard_normal((cfg.T, cfg.d)), "bf16")
    lay.dy.copy_(to_device(dy))
    names = ("out_epd", "y", "d_epd", "dw_gate_up", "dw_down", "dx", "dw_router", "dlogits")

    def bits(t):
        return t.contiguous().view(torch.uint8).clone()

    lay.forward()
    lay.grad_combine()
    lay.expert_backward()
    torch.cuda.synchronize()
    R = int(lay.host("slot_offset")[-1])
    I2 = 2 * cfg.I
    # the recomputed [G | U] (the router gradient reuses the workspace next)
    gu_ref = bits(lay.bwd_ws[:R * I2 * 2])
    lay.router_backward()
    lay.grad_dispatch()
    torch.cuda.synchronize()
    ref = {n: bits(getattr(lay, n)) for n in names}
    lay.poison()
    for n in ("d_epd", "dw_gate_up", "dw_down", "dx", "dw_router", "dlogits", "gu", "bwd_ws"):
        getattr(lay, n).view(torch.uint8).fill_(0xA5)
    torch.cuda.synchronize()
    lay.forward_keep()
    lay.backward_kept()
    torch.cuda.synchronize()
    assert torch.equal(bits(lay.gu.view(-1)[:R * I2]), gu_ref), "kept [G | U]"
    for n in names:
        assert torch.equal(bits(getattr(lay, n)), ref[n]), n


SHARED = {
    # two shared experts beside the routed ones, renormalised routing
    "bf16_shared": W.LayerConfig("bf16_shared", T=200, d=128, E=8, I=64, k=2, D=2,
                                 dtype="bf16", n_shared=2, I_shared=64, renorm=1),
    # more rows than one GEMM tile, a shared intermediate of two weight tiles
    "bf16_shared_wide": W.LayerConfig("bf16_shared_wide", T=300, d=128, E=16, I=64, k=4, D=4,
                                      dtype="bf16", n_shared=2, I_shared=384, clusters=4),
}


def _run_gpu_shared(cfg, inp, dy_bits):
    """Forward, then the whole backward with the shared experts; returns the
    gradients and the shared experts' recomputed [G | U] and [dG | dU]."""
    import torch
    from expert_top_router_amd.layer import MoELayer, to_device, upload_inputs
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert, with_logits=True)
    lay.prepare_backward()
    say(f"  gpu forward+backward {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} "
        f"n_shared={cfg.n_shared} I_shared={cfg.I_shared}")
    for t in (lay.dx_shared, lay.dw_gate_up_sh, lay.dw_down_sh, lay.dx):
        t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).fill_(-1)
    lay.forward()
    lay.dy.copy_(to_device(dy_bits))
    lay.grad_combine()
    lay.expert_backward()
    lay.router_backward()
    lay.shared_backward()
    torch.cuda.synchronize()
    W2 = cfg.n_shared * 2 * cfg.I_shared
    ws = lay.bwd_ws.view(torch.int16)
    half = -(-cfg.T * W2 * 2 // 256) * 256 // 2
    g = {"gu_sh": ws[:cfg.T * W2].cpu().numpy().view(np.uint16).reshape(cfg.T, W2),
         "dgu_sh": ws[half:half + cfg.T * W2].cpu().numpy().view(np.uint16).reshape(cfg.T, W2)}
    lay.grad_dispatch()
    torch.cuda.synchronize()
    for n in ("topk_idx", "topk_w", "logits", "epd_token", "d_epd", "dx_router", "dx_shared",
              "dw_gate_up_sh", "dw_down_sh", "dx", "dw_gate_up", "dw_down"):
        g[n] = lay.host(n)
    del lay
    torch.cuda.empty_cache()
    return g


@pytest.mark.parametrize("name", list(SHARED))
def test_shared_expert_backward_parity(orc, name):
    """Layers with shared experts: the shared experts' recomputed [G | U],
    [dG | dU], input gradient and weight gradients against the oracle end
    to end, the routed experts' weight gradients beside them, and dx (the
    dispatch gradient plus the router's and the shared experts' terms)."""
    import oracle.backward as ob
    cfg = SHARED[name]
    say(f"case shared backward {name}")
    inp = W.make_layer(cfg, seed=13)
    dy = W.from_f64(np.random.default_rng(13).standard_normal((cfg.T, cfg.d)), "bf16")
    g = _run_gpu_shared(cfg, inp, dy)
    lg = oracle_logits_parallel(orc, inp.x, inp.w_router, "bf16")
    assert np.array_equal(g["logits"].view(np.uint32), lg.view(np.uint32))
    idx = g["topk_idx"]
    b = orc.brim(idx, g["topk_w"], inp.slot_expert, cfg.E, cfg.D)
    assert np.array_equal(g["epd_token"], b["epd_token"])
    o = ob.full(_bf(inp.x), _bf(inp.w_router), _bf(inp.w_gate_up), _bf(inp.w_down), lg, idx,
                g["topk_w"], cfg.renorm, b, inp.slot_expert, _bf(dy), cfg.D, "bf16",
                shared=(_bf(inp.w_gate_up_sh), _bf(inp.w_down_sh)))
    Is = cfg.I_shared
    for s in range(cfg.n_shared):
        c0 = s * 2 * Is
        assert_close(_bf(g["gu_sh"][:, c0:c0 + Is]), o["G_sh"][s], "bf16", f"G_sh[{s}]")
        assert_close(_bf(g["gu_sh"][:, c0 + Is:c0 + 2 * Is]), o["U_sh"][s], "bf16", f"U_sh[{s}]")
        assert_close(_bf(g["dgu_sh"][:, c0:c0 + Is]), o["dG_sh"][s], "bf16", f"dG_sh[{s}]")
        assert_close(_bf(g["dgu_sh"][:, c0 + Is:c0 + 2 * Is]), o["dU_sh"][s], "bf16",
                     f"dU_sh[{s}]")
    assert_close(_bf(g["dx_shared"]), o["dx_shared"], "bf16", "dx_shared")
    assert_close(g["dw_gate_up_sh"], o["dW_gate_up_sh"], "bf16", "dW_gate_up_sh")
    assert_close(g["dw_down_sh"], o["dW_down_sh"], "bf16", "dW_down_sh")
    assert_close(g["dw_gate_up"], o["dW_gate_up"], "bf16", "dW_gate_up")
    assert_close(g["dw_down"], o["dW_down"], "bf16", "dW_down")
    # dx on the GPU's own d_epd, dx_router and dx_shared, then end to end
    dx, _ = ob.grad_dispatch(b, lambda r: _bf(g["d_epd"][r]), np.arange(cfg.T), cfg.T, cfg.D,
                             cfg.E // cfg.D, cfg.d, "bf16", g["dx_router"], _bf(g["dx_shared"]))
    assert_close(_bf(g["dx"]), dx, "bf16", "dx")
    assert_close(_bf(g["dx"]), o["dx"], "bf16", "dx (oracle chain)")


def test_full_size_shared_expert_backward(orc):
    """DeepSeek-V2-Lite-shaped layer (64 routed + 2 shared experts, T = 16384):
    the shared experts' input gradient on sampled tokens, their weight
    gradients at sampled intermediate columns (every row contributes), the
    routed backward on the sampled tokens' EPD rows, and dx on those tokens."""
    import oracle.backward as ob
    cfg = W.CONFIGS["dsv2lite_bf16"]
    say("case shared backward full dsv2lite_bf16: generating inputs")
    inp = W.make_layer(cfg, seed=0)
    dy = W.from_f64(np.random.default_rng(14).standard_normal((cfg.T, cfg.d)), "bf16")
    g = _run_gpu_shared(cfg, inp, dy)
    idx = g["topk_idx"]
    b = orc.brim(idx, g["topk_w"], inp.slot_expert, cfg.E, cfg.D)
    assert np.array_equal(g["epd_token"], b["epd_token"])
    X, WGU, WD, DY = (_bf(a) for a in (inp.x, inp.w_gate_up, inp.w_down, dy))
    WGS, WDS = _bf(inp.w_gate_up_sh), _bf(inp.w_down_sh)
    rng = np.random.default_rng(15)
    tok = np.sort(rng.choice(cfg.T, size=16, replace=False))
    sh = ob.shared_backward(X, WGS, WDS, DY, tok, "bf16")
    Is = cfg.I_shared
    for s in range(cfg.n_shared):
        c0 = s * 2 * Is
        assert_close(_bf(g["dgu_sh"][tok, c0:c0 + Is]), sh["dG"][s], "bf16", f"dG_sh[{s}]")
        assert_close(_bf(g["dgu_sh"][tok, c0 + Is:c0 + 2 * Is]), sh["dU"][s], "bf16",
                     f"dU_sh[{s}]")
    assert_close(_bf(g["dx_shared"][tok]), sh["dx_shared"], "bf16", "dx_shared")
    cols = np.array(sorted({0, 1, Is - 1, *rng.choice(Is, size=3, replace=False).tolist()}))
    for s in range(cfg.n_shared):
        say(f"  shared expert {s}: weight gradients at intermediate columns {cols.tolist()}")
        gr, ur, dc = ob.shared_weight_grad_columns(X, WGS, WDS, DY, s, cols, "bf16")
        assert_close(g["dw_gate_up_sh"][s][cols], gr, "bf16", f"dW_gate_sh[{s}]")
        assert_close(g["dw_gate_up_sh"][s][Is + cols], ur, "bf16", f"dW_up_sh[{s}]")
        assert_close(g["dw_down_sh"][s][:, cols], dc, "bf16", f"dW_down_sh[{s}]")
    # dx of the sampled tokens from the GPU's d_epd, dx_router and dx_shared
    L = cfg.E // cfg.D
    dx, _ = ob.grad_dispatch(b, lambda r: _bf(g["d_epd"][r]), tok, cfg.T, cfg.D, L, cfg.d,
                             "bf16", g["dx_router"][tok], _bf(g["dx_shared"][tok]))
    assert_close(_bf(g["dx"][tok]), dx, "bf16", "dx")
    # the routed backward of the sampled tokens' EPD rows, end to end
    rows = []
    for t in tok:
        for dv in range(cfg.D):
            s_ = b["brim0"][dv, t]
            if s_ >= 0:
                rows += [r for r in b["brim1"][:, s_] if r >= 0]
    rows = np.array(sorted(rows), dtype=np.int64)
    o = ob.expert_rows(X, WGU, WD, b, inp.slot_expert, DY, rows, "bf16")
    assert_close(_bf(g["d_epd"][rows]), o["d_epd"], "bf16", "d_epd")


F32 = {
    "tiny_fp32": W.CONFIGS["tiny_fp32"],
    # odd sizes: 12 experts on 3 devices, top-3, a narrow intermediate
    "f32_e12": W.LayerConfig("f32_e12", T=77, d=64, E=12, I=32, k=3, D=3, dtype="f32"),
    # shared experts and renormalised routing
    "f32_shared": W.LayerConfig("f32_shared", T=100, d=64, E=8, I=32, k=2, D=2, dtype="f32",
                                n_shared=2, I_shared=48, renorm=1, clusters=3),
}


@pytest.mark.parametrize("name", list(F32))
def test_fp32_layer_backward_parity(orc, name):
    """fp32 layers: the whole backward (grad-combine, expert backward, router
    gradient, shared experts, grad-dispatch) against the oracle's chain with
    fp32 storage, every tensor within the fp32 tolerance."""
    import torch
    import oracle.backward as ob
    from expert_top_router_amd.layer import MoELayer, to_device, upload_inputs
    cfg = F32[name]
    say(f"case fp32 backward {name}")
    inp = W.make_layer(cfg, seed=17)
    dy = np.random.default_rng(17).standard_normal((cfg.T, cfg.d)).astype(np.float32)
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert, with_logits=True)
    lay.prepare_backward()
    say(f"  gpu forward+backward {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} fp32")
    lay.forward()
    lay.backward(to_device(dy))
    torch.cuda.synchronize()
    names = ["topk_idx", "topk_w", "logits", "epd_token", "d_out_epd", "dw_epd", "d_epd",
             "dw_gate_up", "dw_down", "dlogits", "dx_router", "dw_router", "dx"]
    if cfg.n_shared:
        names += ["dx_shared", "dw_gate_up_sh", "dw_down_sh"]
    g = {n: lay.host(n) for n in names}
    del lay
    torch.cuda.empty_cache()
    lg = oracle_logits_parallel(orc, inp.x, inp.w_router, "f32")
    assert np.array_equal(g["logits"].view(np.uint32), lg.view(np.uint32))
    idx = g["topk_idx"]
    b = orc.brim(idx, g["topk_w"], inp.slot_expert, cfg.E, cfg.D)
    assert np.array_equal(g["epd_token"], b["epd_token"])
    f64 = lambda a: np.asarray(a, np.float64)  # noqa: E731
    shared = (f64(inp.w_gate_up_sh), f64(inp.w_down_sh)) if cfg.n_shared else None
    o = ob.full(f64(inp.x), f64(inp.w_router), f64(inp.w_gate_up), f64(inp.w_down), lg, idx,
                g["topk_w"], cfg.renorm, b, inp.slot_expert, f64(dy), cfg.D, "f32",
                shared=shared)
    for name_g, name_o in [("d_out_epd", "d_out_epd"), ("dw_epd", "dw"), ("d_epd", "d_epd"),
                           ("dw_gate_up", "dW_gate_up"), ("dw_down", "dW_down"),
                           ("dlogits", "dlogits"), ("dx_router", "dx_router"),
                           ("dw_router", "dW_router"), ("dx", "dx")]:
        assert_close(g[name_g], o[name_o], "f32", name_g)
    if cfg.n_shared:
        for name in ("dx_shared", "dw_gate_up_sh", "dw_down_sh"):
            assert_close(g[name], o[name.replace("dw_", "dW_")], "f32", name)
