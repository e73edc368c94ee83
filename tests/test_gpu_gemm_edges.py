"""GPU parity of the grouped expert GEMMs on crafted slot sizes.

The routing is written directly into the top-k buffers so that the slots
(one per expert, contiguous placement) get 0, 1, 31..33, 127..129, 255..257,
301 and 511..513 rows: empty slots, single rows, slots that end one row
before, on and after a 32-row MFMA block and a 256-row tile, and slots of
two and three tiles.  The intermediate size 192 leaves the second SwiGLU
column tile half full.  BRIMs, dispatch, expert outputs (every EPD row),
pre-reduced payload and combined output are compared with the oracle; the
routing kernel is not involved (its own parity is tested elsewhere).
"""
import numpy as np
import pytest

import workloads as W
from tests.gpu_common import as_f32, oracle_expert_rows_parallel, say
from tests.tolerance import assert_close

pytestmark = pytest.mark.gpu

COUNTS = [0, 1, 31, 32, 33, 127, 128, 129, 255, 256, 257, 301, 511, 512, 513, 0]


def crafted_routing(counts, k, seed):
    """Top-k choices with the given number of tokens per expert: the multiset
    of expert ids in a seeded random order, cut into tokens of k, then any
    expert repeated inside a token swapped with a pick of another token
    (which keeps every count).  Tokens with two experts on one device make
    the pre-reduction sum several rows."""
    rng = np.random.default_rng(seed)
    order = rng.permutation(np.repeat(np.arange(len(counts), dtype=np.int32), counts))
    assert order.size % k == 0
    T = order.size // k
    idx = order.reshape(T, k).copy()
    for t in range(T):
        for j in range(1, k):
            while idx[t, j] in idx[t, :j]:
                u, jj = int(rng.integers(T)), int(rng.integers(k))
                others_u = np.delete(idx[u], jj)
                if idx[u, jj] not in idx[t, :j] and idx[t, j] not in others_u:
                    idx[t, j], idx[u, jj] = idx[u, jj], idx[t, j]
    w = np.tile(np.array([0.625, 0.375][:k], np.float32), (T, 1))
    return np.ascontiguousarray(idx), np.ascontiguousarray(w)


@pytest.mark.parametrize("d,I", [(256, 192), (128, 64)])
def test_grouped_gemm_slot_edges(orc, d, I):
    import torch
    from expert_top_router_amd.layer import MoELayer, upload_inputs

    k, E, D = 2, len(COUNTS), 4
    idx, w = crafted_routing(COUNTS, k, seed=11)
    T = idx.shape[0]
    cfg = W.LayerConfig(f"gemm_edges_{d}_{I}", T=T, d=d, E=E, I=I, k=k, D=D, dtype="bf16")
    say(f"case gemm_edges T={T} d={d} I={I} counts={COUNTS}")
    inp = W.make_layer(cfg, seed=9)
    L = E // D

    b = orc.brim(idx, w, inp.slot_expert, E, D)
    assert np.array_equal(np.diff(b["slot_offset"]), np.asarray(COUNTS)[inp.slot_expert])
    S, R = b["S"], b["R"]
    ex_of_row = np.repeat(np.asarray(inp.slot_expert), np.diff(b["slot_offset"])).astype(np.int32)
    out_rows = oracle_expert_rows_parallel(orc, inp.x, b["epd_token"], ex_of_row,
                                           inp.w_gate_up, inp.w_down, "bf16")
    tok = np.arange(T, dtype=np.int32)
    y, osfd = orc.combine(tok, b, T, D, L, d, "bf16", out_rows, np.arange(R, dtype=np.int32),
                          None, want_sfd=True)

    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert)
    lay.poison()
    lay.topk_idx.copy_(torch.from_numpy(idx))
    lay.topk_w.copy_(torch.from_numpy(w))
    lay.build_brim()
    lay.dispatch()
    lay.expert_ffn()
    lay.combine()
    torch.cuda.synchronize()

    assert int(lay.host("S")[0]) == S
    for name in ("brim0", "sfd_offset", "slot_offset"):
        assert np.array_equal(lay.host(name), b[name]), name
    assert np.array_equal(lay.host("brim1")[:, :S], b["brim1"][:, :S]), "brim1"
    assert np.array_equal(lay.host("epd_token")[:R], b["epd_token"]), "epd_token"
    assert np.array_equal(lay.host("epd")[:R], inp.x[b["epd_token"]]), "epd"
    assert_close(as_f32(lay.host("out_epd")[:R], "bf16"), out_rows, "bf16", "out_epd")
    assert_close(as_f32(lay.host("out_sfd")[:S], "bf16"), osfd[:S], "bf16", "out_sfd")
    assert_close(as_f32(lay.host("y"), "bf16"), y, "bf16", "y")


def test_expert_backward_slot_edges(orc):
    """The backward GEMMs on the same crafted slots (empty slots, single rows,
    tile edges): recomputed G and U, dG and dU, d_EPD and both weight
    gradients against the backward oracle.  The router gradient is not
    involved (the crafted routing has no logits)."""
    import torch
    import oracle.backward as ob
    from expert_top_router_amd.layer import MoELayer, to_device, upload_inputs

    k, E, D, d, I = 2, len(COUNTS), 4, 128, 64
    idx, w = crafted_routing(COUNTS, k, seed=12)
    T = idx.shape[0]
    cfg = W.LayerConfig("gemm_edges_backward", T=T, d=d, E=E, I=I, k=k, D=D, dtype="bf16")
    say(f"case gemm_edges_backward T={T} d={d} I={I}")
    inp = W.make_layer(cfg, seed=13)
    dy = W.from_f64(np.random.default_rng(13).standard_normal((T, d)), "bf16")

    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert)
    lay.prepare_backward()
    lay.topk_idx.copy_(torch.from_numpy(idx))
    lay.topk_w.copy_(torch.from_numpy(w))
    lay.build_brim()
    lay.dispatch()
    lay.expert_ffn()
    lay.combine()
    lay.dy.copy_(to_device(dy))
    lay.grad_combine()
    lay.expert_backward()
    torch.cuda.synchronize()
    R = T * k
    ws = lay.bwd_ws.view(torch.int16)
    half = -(-R * 2 * I * 2 // 256) * 256 // 2  # int16 elements before [dG | dU]
    gu = ws[:R * 2 * I].cpu().numpy().view(np.uint16).reshape(R, 2 * I)
    dgu = ws[half:half + R * 2 * I].cpu().numpy().view(np.uint16).reshape(R, 2 * I)
    g = {n: lay.host(n) for n in ("epd_token", "d_epd", "dw_gate_up", "dw_down")}
    del lay
    torch.cuda.empty_cache()

    b = orc.brim(idx, w, inp.slot_expert, E, D)
    assert np.array_equal(g["epd_token"], b["epd_token"])
    bf = lambda a: W.to_f32(a, "bf16").astype(np.float64)  # noqa: E731
    # logits that rank each token's crafted picks first (only the routing
    # gradient reads them, and it is not compared here)
    lg = np.zeros((T, E), np.float32)
    lg[np.arange(T), idx[:, 0]] = 2.0
    lg[np.arange(T), idx[:, 1]] = 1.0
    o = ob.full(bf(inp.x), bf(inp.w_router), bf(inp.w_gate_up), bf(inp.w_down), lg, idx, w, 0, b,
                inp.slot_expert, bf(dy), D, "bf16")
    assert_close(bf(gu[:, :I]), o["G"], "bf16", "G (recomputed)")
    assert_close(bf(gu[:, I:]), o["U"], "bf16", "U (recomputed)")
    assert_close(bf(dgu[:, :I]), o["dG"], "bf16", "dG")
    assert_close(bf(dgu[:, I:]), o["dU"], "bf16", "dU")
    assert_close(bf(g["d_epd"]), o["d_epd"], "bf16", "d_epd")
    assert_close(g["dw_gate_up"], o["dW_gate_up"], "bf16", "dW_gate_up")
    assert_close(g["dw_down"], o["dW_down"], "bf16", "dW_down")
    # the experts without rows get exactly zero weight gradients
    for e in np.flatnonzero(np.asarray(COUNTS) == 0):
        assert not np.any(g["dw_gate_up"][e]) and not np.any(g["dw_down"][e]), f"expert {e}"
