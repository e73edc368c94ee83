"""The layer step captured in a HIP graph (torch's graph API around the same
C-ABI calls) and replayed: every replay must give the eager result bit for
bit.  Between replays the token tensor is replaced and the outputs are
poisoned, so a replay that skipped or reused work would show.  The library
clears its counters with kernels (no memset nodes) and synchronises with
nothing on the host, which is what makes the step capturable.
"""
import numpy as np
import pytest

import workloads as W
from tests.gpu_common import say
from tests.test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def _defined(lay):
    """The parts of the outputs that the step defines (rows < S, < R')."""
    S = int(lay.host("S")[0])
    R = int(lay.host("slot_offset")[-1])
    out = {n: lay.host(n) for n in ("topk_idx", "topk_w", "brim0", "sfd_offset", "slot_offset",
                                    "y")}
    out["brim1"] = lay.host("brim1")[:, :S]
    for n in ("sfd_token", "sfd", "out_sfd"):
        out[n] = lay.host(n)[:S]
    for n in ("epd_token", "epd_sfd", "epd_w", "epd", "out_epd"):
        out[n] = lay.host(n)[:R]
    return out


def _grads(lay):
    R = int(lay.host("slot_offset")[-1])
    S = int(lay.host("S")[0])
    out = {n: lay.host(n) for n in ("dw_gate_up", "dw_down", "dlogits", "dx_router",
                                    "dw_router", "dx")}
    out["d_epd"] = lay.host("d_epd")[:R]
    out["d_sfd"] = lay.host("d_sfd")[:S]
    if lay.cfg.n_shared:
        out.update({n: lay.host(n) for n in ("dx_shared", "dw_gate_up_sh", "dw_down_sh")})
    return out


def _same(a, b, what):
    assert a.keys() == b.keys()
    for n in a:
        assert a[n].shape == b[n].shape, (what, n)
        assert np.array_equal(a[n].view(np.uint8), b[n].view(np.uint8)), (what, n)


@pytest.mark.parametrize("name,budget,backward", [
    ("bf16_ragged", None, False), ("bf16_shared", None, False), ("f32_e12", None, False),
    ("bf16_ragged", 2, False), ("bf16_ragged", None, True), ("bf16_shared", None, True),
    ("f32_e12", None, True),
])
def test_graph_replays_match_eager(name, budget, backward):
    import torch
    from expert_top_router_amd.layer import MoELayer, to_device, upload_inputs

    cfg = SMALL[name]
    say(f"case graph {name} budget={budget} backward={backward}")
    inp = W.make_layer(cfg, seed=21)
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert, budget=budget,
                   with_logits=backward)
    if backward:
        lay.prepare_backward()
        dy = W.from_f64(np.random.default_rng(21).standard_normal((cfg.T, cfg.d)), cfg.dtype)
        lay.dy.copy_(to_device(dy))

    def step():
        lay.forward()
        if backward:
            lay.backward()

    # warm up on a side stream, then capture (torch's recipe)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for token_seed in (31, 32, 33):
        lay.w.x.copy_(to_device(W.make_tokens(cfg, seed=21, token_seed=token_seed)))
        step()
        torch.cuda.synchronize()
        ref = _defined(lay)
        ref_g = _grads(lay) if backward else None
        lay.poison()
        if backward:
            for n in ("d_epd", "dw_gate_up", "dw_down", "dlogits", "dx_router", "dw_router",
                      "d_sfd", "dx", "dx_shared", "dw_gate_up_sh", "dw_down_sh"):
                t = getattr(lay, n)
                if t is None:
                    continue
                t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(_defined(lay), ref, f"replay token_seed={token_seed}")
        if backward:
            _same(_grads(lay), ref_g, f"replay gradients token_seed={token_seed}")
