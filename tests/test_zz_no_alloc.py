"""occ_build_brim_noalloc (the BRIM build whose workspace is the library's
fixed device array) against occ_build_brim with a caller workspace, through
the C ABI: every output bit for bit, on two calls in a row, the second on a
smaller layer (the array keeps the first call's contents)."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

NAMES = ("brim0", "sfd_offset", "slot_offset", "S")


def _outputs(lay, S):
    out = {n: lay.host(n) for n in NAMES}
    out["brim1"] = lay.host("brim1")[:, :S]
    out["sfd_token"] = lay.host("sfd_token")[:S]
    R = int(out["slot_offset"][-1])
    for n in ("epd_token", "epd_sfd", "epd_w"):
        out[n] = lay.host(n)[:R]
    return out


def _check(cfg, seed):
    import torch
    import expert_top_router_amd as occ
    from expert_top_router_amd.layer import MoELayer, upload_inputs
    inp = W.make_layer(cfg, seed=seed, experts=False)
    se = np.random.default_rng(seed).permutation(cfg.E).astype(np.int32)
    lay = MoELayer(cfg, upload_inputs(inp), se)
    say(f"  noalloc case {cfg.name} T={cfg.T} E={cfg.E} k={cfg.k} D={cfg.D}")
    lay.route()
    lay.build_brim()
    torch.cuda.synchronize()
    ref = _outputs(lay, int(lay.host("S")[0]))
    for t in (lay.brim0, lay.brim1, lay.sfd_offset, lay.slot_offset, lay.sfd_token,
              lay.epd_token, lay.epd_sfd, lay.S):
        t.fill_(0x7A7A7A7A)
    lay.epd_w.fill_(float("nan"))
    occ.occ_build_brim_noalloc(lay.desc, lay.topk_idx, lay.topk_w, se, lay.brim)
    torch.cuda.synchronize()
    got = _outputs(lay, int(ref["S"][0]))
    for n in ref:
        assert np.array_equal(got[n].view(np.uint8), ref[n].view(np.uint8)), (cfg.name, n)
    assert int(ref["slot_offset"][-1]) == cfg.R
    del lay
    return int(ref["S"][0])


def test_noalloc_brim_matches_workspace_brim_twice():
    big = W.LayerConfig("noalloc_big", T=9000, d=64, E=128, I=64, k=6, D=16, dtype="bf16",
                        clusters=8)
    small = W.LayerConfig("noalloc_small", T=301, d=64, E=16, I=64, k=4, D=4, dtype="bf16",
                          clusters=4)
    s1 = _check(big, seed=31)
    s2 = _check(small, seed=32)
    say(f"  S = {s1} then {s2}")
