"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small layers are compared element by element at every stage (routing, BRIMs,
dispatch, expert outputs, pre-reduction, combine, co-activation); they span
several GEMM tiles with ragged tails, both dtypes, shared experts, more than
64 (device, expert) pairs, non-power-of-two expert counts, D = 1, L = 1, the
largest device count and picks per token (D = 32, k = 16), top-1, top-E and
an empty batch.
The five full-size layers are compared on the full batch for all integer work
and on sampled tokens for the expert arithmetic.
"""
import numpy as np
import pytest

import workloads as W
from tests.gpu_common import compare, gpu_layer, oracle_layer, prune_decisions, say

pytestmark = pytest.mark.gpu

SMALL = {
    # name: config (several tiles, ragged tails)
    "tiny_fp32": W.CONFIGS["tiny_fp32"],
    "bf16_ragged": W.LayerConfig("bf16_ragged", T=300, d=128, E=16, I=128, k=4, D=4,
                                 dtype="bf16", clusters=4),
    "bf16_shared": W.LayerConfig("bf16_shared", T=200, d=128, E=8, I=64, k=2, D=2,
                                 dtype="bf16", n_shared=2, I_shared=64, renorm=1),
    "bf16_e128_pairs": W.LayerConfig("bf16_e128_pairs", T=513, d=64, E=128, I=64, k=6, D=16,
                                     dtype="bf16", clusters=8),
    "f32_e12": W.LayerConfig("f32_e12", T=77, d=64, E=12, I=32, k=3, D=3, dtype="f32"),
    "bf16_one_device": W.LayerConfig("bf16_one_device", T=129, d=64, E=8, I=64, k=3, D=1,
                                     dtype="bf16"),
    "bf16_one_expert_per_device": W.LayerConfig("bf16_one_expert_per_device", T=150, d=128,
                                                E=8, I=64, k=2, D=8, dtype="bf16"),
    "bf16_wide_rows": W.LayerConfig("bf16_wide_rows", T=130, d=4096, E=4, I=64, k=2, D=2,
                                    dtype="bf16"),
    "f32_empty": W.LayerConfig("f32_empty", T=0, d=64, E=8, I=32, k=2, D=2, dtype="f32"),
    # one expert per token (each token on one device, S = T)
    "bf16_top1": W.LayerConfig("bf16_top1", T=257, d=128, E=16, I=64, k=1, D=4, dtype="bf16",
                               clusters=4),
    # every token picks every expert (S = T * D, EPD = T * E; renormalised
    # weights equal the softmax)
    "bf16_all_experts": W.LayerConfig("bf16_all_experts", T=96, d=64, E=8, I=64, k=8, D=4,
                                      dtype="bf16", renorm=1),
    # the largest device count and picks per token the library takes
    "bf16_max_devices_and_k": W.LayerConfig("bf16_max_devices_and_k", T=200, d=64, E=64, I=64,
                                            k=16, D=32, dtype="bf16", clusters=4),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_parity(orc, name):
    cfg = SMALL[name]
    say(f"case {name}")
    inp = W.make_layer(cfg, seed=3)
    o = oracle_layer(orc, inp)
    g = gpu_layer(inp)
    compare(g, o, inp)


def test_placement_permutation_and_determinism(orc):
    """A non-contiguous placement (greedy from the co-activation counts) and
    two runs that must agree bit for bit."""
    cfg = SMALL["bf16_ragged"]
    inp = W.make_layer(cfg, seed=4)
    base = oracle_layer(orc, inp)
    inp.slot_expert = orc.greedy_placement(base["coact"], cfg.D)
    o = oracle_layer(orc, inp)
    g1, g2 = gpu_layer(inp, runs=2)
    compare(g1, o, inp)
    for n in g1:
        assert np.array_equal(g1[n].view(np.uint8), g2[n].view(np.uint8)), n


def test_routing_ties_lower_index_first(orc):
    """Integer-valued tokens and router rows make many logits equal; the
    chosen experts must still match the oracle (lower index on ties)."""
    cfg = W.LayerConfig("ties", T=256, d=64, E=16, I=64, k=4, D=4, dtype="bf16")
    inp = W.make_layer(cfg, seed=5)
    rng = np.random.default_rng(5)
    inp.x = W.from_f64(rng.integers(-1, 2, size=(cfg.T, cfg.d)).astype(np.float64), "bf16")
    wr = rng.integers(-1, 2, size=(cfg.E, cfg.d)).astype(np.float64)
    wr[8:] = wr[:8]  # duplicated experts: exact ties everywhere
    inp.w_router = W.from_f64(wr, "bf16")
    o = oracle_layer(orc, inp)
    assert (np.diff(np.sort(o["logits"], axis=1), axis=1) == 0).any()
    g = gpu_layer(inp)
    compare(g, o, inp)


@pytest.mark.parametrize("T,E,k,renorm,dtype,d", [
    # from 16384 tokens, routers of 33..128 experts run on the matrix cores
    # when d is a multiple of the chunk width; fp32 tokens with d = 200 keep
    # these on the VALU mappings
    (16384, 64, 16, 0, "f32", 200),   # 16-lane segments, 4 experts per lane
    (16383, 64, 6, 1, "f32", 200),    # the same with a ragged last block
    (4096, 64, 8, 0, "bf16", 192),    # whole-wave segments with DPP broadcasts
    (3001, 128, 16, 0, "bf16", 192),  # 16-lane segments, 8 experts per lane, k = segment width
    (20000, 100, 6, 1, "f32", 200),   # 8 experts per lane, lanes past E idle
])
def test_routing_lane_mappings(orc, T, E, k, renorm, dtype, d):
    """Routing alone on the token and expert counts that select each lane
    mapping of the VALU routing kernel (d: an odd number of LDS chunks):
    logits and indices bit for bit, weights within the fp32 tolerance."""
    import torch

    import expert_top_router_amd as etr
    from expert_top_router_amd.layer import router_f32, to_device
    from tests.tolerance import assert_close

    cfg = W.LayerConfig("route_map", T=T, d=d, E=E, I=64, k=k, D=4, dtype=dtype,
                        renorm=renorm)
    inp = W.make_layer(cfg, seed=11)
    say(f"routing T={T} E={E} k={k} {dtype} d={d}")
    lg, idx, w = orc.route(inp.x, inp.w_router, k, renorm, dtype)
    dev = torch.device("cuda")
    x = to_device(inp.x)
    wr = to_device(router_f32(inp.w_router))
    g_idx = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    g_w = torch.zeros((T, k), dtype=torch.float32, device=dev)
    g_lg = torch.zeros((T, E), dtype=torch.float32, device=dev)
    etr.occ_route_topk(etr.desc_of(cfg), x, wr, g_idx, g_w, g_lg)
    torch.cuda.synchronize()
    assert np.array_equal(g_lg.cpu().numpy().view(np.uint32),
                          np.asarray(lg, np.float32).view(np.uint32))
    assert np.array_equal(g_idx.cpu().numpy(), idx)
    assert_close(g_w.cpu().numpy(), w, "f32", "topk_w")


@pytest.mark.parametrize("T,E,k,renorm,dtype,d,tie", [
    (16384, 128, 6, 0, "bf16", 128, False),   # two accumulators, two chunks
    (16383, 96, 16, 1, "bf16", 192, False),   # ragged last tile, k = row width
    (20000, 33, 1, 0, "bf16", 256, False),    # one accumulator, lanes past E idle
    (16500, 100, 8, 1, "f32", 96, False),     # fp32 tokens, 32-column chunks
    (16400, 40, 3, 0, "f32", 32, False),      # a single chunk
    (16384, 96, 6, 0, "bf16", 128, True),     # equal logits: lower index first
])
def test_routing_on_matrix_cores(orc, T, E, k, renorm, dtype, d, tie):
    """Routing at batches that run the logit chains as K = 1 MFMAs: logits
    and indices bit for bit against the in-order definition, weights within
    the fp32 tolerance; the call without a logits output picks the same."""
    import torch

    import expert_top_router_amd as etr
    from expert_top_router_amd.layer import router_f32, to_device
    from tests.tolerance import assert_close

    cfg = W.LayerConfig("route_mfma", T=T, d=d, E=E, I=64, k=k, D=4 if E % 4 == 0 else 3,
                        dtype=dtype, renorm=renorm)
    inp = W.make_layer(cfg, seed=13)
    wr_host = router_f32(inp.w_router)
    if tie:  # rows repeated in groups of 8: every logit has 7 equal twins
        wr_host = np.repeat(wr_host[::8], 8, axis=0)[:E].copy()
    say(f"routing on the matrix cores T={T} E={E} k={k} {dtype} d={d} tie={tie}")
    lg, idx, w = orc.route(inp.x, wr_host, k, renorm, dtype)
    dev = torch.device("cuda")
    x = to_device(inp.x)
    wr = to_device(wr_host)
    g_idx = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    g_w = torch.zeros((T, k), dtype=torch.float32, device=dev)
    g_lg = torch.zeros((T, E), dtype=torch.float32, device=dev)
    etr.occ_route_topk(etr.desc_of(cfg), x, wr, g_idx, g_w, g_lg)
    torch.cuda.synchronize()
    assert np.array_equal(g_lg.cpu().numpy().view(np.uint32),
                          np.asarray(lg, np.float32).view(np.uint32))
    assert np.array_equal(g_idx.cpu().numpy(), idx)
    assert_close(g_w.cpu().numpy(), w, "f32", "topk_w")
    n_idx = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    n_w = torch.zeros((T, k), dtype=torch.float32, device=dev)
    etr.occ_route_topk(etr.desc_of(cfg), x, wr, n_idx, n_w, None)
    torch.cuda.synchronize()
    assert torch.equal(n_idx, g_idx) and torch.equal(n_w, g_w)


@pytest.mark.parametrize("T,dtype,path", [
    (1000, "f32", "vector ALUs"),
    (16384, "f32", "matrix cores"),
    (16384, "bf16", "matrix cores"),
    (16384, "bf16", "candidate filter"),
])
def test_routing_special_values(orc, T, dtype, path):
    """Tokens with a NaN, a +inf or a -inf component, or components near the
    largest finite value (chains that overflow): NaN logits rank as -inf,
    ties go to the lower index, and every routing path picks the oracle's
    experts bit for bit; logits and weights match where finite and agree on
    NaN and infinity elsewhere (NaN payloads differ between the host and the
    GPU)."""
    import torch

    import expert_top_router_amd as etr
    from expert_top_router_amd.layer import router_f32, to_device

    E, k, d = 64, 4, 128
    cfg = W.LayerConfig("route_special", T=T, d=d, E=E, I=64, k=k, D=4, dtype=dtype)
    inp = W.make_layer(cfg, seed=17)
    x = W.to_f32(inp.x, dtype).astype(np.float64)
    rows = np.arange(64)
    x[rows, rows % d] = np.nan
    x[64 + rows, 3] = np.inf
    x[128 + rows, 5] = -np.inf
    x[192:256] = np.sign(x[192:256]) * 3.0e38
    x[256 + rows, 7] = np.inf
    x[256 + rows, 9] = -np.inf  # +inf and -inf terms: NaN chains
    inp.x = W.from_f64(x, dtype)
    wr_host = router_f32(inp.w_router)
    say(f"routing special values T={T} {dtype} on the {path}")
    lg, idx, w = orc.route(inp.x, wr_host, k, 0, dtype)
    dev = torch.device("cuda")
    g_idx = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    g_w = torch.zeros((T, k), dtype=torch.float32, device=dev)
    g_lg = None
    desc = etr.desc_of(cfg)
    if path == "candidate filter":
        nbytes = etr.occ_route_workspace_bytes(desc)
        assert nbytes > 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        etr.occ_route_topk_ws(desc, to_device(inp.x), to_device(wr_host), g_idx, g_w, ws, nbytes)
    else:
        g_lg = torch.zeros((T, E), dtype=torch.float32, device=dev)
        etr.occ_route_topk(desc, to_device(inp.x), to_device(wr_host), g_idx, g_w, g_lg)
    torch.cuda.synchronize()
    assert np.isnan(lg[:64]).all() and np.isnan(lg[256:320]).any()
    assert np.isinf(lg[64:192]).any() and np.isinf(lg[192:256]).any()
    assert np.array_equal(g_idx.cpu().numpy(), idx)

    def same(g, o, what):
        fin = np.isfinite(o)
        assert np.array_equal(np.isnan(g), np.isnan(o)), what
        assert np.array_equal(g[np.isinf(o)], o[np.isinf(o)]), what
        return fin

    if g_lg is not None:
        gl = g_lg.cpu().numpy()
        fin = same(gl, lg, "logits")
        assert np.array_equal(gl[fin].view(np.uint32), np.asarray(lg, np.float32)[fin].view(np.uint32))
    gw = g_w.cpu().numpy()
    fin = same(gw, w, "topk_w")
    assert np.all(np.abs(gw[fin] - w[fin]) <= 1e-4 * np.maximum(np.abs(w[fin]), 1e-30) + 1e-7)


def _filtered_route(cfg, inp):
    """occ_route_topk_ws on the layer's inputs: (indices, weights) on the host."""
    import torch

    import expert_top_router_amd as etr
    from expert_top_router_amd.layer import router_f32, to_device

    desc = etr.desc_of(cfg)
    nbytes = etr.occ_route_workspace_bytes(desc)
    assert nbytes > 0, "the candidate filter should apply to this layer"
    dev = torch.device("cuda")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    g_idx = torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, device=dev)
    g_w = torch.zeros((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    etr.occ_route_topk_ws(desc, to_device(inp.x), to_device(router_f32(inp.w_router)), g_idx, g_w,
                          ws, nbytes)
    torch.cuda.synchronize()
    return g_idx.cpu().numpy(), g_w.cpu().numpy()


@pytest.mark.parametrize("T,E,k,renorm", [
    # 32-token blocks below 32768 tokens, 128-token blocks from there
    (300, 33, 4, 0),      # 64 padded expert rows, ragged last block
    (1000, 64, 8, 1),
    (3001, 128, 16, 0),   # k at the candidate cap
    (20000, 100, 6, 1),
    (128, 128, 1, 0),     # whole blocks, top-1
    (1, 64, 4, 0),        # a single token
    (33, 33, 4, 1),       # a block of 32 and one token alone
    (40000, 96, 6, 1),    # 128-token blocks, ragged last block
])
def test_filtered_routing(orc, T, E, k, renorm):
    """Routing through the candidate filter (occ_route_topk_ws): the indices
    of the in-order definition bit for bit, the weights within the fp32
    tolerance (the softmax sum takes approximate logits for the experts
    outside the certified candidates)."""
    from tests.tolerance import assert_close

    cfg = W.LayerConfig("route_filter", T=T, d=256, E=E, I=64, k=k, D=1, dtype="bf16",
                        renorm=renorm, clusters=8)
    inp = W.make_layer(cfg, seed=12)
    say(f"filtered routing T={T} E={E} k={k} renorm={renorm}")
    _, idx, w = orc.route(inp.x, inp.w_router, k, renorm, "bf16")
    g_idx, g_w = _filtered_route(cfg, inp)
    assert np.array_equal(g_idx, idx)
    assert_close(g_w, w, "f32", "topk_w")


def test_filtered_routing_falls_back_on_ties(orc):
    """Router rows repeated in groups of 20: equal logits leave more than 16
    candidates for most tokens, so those blocks run every chain; the result
    is still the definition's, ties to the lower expert index."""
    from tests.tolerance import assert_close

    cfg = W.LayerConfig("route_ties", T=700, d=128, E=96, I=64, k=6, D=1, dtype="bf16",
                        renorm=0, clusters=4)
    inp = W.make_layer(cfg, seed=13)
    wr = np.array(inp.w_router)
    for e in range(cfg.E):
        wr[e] = wr[(e // 20) * 20]
    inp.w_router = wr
    say("filtered routing with tied router rows")
    _, idx, w = orc.route(inp.x, inp.w_router, cfg.k, 0, "bf16")
    g_idx, g_w = _filtered_route(cfg, inp)
    assert np.array_equal(g_idx, idx)
    assert_close(g_w, w, "f32", "topk_w")



def test_filtered_routing_fp32_router(orc):
    """A router that is not bf16-representable: the filter's bound takes the
    bf16 rounding residual of its rows, and the chains stream the fp32 rows."""
    from expert_top_router_amd.layer import router_f32
    from tests.tolerance import assert_close

    cfg = W.LayerConfig("route_f32r", T=1500, d=256, E=128, I=64, k=6, D=1, dtype="bf16",
                        renorm=0, clusters=8)
    inp = W.make_layer(cfg, seed=14)
    wr = router_f32(inp.w_router).copy()
    rng = np.random.default_rng(14)
    wr += (rng.standard_normal(wr.shape) * 1e-3 * np.abs(wr)).astype(np.float32)
    assert np.any((wr.view(np.uint32) & 0xffff) != 0)
    inp.w_router = wr
    say("filtered routing with an fp32 router")
    _, idx, w = orc.route(inp.x, inp.w_router, cfg.k, 0, "bf16")
    g_idx, g_w = _filtered_route(cfg, inp)
    assert np.array_equal(g_idx, idx)
    assert_close(g_w, w, "f32", "topk_w")

@pytest.mark.parametrize("name", ["olmoe_bf16", "dsv2lite_bf16", "stress_bf16"])
def test_full_size_filtered_routing(orc, name):
    """The benchmark layers' routing through the candidate filter against the
    oracle on the full batch."""
    from tests.tolerance import assert_close

    cfg = W.CONFIGS[name]
    inp = W.make_layer(cfg, seed=0, experts=False)
    say(f"full-size filtered routing {name}")
    _, idx, w = orc.route(inp.x, inp.w_router, cfg.k, cfg.renorm, cfg.dtype)
    g_idx, g_w = _filtered_route(cfg, inp)
    assert np.array_equal(g_idx, idx)
    assert_close(g_w, w, "f32", "topk_w")

def test_coactivation_accumulates(orc):
    import torch
    from expert_top_router_amd.layer import MoELayer, upload_inputs
    cfg = SMALL["bf16_ragged"]
    inp = W.make_layer(cfg, seed=6)
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert)
    say("case coactivation accumulate")
    lay.route()
    lay.coactivation(accumulate=0)
    lay.coactivation(accumulate=1)
    torch.cuda.synchronize()
    o = oracle_layer(orc, inp)
    assert np.array_equal(lay.host("counts"), 2 * o["coact"])


@pytest.mark.parametrize("name,budget,rescale", [
    ("bf16_ragged", 1, 1), ("bf16_ragged", 2, 0), ("bf16_ragged", 3, 1),
    ("bf16_e128_pairs", 2, 1), ("f32_e12", 1, 1), ("bf16_shared", 1, 1),
])
def test_pruned_layer_parity(orc, name, budget, rescale):
    """Collaboration pruning under an all-to-all budget: the pruned BRIMs and
    rescaled weights bit for bit, the layer (both strategies) by tolerance."""
    cfg = SMALL[name]
    say(f"case pruned {name} budget={budget} rescale={rescale}")
    inp = W.make_layer(cfg, seed=7)
    g = gpu_layer(inp, budget=budget, rescale=rescale)
    o = oracle_layer(orc, inp, budget=budget, rescale=rescale, w_route=g["topk_w"])
    assert o["brim"]["R"] < cfg.R  # pairs were dropped
    compare(g, o, inp)


def _pruned_end_to_end(orc, cfg, inp, budget, rescale, tokens_of=None):
    """The pruned layer with the oracle deciding from its own routing
    weights.  Tokens whose decision lies within the weights' rounding are
    certified (prune_decisions) and take the GPU's weights for the oracle's
    decision; every other token is pruned from the oracle's softmax."""
    g = gpu_layer(inp, budget=budget, rescale=rescale)
    o0 = oracle_layer(orc, W.LayerInputs(cfg, inp.x, inp.w_router, None, None, None, None,
                                         inp.slot_expert))
    assert np.array_equal(g["topk_idx"], o0["idx"]), "topk_idx"
    near, delta = prune_decisions(o0["idx"], o0["w"], g["topk_w"], g["brim0"], inp.slot_expert,
                                  cfg.E, cfg.D, budget)
    w_mix = o0["w"].copy()
    w_mix[near] = g["topk_w"][near]
    say(f"  {len(near)} of {cfg.T} tokens within delta={delta:.2e} of a tie: certified")
    tok = None
    if tokens_of is not None:
        ob = oracle_layer(orc, W.LayerInputs(cfg, inp.x, inp.w_router, None, None, None, None,
                                             inp.slot_expert), budget=budget, rescale=rescale,
                          w_route=w_mix)
        tok = tokens_of(ob["brim"])
    o = oracle_layer(orc, inp, tokens=tok, budget=budget, rescale=rescale, w_route=w_mix)
    assert o["brim"]["R"] < cfg.R  # pairs were dropped
    compare(g, o, inp, full=tok is None, pruned_w_exact=False)
    return o


@pytest.mark.parametrize("name,budget,rescale", [
    ("bf16_ragged", 1, 1), ("bf16_ragged", 2, 0), ("bf16_e128_pairs", 2, 1),
    ("f32_e12", 1, 1), ("bf16_shared", 1, 1),
])
def test_pruned_layer_end_to_end(orc, name, budget, rescale):
    """Collaboration pruning decided by the oracle from its own softmax
    weights (not the GPU's): BRIMs bit for bit, weights and layer outputs
    by tolerance; near-tie decisions certified."""
    cfg = SMALL[name]
    say(f"case pruned end to end {name} budget={budget} rescale={rescale}")
    _pruned_end_to_end(orc, cfg, W.make_layer(cfg, seed=7), budget, rescale)


def _two_layer_routing(orc, cfg, token_seed=None):
    """Oracle routing of a synthetic two-layer stack: the same clustered
    tokens through two independently drawn routers."""
    from tests.gpu_common import oracle_logits_parallel
    x = W.make_tokens(cfg, seed=0, token_seed=token_seed)
    out = []
    for layer in (0, 1):
        wr = W.make_router(cfg, seed=0, layer=layer)
        lg = oracle_logits_parallel(orc, x, wr, cfg.dtype)
        out.append(orc.topk(lg, cfg.k, cfg.renorm)[0])
    return out


@pytest.mark.parametrize("name", ["bf16_ragged", "bf16_e128_pairs", "olmoe_bf16"])
def test_cross_layer_affinity_parity(orc, name):
    """Cross-layer counts (calibration batch), predicted home devices and
    local hits (test batch), bit for bit against the oracle."""
    import torch
    import expert_top_router_amd as occ
    cfg = SMALL[name] if name in SMALL else W.CONFIGS[name]
    say(f"case affinity {name}")
    c1, c2 = _two_layer_routing(orc, cfg, token_seed=1)
    i1, i2 = _two_layer_routing(orc, cfg)
    T, E, k, D = cfg.T, cfg.E, cfg.k, cfg.D
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    A = torch.empty((E, E), dtype=torch.int32, device="cuda")
    occ.occ_cross_coactivation(T, k, E, dev(c1), k, E, dev(c2), A, accumulate=0)
    occ.occ_cross_coactivation(T, k, E, dev(c1), k, E, dev(c2), A, accumulate=1)
    torch.cuda.synchronize()
    A_o = orc.cross_coactivation(c1, E, c2, E)
    assert np.array_equal(A.cpu().numpy(), 2 * A_o), "cross-layer counts (accumulated twice)"
    occ.occ_cross_coactivation(T, k, E, dev(c1), k, E, dev(c2), A, accumulate=0)
    se2 = np.random.default_rng(12).permutation(E).astype(np.int32)
    home = torch.empty(T, dtype=torch.int32, device="cuda")
    occ.occ_home_device(T, k, E, dev(i1), E, D, se2, A, home)
    torch.cuda.synchronize()
    home_o = orc.home_device(i1, E, A_o, se2, D)
    assert np.array_equal(home.cpu().numpy(), home_o), "home devices"
    hits = torch.empty(1, dtype=torch.int32, device="cuda")
    shard = dev((np.arange(T) * D // T).astype(np.int32))
    for h_dev, h_host in [(home, home_o), (shard, shard.cpu().numpy())]:
        occ.occ_local_hits(T, k, E, dev(i2), D, se2, h_dev, hits)
        torch.cuda.synchronize()
        assert int(hits.cpu()[0]) == orc.local_hits(i2, E, se2, D, h_host), "local hits"
    say(f"  local share: predicted {orc.local_hits(i2, E, se2, D, home_o) / (T * k):.3f}, "
        f"sharded {orc.local_hits(i2, E, se2, D, shard.cpu().numpy()) / (T * k):.3f}")


FULL = ["tiny_fp32", "olmoe_bf16", "mixtral_bf16", "dsv2lite_bf16", "stress_bf16"]


def _sample_tokens(cfg, b, n=48, seed=11):
    rng = np.random.default_rng(seed)
    tok = set(rng.choice(cfg.T, size=min(n, cfg.T), replace=False).tolist())
    tok |= {0, cfg.T - 1}
    # the tokens of the least-loaded non-empty slot (a ragged tile)
    cnt = np.diff(b["slot_offset"])
    g = int(np.argmin(np.where(cnt > 0, cnt, cnt.max() + 1)))
    seg = b["epd_token"][b["slot_offset"][g]:b["slot_offset"][g + 1]]
    tok |= set(seg[:16].tolist())
    return np.array(sorted(tok), dtype=np.int32)


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer_parity(orc, name):
    """Full batch for routing, BRIMs, dispatch and co-activation; sampled
    tokens (and all of their EPD/SFD rows) for the expert arithmetic."""
    cfg = W.CONFIGS[name]
    say(f"case full {name}: generating inputs")
    inp = W.make_layer(cfg, seed=0)
    o_route = oracle_layer(orc, W.LayerInputs(cfg, inp.x, inp.w_router, None, None, None, None,
                                              inp.slot_expert))
    tok = _sample_tokens(cfg, o_route["brim"])
    say(f"case full {name}: oracle on {tok.size} tokens")
    o = oracle_layer(orc, inp, tokens=tok)
    g = gpu_layer(inp)
    compare(g, o, inp, full=False)
    say(f"case full {name}: S={o['brim']['S']} of T*k={cfg.R}")


def test_full_size_pruned_layer_parity(orc):
    """The OLMoE-shaped layer under a budget of 2 of its 8 devices."""
    cfg = W.CONFIGS["olmoe_bf16"]
    say("case full pruned olmoe_bf16 budget=2: generating inputs")
    inp = W.make_layer(cfg, seed=0)
    g = gpu_layer(inp, budget=2)
    o_route = oracle_layer(orc, W.LayerInputs(cfg, inp.x, inp.w_router, None, None, None, None,
                                              inp.slot_expert), budget=2, w_route=g["topk_w"])
    tok = _sample_tokens(cfg, o_route["brim"])
    o = oracle_layer(orc, inp, tokens=tok, budget=2, w_route=g["topk_w"])
    compare(g, o, inp, full=False)
    say(f"case full pruned: S={o['brim']['S']}, R'={o['brim']['R']} of T*k={cfg.R}")


def test_full_size_pruned_layer_end_to_end(orc):
    """The OLMoE-shaped layer under a budget of 2 of its 8 devices, pruned by
    the oracle from its own softmax weights (near ties certified)."""
    cfg = W.CONFIGS["olmoe_bf16"]
    say("case full pruned end to end olmoe_bf16 budget=2: generating inputs")
    inp = W.make_layer(cfg, seed=0)
    o = _pruned_end_to_end(orc, cfg, inp, 2, 1, tokens_of=lambda b: _sample_tokens(cfg, b))
    say(f"case full pruned end to end: S={o['brim']['S']}, R'={o['brim']['R']} of T*k={cfg.R}")


def test_full_size_correlated_placement(orc):
    """The DeepSeek-V2-Lite-shaped layer under correlated placement, run end
    to end by the product: a calibration batch (token seed 1) through
    occ_route_topk and occ_coactivation, occ_place_greedy on those counts,
    then the layer on the seed-0 batch with that placement.  Counts and
    placement bit for bit against the oracle's own chain; S, BRIMs and the
    dispatch bit for bit, the outputs by tolerance; Y within tolerance of
    the contiguous-placement run (placement moves no arithmetic but the
    order of the per-device sums)."""
    import torch
    import expert_top_router_amd as occ
    from expert_top_router_amd.layer import MoELayer, upload_inputs
    from tests.gpu_common import oracle_logits_parallel
    from tests.tolerance import assert_close
    cfg = W.CONFIGS["dsv2lite_bf16"]
    say("case correlated placement dsv2lite_bf16: calibration batch")
    cal = W.make_layer(cfg, seed=0, token_seed=1, experts=False)
    lay = MoELayer(cfg, upload_inputs(cal), cal.slot_expert)
    lay.route()
    lay.coactivation()
    torch.cuda.synchronize()
    counts = lay.host("counts")
    del lay
    se = occ.occ_place_greedy(cfg.E, cfg.D, counts)
    idx_c, _ = orc.topk(oracle_logits_parallel(orc, cal.x, cal.w_router, cfg.dtype), cfg.k,
                        cfg.renorm)
    C_o = orc.coactivation(idx_c, cfg.E)
    assert np.array_equal(counts, C_o), "calibration co-activation counts"
    assert np.array_equal(se, orc.greedy_placement(C_o, cfg.D)), "greedy placement"
    assert not np.array_equal(se, np.arange(cfg.E)), "the placement moved experts"
    say("case correlated placement dsv2lite_bf16: layer with the greedy placement")
    inp = W.make_layer(cfg, seed=0)
    contiguous = inp.slot_expert.copy()
    inp.slot_expert = np.asarray(se, dtype=np.int32)
    o_route = oracle_layer(orc, W.LayerInputs(cfg, inp.x, inp.w_router, None, None, None, None,
                                              inp.slot_expert))
    tok = _sample_tokens(cfg, o_route["brim"])
    o = oracle_layer(orc, inp, tokens=tok)
    g = gpu_layer(inp)
    compare(g, o, inp, full=False)
    inp.slot_expert = contiguous
    g_c = gpu_layer(inp)
    S_c = int(g_c["S"][0])
    b_c = orc.brim(o["idx"], o["w"], contiguous, cfg.E, cfg.D)
    assert S_c == b_c["S"], "S under contiguous placement"
    assert_close(W.to_f32(g["y"], cfg.dtype), W.to_f32(g_c["y"], cfg.dtype), cfg.dtype,
                 "y (greedy vs contiguous placement)")
    intra_g = orc.intra_share(C_o, se, cfg.D)
    intra_c = orc.intra_share(C_o, contiguous, cfg.D)
    say(f"case correlated placement: S/(T*k) greedy {o['brim']['S'] / cfg.R:.3f} "
        f"({o['brim']['S']}), contiguous {S_c / cfg.R:.3f} ({S_c}); intra-device share of "
        f"co-selections {intra_g[0] / max(intra_g[1], 1):.3f} vs "
        f"{intra_c[0] / max(intra_c[1], 1):.3f}")
    assert o["brim"]["S"] < S_c, "correlated placement sends fewer rows"
