"""The seeded workloads have the structure their recipe states."""
import math

import numpy as np

import workloads as W
from tests.calibrate_stress_alpha import share_for, top_pair_share


def test_stress_router_skew_holds_on_other_tokens(orc):
    """Top 1% of expert pairs carry about 40% of co-selections (Expert
    Coupling, Abstract: 0.8% of pairs / 42% of tokens at top-2), checked on
    tokens the calibration did not see."""
    cfg = W.CONFIGS["stress_bf16"]
    assert cfg.alpha > 0
    x = W.make_tokens(cfg, T=16384)[8192:]
    share = share_for(cfg, x, cfg.alpha)
    assert abs(share - 0.40) < 0.015, share
    # and the unskewed router is far from it
    assert share_for(cfg, x[:2048], 0.0) < 0.2


def test_top_pair_share_counts_pairs_once():
    E, k = 16, 3
    Cm = np.zeros((E, E), np.int64)
    Cm[0, 1] = Cm[1, 0] = 30  # 30 tokens chose experts 0 and 1 together
    share = top_pair_share(Cm, k, n_tok=10)
    assert math.ceil(0.01 * E * (E - 1) / 2) == 2
    assert share == 30 / (10 * 3)


def test_cluster_tokens_sit_near_their_centres():
    cfg = W.CONFIGS["olmoe_bf16"]
    x = W.to_f32(W.make_tokens(cfg, T=512), "bf16").astype(np.float64)
    c = W.cluster_centres(cfg)
    dist = ((x[:, None, :] - c[None]) ** 2).sum(-1)  # [T, clusters]
    nearest = np.sort(dist, axis=1)
    # spread 0.3 per coordinate: ~0.09 d to the own centre, ~2 d to others
    assert np.all(nearest[:, 0] < 0.2 * cfg.d)
    assert np.all(nearest[:, 1] > 1.0 * cfg.d)


def test_weights_have_the_stated_variance():
    cfg = W.CONFIGS["olmoe_bf16"]
    wr = W.to_f32(W.make_router(cfg), "bf16")
    assert abs(wr.var() * cfg.d - 1.0) < 0.02
