"""Calibrate the router skew of the large top-6 stress workload.

    python tests/calibrate_stress_alpha.py      (writes workloads/stress_alpha.json)

Expert Coupling in MoE Pretraining (Abstract) reports that at top-2, 0.8% of
the expert pairs of a layer are selected together by 42% of tokens.  The
stress workload mirrors that concentration at top-6: the skew strength alpha
is chosen by bisection so that the top ceil(1% of C(E, 2)) expert pairs carry
40% of all co-selection events (each token contributes C(k, 2) events), with
routing computed by the oracle on the first 8192 tokens of the seed-0 batch.
The workload generator only reads the frozen value.
"""
import concurrent.futures as cf
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

TARGET = 0.40
N_TOKENS = 8192


def top_pair_share(Cm, k, n_tok):
    """Share of co-selection events carried by the top 1% of expert pairs."""
    E = Cm.shape[0]
    iu = np.triu_indices(E, 1)
    pairs = np.sort(Cm[iu])[::-1]
    n_top = math.ceil(0.01 * E * (E - 1) / 2)
    return pairs[:n_top].sum() / (n_tok * k * (k - 1) / 2)


def share_for(cfg, x, alpha, workers=8):
    wr = W.make_router(cfg, alpha=alpha)
    parts = np.array_split(np.arange(x.shape[0]), workers)
    with cf.ThreadPoolExecutor(workers) as ex:
        lg = np.concatenate(list(ex.map(lambda p: oracle.logits(x[p], wr), parts)))
    idx, _ = oracle.topk(lg, cfg.k, cfg.renorm)
    return top_pair_share(oracle.coactivation(idx, cfg.E), cfg.k, x.shape[0])


def main():
    cfg = W.CONFIGS["stress_bf16"]
    x = W.make_tokens(cfg, T=N_TOKENS)
    lo, hi = 0.0, 64.0
    assert share_for(cfg, x, hi) > TARGET
    for _ in range(18):
        mid = 0.5 * (lo + hi)
        if share_for(cfg, x, mid) < TARGET:
            lo = mid
        else:
            hi = mid
    alpha = round(0.5 * (lo + hi), 4)
    share = share_for(cfg, x, alpha)
    out = {"alpha": alpha, "top_1pct_pair_share": round(float(share), 4),
           "tokens": N_TOKENS, "target": TARGET,
           "written_by": "tests/calibrate_stress_alpha.py"}
    with open(os.path.join(ROOT, "workloads", "stress_alpha.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()
