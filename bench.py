"""Benchmark of the collaboration-aware MoE layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one forward pass of the whole layer over one batch: routing and
top-k, BRIM build, dispatch ORI -> SFD -> EPD, the grouped SwiGLU experts and
the pre-reduction + combine back to ORI, issued back to back on one stream
with every input already resident in HBM.  The default workload is the
OLMoE-shaped layer (T=4096, d=2048, E=64, I=1024, top-8, 8 logical devices,
clustered tokens).  Prints one JSON line.

The roofline object describes the dominant kernel (the gate/up GEMM with the
SwiGLU epilogue): achieved = algorithmic flops per launch / its mean launch
time from HIP events on the stream it runs on.  cpu_baseline times the CPU
oracle (single thread) on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "MoE-layer tokens/sec (route+dispatch+FFN+combine); % HBM and % MFMA peak"
DEFAULT_WORKLOAD = "olmoe_bf16"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", default=DEFAULT_WORKLOAD)
    p.add_argument("--placement", default="contiguous", choices=["contiguous", "greedy"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=192)
    p.add_argument("--profile-steps", type=int, default=0,
                   help="only run this many forward steps (for rocprofv3), print nothing else")
    return p.parse_args()


def elem_bytes(cfg):
    return 2 if cfg.dtype == "bf16" else 4


def algorithmic(cfg, S):
    """Per-launch algorithmic work of each stage (bytes or flops)."""
    T, d, E, k, D, I = cfg.T, cfg.d, cfg.E, cfg.k, cfg.D, cfg.I
    L, R, b = E // D, T * k, elem_bytes(cfg)
    nsh, Ish = cfg.n_shared, cfg.I_shared
    return {
        "route_flop": 2.0 * T * d * E,
        "route_bytes": T * d * b + E * d * b + 8.0 * T * k,
        "brim_bytes": 8.0 * T * k + 4.0 * D * T + 4.0 * L * S + 4.0 * S + 12.0 * R,
        "dispatch_bytes": (T + S + R) * d * b + 4.0 * D * T + 4.0 * L * S + 4.0 * R,
        "up_flop": 4.0 * R * d * I + 4.0 * T * d * Ish * nsh,
        "down_flop": 2.0 * R * d * I + 2.0 * T * d * Ish * nsh,
        "combine_bytes": (R + S + T + (T if nsh else 0)) * d * b + 4.0 * D * T + 4.0 * L * S
                         + 8.0 * R,
    }


def time_calls(fn, n, torch):
    """Mean duration (s) of fn() over n back-to-back calls, HIP events on the
    current stream (the one the library launches on)."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(n):
        fn()
    stop.record()
    stop.synchronize()
    return start.elapsed_time(stop) / 1e3 / n


def cpu_baseline(inp, n_tok):
    """The oracle as it stands, one thread: routing and BRIMs on the full
    batch, expert FFN and combine on a seeded sample of tokens; tokens/s
    extrapolated linearly from the per-token cost of each part."""
    import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build()
    cfg = inp.cfg
    T, E, k, D, d = cfg.T, cfg.E, cfg.k, cfg.D, cfg.d
    L = E // D
    t0 = time.perf_counter()
    lg = oracle.logits(inp.x, inp.w_router, cfg.dtype)
    idx, w = oracle.topk(lg, k, cfg.renorm)
    b = oracle.brim(idx, w, inp.slot_expert, E, D)
    sfd = oracle.gather(inp.x, b["sfd_token"][:b["S"]])
    oracle.gather(sfd, b["epd_sfd"])
    t_full = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    tok = np.sort(rng.choice(T, size=min(n_tok, T), replace=False)).astype(np.int32)
    t1 = time.perf_counter()
    rows = []
    for dv in range(D):
        s = b["brim0"][dv, tok]
        s = s[s >= 0]
        for l in range(L):
            r = b["brim1"][l, s]
            rows.append(r[r >= 0])
    rows = np.sort(np.concatenate(rows)).astype(np.int64)
    ex_of_slot = np.repeat(np.asarray(inp.slot_expert), np.diff(b["slot_offset"]))
    out = oracle.expert_rows(inp.x, b["epd_token"][rows], ex_of_slot[rows], inp.w_gate_up,
                             inp.w_down, cfg.dtype)
    epd_row = np.full(T * k, -1, np.int32)
    epd_row[rows] = np.arange(rows.size, dtype=np.int32)
    shared = None
    if cfg.n_shared:
        shared = oracle.shared_rows(inp.x, tok, inp.w_gate_up_sh, inp.w_down_sh, cfg.dtype)
    oracle.combine(tok, b, T, D, L, d, cfg.dtype, out, epd_row, shared)
    t_sample = time.perf_counter() - t1
    per_token = t_full / T + t_sample / tok.size
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": (f"routing, BRIMs and gathers on all {T} tokens ({t_full:.2f} s); "
                       f"expert FFN and combine on {tok.size} seeded tokens with all their "
                       f"{rows.size} EPD rows ({t_sample:.2f} s); tokens/s = 1 / (full-batch "
                       f"time / T + sample time / sample tokens), one thread")}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: this layer step runs on one GPU, with the expert-"
              "parallel devices as logical partitions of its buffers; --gpus must be 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from expert_top_router_amd.layer import MoELayer, upload_inputs

    cfg = W.CONFIGS[args.config]
    inp = W.make_layer(cfg, seed=0)
    if args.placement == "greedy":
        # correlated placement from a calibration batch (token seed 1)
        import expert_top_router_amd as occ
        cal = W.make_layer(cfg, seed=0, token_seed=1, experts=False)
        lay_cal = MoELayer(cfg, upload_inputs(W.LayerInputs(cfg, cal.x, cal.w_router, None, None,
                                                            None, None, cal.slot_expert)),
                           cal.slot_expert)
        lay_cal.route()
        lay_cal.coactivation()
        torch.cuda.synchronize()
        inp.slot_expert = occ.occ_place_greedy(cfg.E, cfg.D, lay_cal.host("counts"))
        del lay_cal
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert)
    torch.cuda.synchronize()

    if args.profile_steps:
        for _ in range(args.profile_steps):
            lay.forward()
            lay.coactivation()
        torch.cuda.synchronize()
        print(f"profiled {args.profile_steps} steps of {cfg.name}", flush=True)
        return

    for _ in range(args.warmup):
        lay.forward()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        lay.forward()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = cfg.T * args.steps / elapsed

    # per-stage mean launch times (inputs of each stage are valid from the last forward)
    n = max(10, min(args.steps, 50))
    S = int(lay.host("S")[0])
    alg = algorithmic(cfg, S)
    t = {
        "route": time_calls(lay.route, n, torch),
        "build_brim": time_calls(lay.build_brim, n, torch),
        "dispatch": time_calls(lay.dispatch, n, torch),
        "expert_up": time_calls(lay.expert_up, n, torch),
        "expert_down": time_calls(lay.expert_down, n, torch),
        "combine": time_calls(lay.combine, n, torch),
        "coactivation": time_calls(lay.coactivation, n, torch),
    }
    lay.forward()
    torch.cuda.synchronize()
    peak_mfma = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    up_tf = alg["up_flop"] / t["expert_up"] / 1e12
    stages = {
        "route_us": t["route"] * 1e6,
        "route_valu_frac": alg["route_flop"] / t["route"] / 1e12 / 78.6,
        "build_brim_us": t["build_brim"] * 1e6,
        "dispatch_us": t["dispatch"] * 1e6,
        "dispatch_hbm_frac": alg["dispatch_bytes"] / t["dispatch"] / 1e9 / PEAK_HBM_GBS,
        "expert_up_us": t["expert_up"] * 1e6,
        "expert_up_mfma_frac": up_tf / peak_mfma,
        "expert_down_us": t["expert_down"] * 1e6,
        "expert_down_mfma_frac": alg["down_flop"] / t["expert_down"] / 1e12 / peak_mfma,
        "combine_us": t["combine"] * 1e6,
        "combine_hbm_frac": alg["combine_bytes"] / t["combine"] / 1e9 / PEAK_HBM_GBS,
        "coactivation_us": t["coactivation"] * 1e6,
    }
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian-mixture tokens, random-init router and experts)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "I": cfg.I,
                   "k": cfg.k, "D": cfg.D, "n_shared": cfg.n_shared, "I_shared": cfg.I_shared,
                   "placement": args.placement, "sfd_rows": S, "epd_rows": cfg.R,
                   "sfd_over_tk": S / max(cfg.R, 1)},
        "roofline": {"kernel": "gemm_bf16_kernel<128,128,SwiGLU> (occ_expert_up)",
                     "bound": "mfma", "achieved": up_tf, "peak": peak_mfma, "unit": "TFLOP/s",
                     "frac": up_tf / peak_mfma, "traffic": None,
                     "launch_us": t["expert_up"] * 1e6,
                     "flop_per_launch": alg["up_flop"]},
        "stages": stages,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
