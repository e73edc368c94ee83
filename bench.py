"""Benchmark of the collaboration-aware MoE layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one forward pass of the whole layer over one batch: routing and
top-k, BRIM build, dispatch ORI -> SFD -> EPD, the grouped SwiGLU experts and
the pre-reduction + combine back to ORI, issued back to back on one stream
with every input already resident in HBM.  The default workload is the
largest single-GPU layer of the suite, the skewed top-6 stress layer
(T=65536, d=2048, E=128, I=768, 16 logical devices, 64 token clusters, a
router skewed toward 14 hot expert groups).  Prints one JSON line.

The roofline object describes the dominant kernel (the gate/up GEMM with the
SwiGLU epilogue): achieved = algorithmic flops per launch / its mean launch
time, from HIP events recorded around it in every timed step on the stream
it runs on.  The per-stage times come from a second pass of the same steps
with an event between every two stages; step_breakdown sets their sum
against the wall time per step and gives the step replayed from a HIP
graph.  cpu_baseline times the CPU oracle (single thread) on a bounded
sample of the same workload.  After the headline steps the line also
carries the widened rows (conventional, pruned, affinity, backward), a
calibration (the vendor library's dense bf16 matmul with the gate/up GEMM's
flop on the same box: context for the roofline fraction, not part of any
measured step) and, under "workloads", the other bf16 layers (the
DeepSeek-V2-Lite-shaped one under contiguous and correlated placement).
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
# fp32 peak as published, vector and matrix alike (256 CU x 4 SIMD x 32 FMA x 2 flop x
# 2.4 GHz): the fp32 layers' expert GEMMs, the routing chains (plain v_fmac_f32 reaches
# it without packed math once two waves share a SIMD, and so does the K = 1 fp32 MFMA
# that routing uses at large batches) and the router backward's fp32 MFMA products
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "MoE-layer tokens/sec (route+dispatch+FFN+combine); % HBM and % MFMA peak"
DEFAULT_WORKLOAD = "stress_bf16"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", default=DEFAULT_WORKLOAD)
    p.add_argument("--placement", default="contiguous", choices=["contiguous", "greedy"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-others", action="store_true",
                   help="skip the secondary workloads (the other bf16 layers)")
    p.add_argument("--cpu-route-tokens", type=int, default=4096,
                   help="oracle baseline: tokens of the sub-batch routed and re-indexed")
    p.add_argument("--cpu-sample-tokens", type=int, default=768,
                   help="oracle baseline: tokens whose expert FFN and combine are timed")
    p.add_argument("--profile-steps", type=int, default=0,
                   help="only run this many forward steps (for rocprofv3), print nothing else")
    p.add_argument("--profile-backward", action="store_true",
                   help="with --profile-steps: run the backward after every forward step")
    p.add_argument("--copy-calibration", action="store_true",
                   help="with --profile-steps: first copy 256 MiB twice (counter scale factors)")
    return p.parse_args()


def elem_bytes(cfg):
    return 2 if cfg.dtype == "bf16" else 4


def route_unit(cfg) -> str:
    """Where occ_route_topk runs every chain (the library's choice, restated
    for the report): the matrix cores from 16384 tokens for routers of 33..128
    experts when d is a whole number of chunks, else the vector ALUs."""
    jc = 64 if cfg.dtype == "bf16" else 32
    mfma = 32 < cfg.E <= 128 and cfg.k <= 16 and cfg.d % jc == 0 and cfg.T >= 16384
    return "every chain, matrix cores" if mfma else "every chain, vector ALUs"


def algorithmic(cfg, S):
    """Per-launch algorithmic work of each stage (bytes or flops)."""
    T, d, E, k, D, I = cfg.T, cfg.d, cfg.E, cfg.k, cfg.D, cfg.I
    L, R, b = E // D, T * k, elem_bytes(cfg)
    nsh, Ish = cfg.n_shared, cfg.I_shared
    return {
        "route_flop": 2.0 * T * d * E,
        "route_bytes": T * d * b + E * d * 4.0 + 8.0 * T * k,  # the router is fp32
        "brim_bytes": 8.0 * T * k + 4.0 * D * T + 4.0 * L * S + 4.0 * S + 12.0 * R,
        "dispatch_bytes": (T + S + R) * d * b + 4.0 * D * T + 4.0 * L * S + 4.0 * R,
        "up_flop": 4.0 * R * d * I + 4.0 * T * d * Ish * nsh,
        "down_flop": 2.0 * R * d * I + 2.0 * T * d * Ish * nsh,
        "combine_bytes": (R + S + T + (T if nsh else 0)) * d * b + 4.0 * D * T + 4.0 * L * S
                         + 8.0 * R,
    }


def gemm_source_sha256():
    """Hash of the forward GEMM's sources (kernel file and shared header)."""
    import hashlib
    csrc = os.path.join(ROOT, "expert_top_router_amd", "csrc")
    h = hashlib.sha256()
    for name in ("occ_gemm.hip", "occ_gemm_common.h"):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def measured_traffic(cfg):
    """HBM bytes per launch of the gate/up GEMM from the committed counter
    summary (two rocprofv3 --pmc passes, scaled by a plain copy), or None when
    the workload differs or the GEMM source changed since they were taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{cfg.name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    h = re.search(r"gemm_source_sha256: ([0-9a-f]+)", text)
    if not m or not h or gemm_source_sha256() != h.group(1):
        return None
    return int(m.group(1))


STAGES = ("route", "build_brim", "dispatch", "expert_up", "expert_down", "combine")


def step(lay, marks=None):
    """One forward step of the layer, stage by stage (occ_expert_ffn split
    into its two launches).  With marks (a list of len(STAGES) + 1 events)
    an event is recorded on the launch stream before every stage and after
    the last one."""
    for i, name in enumerate(STAGES):
        if marks is not None:
            marks[i].record()
        getattr(lay, name)()
    if marks is not None:
        marks[-1].record()


DIRECT_STAGES = ("route", "build_brim", "dispatch_direct", "expert_up", "expert_down",
                 "combine_direct")


def conventional(lay, cfg, steps, torch):
    """The conventional per-(token, expert) strategy (Occult, Figure 2) on
    the same BRIMs: EPD straight from ORI, combine with no pre-reduction.
    Times K whole steps, then each stage with events between stages, and
    states the rows and bytes each strategy would send between devices."""
    for _ in range(3):
        for name in DIRECT_STAGES:
            getattr(lay, name)()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for name in DIRECT_STAGES:
            getattr(lay, name)()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    n = max(10, min(steps, 50))
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(DIRECT_STAGES) + 1)]
             for _ in range(n)]
    for i in range(n):
        for j, name in enumerate(DIRECT_STAGES):
            marks[i][j].record()
            getattr(lay, name)()
        marks[i][-1].record()
    torch.cuda.synchronize()
    t = {name: float(np.mean([m[j].elapsed_time(m[j + 1]) for m in marks])) * 1e3
         for j, name in enumerate(DIRECT_STAGES)}
    S = int(lay.host("S")[0])
    rowb = cfg.d * elem_bytes(cfg)
    return {"ms_per_step": elapsed / steps * 1e3, "tokens_per_s": cfg.T * steps / elapsed,
            "dispatch_us": t["dispatch_direct"], "combine_us": t["combine_direct"],
            "rows_sent": cfg.R, "occult_rows_sent": S, "row_saving": 1.0 - S / max(cfg.R, 1),
            "send_bytes": cfg.R * rowb, "occult_send_bytes": S * rowb}


def pruned(cfg, weights, slot_expert, budget, steps, torch):
    """The layer under collaboration pruning with an all-to-all budget of
    `budget` devices per token (kept weights rescaled): rows that would be
    sent and the step time."""
    from expert_top_router_amd.layer import MoELayer
    lay = MoELayer(cfg, weights, slot_expert, budget=budget, rescale=1)
    for _ in range(3):
        step(lay)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(lay)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    S = int(lay.host("S")[0])
    Rp = int(lay.host("slot_offset")[cfg.E])
    del lay
    return {"budget": budget, "rescale": 1, "sfd_rows": S, "epd_rows": Rp,
            "sfd_over_tk": S / max(cfg.R, 1), "ms_per_step": elapsed / steps * 1e3,
            "tokens_per_s": cfg.T * steps / elapsed}


def affinity(cfg, lay, torch):
    """Cross-layer affinity on a synthetic two-layer stack (the layer's tokens
    through a second, independently drawn router): counts from a calibration
    batch (token seed 1), then the share of the next layer's assignments
    served on the token's device, for plain sharding (t * D / T) and for the
    predicted home devices, and the time of each call."""
    import expert_top_router_amd as occ
    import workloads as W
    from expert_top_router_amd.layer import router_f32, to_device
    T, E, k, D = cfg.T, cfg.E, cfg.k, cfg.D
    dsc = occ.desc_of(cfg)
    routers = [to_device(router_f32(W.make_router(cfg, seed=0, layer=l))) for l in (0, 1)]
    batches = [lay.w.x, to_device(W.make_tokens(cfg, seed=0, token_seed=1))]
    idx = {}
    for b, xb in enumerate(batches):
        for l in (0, 1):
            i = torch.empty((T, k), dtype=torch.int32, device="cuda")
            wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
            occ.occ_route_topk(dsc, xb, routers[l], i, wt)
            idx[(b, l)] = i
    A = torch.empty((E, E), dtype=torch.int32, device="cuda")
    home = torch.empty(T, dtype=torch.int32, device="cuda")
    hits = torch.empty(1, dtype=torch.int32, device="cuda")
    shard = (torch.arange(T, device="cuda", dtype=torch.int64) * D // T).to(torch.int32)
    se2 = np.asarray(W.contiguous_placement(cfg), dtype=np.int32)
    calls = {
        "cross_coactivation": lambda: occ.occ_cross_coactivation(T, k, E, idx[(1, 0)], k, E,
                                                                 idx[(1, 1)], A),
        "home_device": lambda: occ.occ_home_device(T, k, E, idx[(0, 0)], E, D, se2, A, home),
        "local_hits": lambda: occ.occ_local_hits(T, k, E, idx[(0, 1)], D, se2, home, hits),
    }
    us = {}
    for name, fn in calls.items():
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(10):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        us[name + "_us"] = ev[0].elapsed_time(ev[1]) * 1e3 / 10
    predicted = int(hits.cpu()[0])
    occ.occ_local_hits(T, k, E, idx[(0, 1)], D, se2, shard, hits)
    torch.cuda.synchronize()
    sharded = int(hits.cpu()[0])
    return {"layers": 2, "calibration": "token seed 1", "placement": "contiguous",
            "sharded_local_share": sharded / (T * k), "predicted_local_share": predicted / (T * k),
            **us}


BACKWARD_STAGES = ("grad_combine", "expert_backward", "router_backward", "shared_backward",
                   "grad_dispatch")


def backward(lay, cfg, steps, torch):
    """Forward + backward step (bf16 layers): the backward walks the BRIMs in
    reverse (grad-combine, expert backward GEMMs, router gradient, the shared
    experts' backward when there are any, grad-dispatch) for a seeded
    upstream gradient.  Times K whole steps, then each backward stage with
    events between stages; without shared experts also the step that keeps
    the experts' pre-activations."""
    lay.prepare_backward()
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    lay.dy.copy_(torch.randn(lay.dy.shape, generator=g, device="cuda").to(lay.dy.dtype))

    def fwd_bwd(marks=None):
        step(lay)
        for j, name in enumerate(BACKWARD_STAGES):
            if marks is not None:
                marks[j].record()
            getattr(lay, name)()
        if marks is not None:
            marks[-1].record()

    for _ in range(3):
        fwd_bwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd_bwd()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    n = max(10, min(steps, 50))
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(BACKWARD_STAGES) + 1)]
             for _ in range(n)]
    for i in range(n):
        fwd_bwd(marks[i])
    torch.cuda.synchronize()
    t = {name: float(np.mean([m[j].elapsed_time(m[j + 1]) for m in marks])) / 1e3
         for j, name in enumerate(BACKWARD_STAGES)}
    S = int(lay.host("S")[0])
    T, d, E, I, R, b = cfg.T, cfg.d, cfg.E, cfg.I, cfg.R, elem_bytes(cfg)
    # expert backward: G/U recompute (2I), dh (I), d_epd (2I), dW_down (I), dW_gate_up (2I)
    ebw_flop = 2.0 * R * d * 8 * I
    gc_bytes = (T + S + 2 * R) * d * b + 4.0 * R + 4.0 * cfg.D * T + 4.0 * (E // cfg.D) * S
    gd_bytes = (R + S + T) * d * b + 4.0 * T * d + 4.0 * cfg.D * T + 4.0 * (E // cfg.D) * S
    rb_flop = 4.0 * T * E * d
    # shared experts: [G | U] 4, dh 2, dW_down 2, dW_gate_up 4, dx 4 (units of T d I_sh n_sh)
    sh_flop = 16.0 * T * d * cfg.I_shared * cfg.n_shared
    out = {"ms_per_step": elapsed / steps * 1e3, "tokens_per_s": T * steps / elapsed}
    if cfg.n_shared == 0:
        # the same step with the forward keeping [G | U] for the expert backward
        def fwd_bwd_kept():
            lay.forward_keep()
            lay.backward_kept()

        for _ in range(3):
            fwd_bwd_kept()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fwd_bwd_kept()
        torch.cuda.synchronize()
        kept = time.perf_counter() - t0
        out.update(kept_gu_ms_per_step=kept / steps * 1e3,
                   kept_gu_tokens_per_s=T * steps / kept)
    else:
        out.update(shared_backward_us=t["shared_backward"] * 1e6, shared_backward_flop=sh_flop,
                   shared_backward_mfma_frac=sh_flop / t["shared_backward"] / 1e12
                   / PEAK_BF16_TFLOPS)
    return {**out,
            "grad_combine_us": t["grad_combine"] * 1e6,
            "grad_combine_hbm_frac": gc_bytes / t["grad_combine"] / 1e9 / PEAK_HBM_GBS,
            "expert_backward_us": t["expert_backward"] * 1e6,
            "expert_backward_flop": ebw_flop,
            "expert_backward_mfma_frac": ebw_flop / t["expert_backward"] / 1e12
                                         / PEAK_BF16_TFLOPS,
            "router_backward_us": t["router_backward"] * 1e6,
            "router_backward_fp32_frac": rb_flop / t["router_backward"] / 1e12
                                         / PEAK_F32_TFLOPS,
            "grad_dispatch_us": t["grad_dispatch"] * 1e6,
            "grad_dispatch_hbm_frac": gd_bytes / t["grad_dispatch"] / 1e9 / PEAK_HBM_GBS}


def dense_library_rate(cfg, torch):
    """Context for the grouped GEMM's fraction: torch's bf16 matmul (the vendor
    library) on one dense GEMM with the gate/up GEMM's flop (T*k x d @ d x 2I),
    timed on the same box, outside the measured steps."""
    M, K, N = cfg.R, cfg.d, 2 * cfg.I
    a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(10):
        c = a @ b
    ev[1].record()
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) / 10 * 1e-3
    del a, b, c
    tf = 2.0 * M * K * N / t / 1e12
    return {"dense_matmul": f"{M}x{K}x{N} bf16, torch.matmul", "us": t * 1e6, "tflops": tf,
            "frac": tf / PEAK_BF16_TFLOPS}


def cpu_baseline(inp, n_route, n_ffn):
    """The oracle as it stands, one thread, on a bounded sample of the
    workload: routing, BRIMs and gathers on a sub-batch of the first n_route
    tokens, expert FFN and combine on n_ffn seeded tokens of that sub-batch;
    tokens/s extrapolated linearly from the per-token cost of each part."""
    import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build()
    # one thread on one core (the calling thread is pinned to the first core
    # of its mask for the timing, then released)
    mask = os.sched_getaffinity(0)
    core = min(mask)
    os.sched_setaffinity(0, {core})
    try:
        res = _cpu_baseline_timed(inp, n_route, n_ffn)
    finally:
        os.sched_setaffinity(0, mask)
    res.update({"pinned_core": core, "host_cpus": len(mask), "cpu_model": _cpu_model()})
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline_timed(inp, n_route, n_ffn):
    import oracle
    cfg = inp.cfg
    E, k, D, d = cfg.E, cfg.k, cfg.D, cfg.d
    L = E // D
    Tb = min(n_route, cfg.T)
    x = inp.x[:Tb]
    t0 = time.perf_counter()
    lg = oracle.logits(x, inp.w_router, cfg.dtype)
    idx, w = oracle.topk(lg, k, cfg.renorm)
    b = oracle.brim(idx, w, inp.slot_expert, E, D)
    sfd = oracle.gather(x, b["sfd_token"][:b["S"]])
    oracle.gather(sfd, b["epd_sfd"])
    t_batch = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    tok = np.sort(rng.choice(Tb, size=min(n_ffn, Tb), replace=False)).astype(np.int32)
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
    out = oracle.expert_rows(x, b["epd_token"][rows], ex_of_slot[rows], inp.w_gate_up,
                             inp.w_down, cfg.dtype)
    epd_row = np.full(Tb * k, -1, np.int32)
    epd_row[rows] = np.arange(rows.size, dtype=np.int32)
    shared = None
    if cfg.n_shared:
        shared = oracle.shared_rows(x, tok, inp.w_gate_up_sh, inp.w_down_sh, cfg.dtype)
    oracle.combine(tok, b, Tb, D, L, d, cfg.dtype, out, epd_row, shared)
    t_sample = time.perf_counter() - t1
    per_token = t_batch / Tb + t_sample / tok.size
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": (f"routing, BRIMs and gathers on a sub-batch of the first {Tb} of the "
                       f"{cfg.T} tokens ({t_batch:.2f} s); expert FFN and combine on {tok.size} "
                       f"seeded tokens of it with all their {rows.size} EPD rows "
                       f"({t_sample:.2f} s); tokens/s = 1 / (sub-batch time / {Tb} + sample "
                       f"time / {tok.size}), one thread")}


def stage_times(lay, cfg, n, torch):
    """Mean time of each stage over n steps (an event between every two
    stages on the launch stream), with the derived roofline fractions, and
    the co-activation side output timed alone."""
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
             for _ in range(n)]
    for i in range(n):
        step(lay, marks[i])
    ca = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ca[0].record()
    for _ in range(n):
        lay.coactivation()
    ca[1].record()
    torch.cuda.synchronize()
    t = {name: float(np.mean([m[j].elapsed_time(m[j + 1]) for m in marks])) / 1e3
         for j, name in enumerate(STAGES)}
    t["coactivation"] = ca[0].elapsed_time(ca[1]) / 1e3 / n
    S = int(lay.host("S")[0])
    alg = algorithmic(cfg, S)
    peak_mfma = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    filtered = bool(lay.logits is None and lay.route_filtered and lay.route_ws is not None)
    return {
        "route_us": t["route"] * 1e6,
        # the candidate filter (occ_route_topk_ws) runs the chains of only the
        # certified candidates: against the plain kernel's 2 T d E flop this is
        # an equivalent rate, not the VALU's own
        "route_path": "candidate filter" if filtered else route_unit(cfg),
        "route_fp32_frac": alg["route_flop"] / t["route"] / 1e12 / PEAK_F32_TFLOPS,
        "route_hbm_frac": alg["route_bytes"] / t["route"] / 1e9 / PEAK_HBM_GBS,
        "build_brim_us": t["build_brim"] * 1e6,
        "build_brim_hbm_frac": alg["brim_bytes"] / t["build_brim"] / 1e9 / PEAK_HBM_GBS,
        "dispatch_us": t["dispatch"] * 1e6,
        "dispatch_hbm_frac": alg["dispatch_bytes"] / t["dispatch"] / 1e9 / PEAK_HBM_GBS,
        "expert_up_us": t["expert_up"] * 1e6,
        "expert_up_mfma_frac": alg["up_flop"] / t["expert_up"] / 1e12 / peak_mfma,
        "expert_down_us": t["expert_down"] * 1e6,
        "expert_down_mfma_frac": alg["down_flop"] / t["expert_down"] / 1e12 / peak_mfma,
        "combine_us": t["combine"] * 1e6,
        "combine_hbm_frac": alg["combine_bytes"] / t["combine"] / 1e9 / PEAK_HBM_GBS,
        "coactivation_us": t["coactivation"] * 1e6,
        "sum_us": sum(t[name] for name in STAGES) * 1e6,
    }


def timed_steps(lay, steps, torch):
    """Seconds for `steps` whole steps back to back (synchronised both sides)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(lay)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def graph_replay(lay, steps, torch):
    """The same step captured once into a HIP graph (torch's graph API around
    the same C-ABI calls) and replayed: ms per step without host launch
    overhead.  The library allocates nothing, so nothing is captured but its
    kernels."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step(lay)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(lay)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    del g
    return el / steps * 1e3


def greedy_placement(cfg, torch):
    """Correlated placement from a calibration batch (token seed 1): its
    routing and co-activation counts on the GPU, then occ_place_greedy."""
    import expert_top_router_amd as occ
    import workloads as W
    from expert_top_router_amd.layer import MoELayer, upload_inputs
    cal = W.make_layer(cfg, seed=0, token_seed=1, experts=False)
    lay = MoELayer(cfg, upload_inputs(cal), cal.slot_expert)
    lay.route()
    lay.coactivation()
    torch.cuda.synchronize()
    counts = lay.host("counts")
    del lay
    return occ.occ_place_greedy(cfg.E, cfg.D, counts), counts


def intra_share(counts, slot_expert, D):
    """Share of co-selection events (pairs i < j of a token's experts) whose
    two experts sit on one device."""
    E = counts.shape[0]
    L = E // D
    dev = np.empty(E, np.int64)
    dev[np.asarray(slot_expert)] = np.arange(E) // L
    iu = np.triu_indices(E, 1)
    c = counts[iu].astype(np.int64)
    same = dev[iu[0]] == dev[iu[1]]
    return float(c[same].sum()) / max(float(c.sum()), 1.0)


def other_workload(name, steps, warmup, torch, placements=("contiguous",), with_backward=False):
    """A secondary workload: whole-step time and per-stage times for each
    placement (a fresh layer per placement, freed afterwards); with_backward:
    the forward + backward step as well (first placement)."""
    import workloads as W
    from expert_top_router_amd.layer import MoELayer, upload_inputs
    cfg = W.CONFIGS[name]
    inp = W.make_layer(cfg, seed=0)
    weights = upload_inputs(inp)
    out = {"T": cfg.T, "d": cfg.d, "E": cfg.E, "I": cfg.I, "k": cfg.k, "D": cfg.D,
           "n_shared": cfg.n_shared}
    for pl in placements:
        rec = {}
        se = inp.slot_expert
        if pl == "greedy":
            se, counts = greedy_placement(cfg, torch)
            rec["intra_share"] = intra_share(counts, se, cfg.D)
            rec["contiguous_intra_share"] = intra_share(counts, inp.slot_expert, cfg.D)
        lay = MoELayer(cfg, weights, se)
        for _ in range(warmup):
            step(lay)
        el = timed_steps(lay, steps, torch)
        S = int(lay.host("S")[0])
        rec.update({"ms_per_step": el / steps * 1e3, "tokens_per_s": cfg.T * steps / el,
                    "sfd_rows": S, "sfd_over_tk": S / max(cfg.R, 1),
                    "stages": stage_times(lay, cfg, max(5, min(steps, 20)), torch)})
        if with_backward and pl == placements[0]:
            rec["backward"] = backward(lay, cfg, steps, torch)
        out[pl] = rec
        del lay
        torch.cuda.empty_cache()
    del weights
    torch.cuda.empty_cache()
    return out


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
        inp.slot_expert, _ = greedy_placement(cfg, torch)
    lay = MoELayer(cfg, upload_inputs(inp), inp.slot_expert)
    torch.cuda.synchronize()

    if args.profile_steps:
        if args.copy_calibration:
            # a plain copy of known size: what the traffic counters read for it
            # scales their readings for the layer's kernels
            src = torch.ones(256 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            for _ in range(2):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        if args.profile_backward:
            lay.prepare_backward()
            lay.dy.normal_()
        for _ in range(args.profile_steps):
            step(lay)
            lay.coactivation()
            if args.profile_backward:
                lay.backward()
        torch.cuda.synchronize()
        print(f"profiled {args.profile_steps} steps of {cfg.name}", flush=True)
        return

    for _ in range(args.warmup):
        step(lay)
    torch.cuda.synchronize()
    # Timed region: K steps back to back.  The dominant kernel (gate/up GEMM)
    # is bracketed by HIP events on the launch stream in every step.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        lay.route()
        lay.build_brim()
        lay.dispatch()
        ev[i][0].record()
        lay.expert_up()
        ev[i][1].record()
        lay.expert_down()
        lay.combine()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = cfg.T * args.steps / elapsed
    up_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3

    # Per-stage mean times in the same sequence (separate pass, an event
    # between every two stages), and the co-activation side output alone.
    stages = stage_times(lay, cfg, max(10, min(args.steps, 50)), torch)
    S = int(lay.host("S")[0])
    alg = algorithmic(cfg, S)
    peak_mfma = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    up_tf = alg["up_flop"] / up_s / 1e12
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
        "roofline": {"kernel": "gemm_bf16_kernel, gate/up GEMM with SwiGLU (occ_expert_up)",
                     "bound": "mfma", "achieved": up_tf, "peak": peak_mfma, "unit": "TFLOP/s",
                     "frac": up_tf / peak_mfma, "traffic": measured_traffic(cfg),
                     "launch_us": up_s * 1e6,
                     "flop_per_launch": alg["up_flop"]},
        "stages": stages,
    }
    # where the step's wall time goes: kernels (stage pass) against the rest
    # (launch gaps), and the same step replayed from a HIP graph
    out["step_breakdown"] = {"kernel_sum_us": stages["sum_us"],
                             "wall_minus_kernels_us": ms_per_step * 1e3 - stages["sum_us"],
                             "graph_ms_per_step": graph_replay(lay, args.steps, torch)}
    out["conventional"] = conventional(lay, cfg, args.steps, torch)
    if cfg.D >= 4:
        out["pruned"] = pruned(cfg, lay.w, inp.slot_expert, max(1, cfg.D // 4), args.steps, torch)
    out["affinity"] = affinity(cfg, lay, torch)
    if cfg.dtype == "bf16":
        out["backward"] = backward(lay, cfg, args.steps, torch)
    if cfg.dtype == "bf16":
        out["calibration"] = dense_library_rate(cfg, torch)
    del lay
    torch.cuda.empty_cache()
    if not args.no_others:
        others = {}
        for name in ("olmoe_bf16", "mixtral_bf16", "dsv2lite_bf16", "stress_bf16"):
            if name == cfg.name:
                continue
            pls = ("contiguous", "greedy") if name == "dsv2lite_bf16" else ("contiguous",)
            others[name] = other_workload(name, args.steps, args.warmup, torch, pls,
                                          with_backward=name == "dsv2lite_bf16")
        out["workloads"] = others
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_route_tokens, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
