"""Seeded synthetic inputs for the collaboration-aware MoE layer.

This module is the only code that the CPU oracle (``oracle/``) and the HIP
path (``expert_top_router_amd``) have in common.  It draws random numbers and
shapes them into layer inputs; it holds none of the layer's arithmetic
(routing, re-indexing, expert networks, combining are all elsewhere).

Recipe (every tensor is keyed by ``(seed, tensor name, chunk)``):

* bits: Philox4x64-10 (Salmon et al., "Parallel random numbers: as easy as
  1, 2, 3", SC 2011), one counter-based stream per key, via numpy's
  ``Philox`` bit generator (the raw 64-bit outputs only, which numpy keeps
  stable across versions).
* normals: Box-Muller on pairs of 53-bit uniforms, in float64.
* rounding: float64 -> float32 (round to nearest even) -> bfloat16 (round to
  nearest even) for bf16 layers; float64 -> float32 for fp32 layers.
* "N(0, v)" means variance v.

The five workloads stand in for the models the Occult, ExFlow and
correlated-placement pages measure on (no weights or datasets are used):
tiny fp32, OLMoE-shaped, Mixtral-shaped, DeepSeek-V2-Lite-shaped (routed plus
shared experts) and a large top-6 stress layer whose router is skewed so that
about 1% of expert pairs carry about 40% of co-selections (the concentration
the correlated-placement page reports at top-2).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import hashlib
import json
import math
import os
from typing import Dict, Optional

import numpy as np

CHUNK = 1 << 22  # normals per independently keyed chunk
_HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens in the batch (ORI rows)
    d: int            # hidden size
    E: int            # routed experts
    I: int            # intermediate size of one routed expert
    k: int            # experts per token
    D: int            # logical expert-parallel devices
    dtype: str        # "f32" or "bf16": storage type of tokens, weights, outputs
    renorm: int = 0   # 1: top-k weights divided by their sum
    n_shared: int = 0
    I_shared: int = 0
    clusters: int = 0           # 0: i.i.d. N(0,1) tokens; else Gaussian mixture
    spread: float = 0.3         # std of a token around its cluster centre
    skew_groups: int = 0        # >0: router skewed toward hot expert groups
    skew_group_size: int = 4
    alpha: float = 0.0          # skew strength (frozen by calibration)

    @property
    def L(self) -> int:
        return self.E // self.D

    @property
    def S_max(self) -> int:
        return self.T * min(self.k, self.D)

    @property
    def R(self) -> int:
        return self.T * self.k

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


def _load_alpha() -> float:
    path = os.path.join(_HERE, "stress_alpha.json")
    if not os.path.exists(path):
        return 0.0
    with open(path) as f:
        return float(json.load(f)["alpha"])


CONFIGS: Dict[str, LayerConfig] = {
    "tiny_fp32": LayerConfig("tiny_fp32", T=256, d=64, E=8, I=128, k=2, D=2, dtype="f32"),
    "olmoe_bf16": LayerConfig("olmoe_bf16", T=4096, d=2048, E=64, I=1024, k=8, D=8,
                              dtype="bf16", clusters=16),
    "mixtral_bf16": LayerConfig("mixtral_bf16", T=8192, d=4096, E=8, I=14336, k=2, D=4,
                                dtype="bf16", renorm=1),
    "dsv2lite_bf16": LayerConfig("dsv2lite_bf16", T=16384, d=2048, E=64, I=1408, k=6, D=8,
                                 dtype="bf16", n_shared=2, I_shared=1408, clusters=32),
    "stress_bf16": LayerConfig("stress_bf16", T=65536, d=2048, E=128, I=768, k=6, D=16,
                               dtype="bf16", clusters=64, skew_groups=14,
                               alpha=_load_alpha()),
}
CONFIG_ORDER = ["tiny_fp32", "olmoe_bf16", "mixtral_bf16", "dsv2lite_bf16", "stress_bf16"]


# ---------------------------------------------------------------------------
# bits and normals
# ---------------------------------------------------------------------------
def _key(seed: int, name: str, chunk: int) -> int:
    h = hashlib.sha256(f"{seed}/{name}/{chunk}".encode()).digest()
    return int.from_bytes(h[:16], "little")


def raw_u64(seed: int, name: str, n: int, chunk: int = 0) -> np.ndarray:
    """n raw 64-bit words of the Philox stream keyed by (seed, name, chunk)."""
    bg = np.random.Philox(key=_key(seed, name, chunk))
    return bg.random_raw(n).astype(np.uint64, copy=False)


def uniform01(seed: int, name: str, n: int) -> np.ndarray:
    """n float64 uniforms in [0, 1) with 53 random bits each."""
    return (raw_u64(seed, name, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def _normal_chunk(seed: int, name: str, chunk: int, n: int) -> np.ndarray:
    m = (n + 1) // 2
    bits = raw_u64(seed, name, 2 * m, chunk)
    u1 = ((bits[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)  # (0, 1]
    u2 = (bits[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)          # [0, 1)
    r = np.sqrt(-2.0 * np.log(u1))
    th = (2.0 * math.pi) * u2
    out = np.empty(2 * m, dtype=np.float64)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    return out[:n]


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_into(out: np.ndarray, seed: int, name: str, scale: float, dtype: str) -> None:
    """Fill the flat array ``out`` (float32 or uint16 bf16 bits) with
    scale * N(0, 1), rounded to ``dtype``.  Chunks are keyed independently, so
    the result does not depend on the number of worker threads."""
    n = out.size
    flat = out.reshape(-1)

    def job(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        v = _normal_chunk(seed, name, c, hi - lo)
        if scale != 1.0:
            v *= scale
        flat[lo:hi] = from_f64(v, dtype)

    nch = (n + CHUNK - 1) // CHUNK
    if nch <= 1:
        for c in range(nch):
            job(c)
    else:
        with _cf.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(job, range(nch)))


def normal(seed: int, name: str, shape, scale: float = 1.0, dtype: str = "f64") -> np.ndarray:
    n = int(np.prod(shape))
    if dtype == "f64":
        parts = [_normal_chunk(seed, name, c, min(CHUNK, n - c * CHUNK))
                 for c in range((n + CHUNK - 1) // CHUNK)]
        v = np.concatenate(parts) if parts else np.zeros(0)
        return (v * scale).reshape(shape)
    out = np.empty(n, dtype=storage_np(dtype))
    normal_into(out, seed, name, scale, dtype)
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# storage types (bfloat16 is kept as raw uint16 bits)
# ---------------------------------------------------------------------------
def storage_np(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16}[dtype]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def from_f64(v: np.ndarray, dtype: str) -> np.ndarray:
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f
    if dtype == "bf16":
        return f32_to_bf16_bits(f)
    raise ValueError(dtype)


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float32."""
    return np.asarray(a, dtype=np.float32) if dtype == "f32" else bf16_bits_to_f32(a)


# ---------------------------------------------------------------------------
# layer inputs
# ---------------------------------------------------------------------------
def cluster_centres(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    return normal(seed, "centres", (cfg.clusters, cfg.d))


def skew_groups(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    """[skew_groups, skew_group_size] disjoint expert groups from a seeded
    permutation (so they are not aligned with contiguous placement)."""
    perm = np.argsort(raw_u64(seed, "skew_perm", cfg.E), kind="stable")
    n = cfg.skew_groups * cfg.skew_group_size
    return perm[:n].reshape(cfg.skew_groups, cfg.skew_group_size).astype(np.int64)


def make_tokens(cfg: LayerConfig, seed: int = 0, token_seed: Optional[int] = None,
                T: Optional[int] = None) -> np.ndarray:
    """ORI token tensor X [T, d] in the layer's storage type.

    i.i.d. N(0,1), or a Gaussian mixture x_t = c_{z_t} + spread * N(0, I)
    with centres c ~ N(0, I) drawn from ``seed`` and z_t uniform."""
    ts = seed if token_seed is None else token_seed
    T = cfg.T if T is None else T
    if cfg.clusters == 0:
        return normal(ts, "tokens", (T, cfg.d), 1.0, cfg.dtype)
    centres = cluster_centres(cfg, seed)
    z = np.floor(uniform01(ts, "cluster_of_token", T) * cfg.clusters).astype(np.int64)
    out = np.empty((T, cfg.d), dtype=storage_np(cfg.dtype))
    rows_per = max(1, CHUNK // cfg.d)
    # noise drawn chunk-wise in f64 then shifted by the centre of each row
    flat = out.reshape(-1)

    def job(c):
        lo = c * CHUNK
        hi = min(T * cfg.d, lo + CHUNK)
        v = _normal_chunk(ts, "tokens", c, hi - lo) * cfg.spread
        r0 = lo // cfg.d
        v = v.reshape(-1, cfg.d) + centres[z[r0:r0 + (hi - lo) // cfg.d]]
        flat[lo:hi] = from_f64(v.reshape(-1), cfg.dtype)

    assert CHUNK % cfg.d == 0 and rows_per >= 1
    nch = (T * cfg.d + CHUNK - 1) // CHUNK
    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range(nch)))
    return out


def make_router(cfg: LayerConfig, seed: int = 0, alpha: Optional[float] = None,
                layer: int = 0) -> np.ndarray:
    """Router W_r [E, d]: N(0, 1/d), plus for the skewed workload
    alpha * sum over the clusters c mapped to e's hot group of c_c/|c_c|^2.
    `layer` > 0 draws the router of a further layer of a stack (its own
    stream; the same tokens feed every layer of a synthetic stack)."""
    a = cfg.alpha if alpha is None else alpha
    name = "router" if layer == 0 else f"router{layer}"
    w = normal(seed, name, (cfg.E, cfg.d), 1.0 / math.sqrt(cfg.d))
    if cfg.skew_groups > 0 and a != 0.0:
        centres = cluster_centres(cfg, seed)
        groups = skew_groups(cfg, seed)
        for c in range(cfg.clusters):
            g = c % cfg.skew_groups
            dirn = centres[c] / np.dot(centres[c], centres[c])
            for e in groups[g]:
                w[e] += a * dirn
    return from_f64(w.reshape(-1), cfg.dtype).reshape(cfg.E, cfg.d)


def make_experts(cfg: LayerConfig, seed: int = 0):
    """Routed expert weights: W_gate_up [E, 2I, d] (rows 0..I-1 gate, I..2I-1
    up) and W_down [E, d, I], all N(0, 1/d) and K-contiguous."""
    s = 1.0 / math.sqrt(cfg.d)
    st = storage_np(cfg.dtype)
    wgu = np.empty((cfg.E, 2 * cfg.I, cfg.d), dtype=st)
    normal_into(wgu.reshape(-1), seed, "w_gate_up", s, cfg.dtype)
    wdn = np.empty((cfg.E, cfg.d, cfg.I), dtype=st)
    normal_into(wdn.reshape(-1), seed, "w_down", s, cfg.dtype)
    return wgu, wdn


def make_shared_experts(cfg: LayerConfig, seed: int = 0):
    """Shared expert weights [n_shared, 2*I_shared, d] and [n_shared, d, I_shared]."""
    if cfg.n_shared == 0:
        return None, None
    s = 1.0 / math.sqrt(cfg.d)
    st = storage_np(cfg.dtype)
    wgu = np.empty((cfg.n_shared, 2 * cfg.I_shared, cfg.d), dtype=st)
    normal_into(wgu.reshape(-1), seed, "w_gate_up_shared", s, cfg.dtype)
    wdn = np.empty((cfg.n_shared, cfg.d, cfg.I_shared), dtype=st)
    normal_into(wdn.reshape(-1), seed, "w_down_shared", s, cfg.dtype)
    return wgu, wdn


def contiguous_placement(cfg: LayerConfig) -> np.ndarray:
    """slot_expert = iota: slot g = device * L + local holds expert g."""
    return np.arange(cfg.E, dtype=np.int32)


@dataclasses.dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray
    w_router: np.ndarray
    w_gate_up: Optional[np.ndarray]
    w_down: Optional[np.ndarray]
    w_gate_up_sh: Optional[np.ndarray]
    w_down_sh: Optional[np.ndarray]
    slot_expert: np.ndarray


def make_layer(cfg: LayerConfig, seed: int = 0, token_seed: Optional[int] = None,
               experts: bool = True) -> LayerInputs:
    x = make_tokens(cfg, seed, token_seed)
    wr = make_router(cfg, seed)
    wgu = wdn = wgus = wdns = None
    if experts:
        wgu, wdn = make_experts(cfg, seed)
        wgus, wdns = make_shared_experts(cfg, seed)
    return LayerInputs(cfg, x, wr, wgu, wdn, wgus, wdns, contiguous_placement(cfg))


def checksum(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
