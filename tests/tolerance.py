"""Float comparison used by every parity test.

Per tensor: max_i |g_i - o_i| / max(|o_i|, rms(o)).  The bound is 1e-4 for
fp32 layers (and for the fp32 routing weights of every layer) and 2e-2 for
bf16 layers.  The normwise error |g - o|_2 / |o|_2 is reported beside it."""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.abs(o), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(g - o) / den))


def norm_err(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    n = float(np.linalg.norm(o))
    return float(np.linalg.norm(g - o)) / (n if n > 0 else 1.0)


def assert_close(g, o, dtype, what=""):
    e = rel_err(g, o)
    assert e <= TOL[dtype], f"{what}: max rel err {e:.3e} > {TOL[dtype]} (normwise {norm_err(g, o):.3e})"
    return e
