"""Float comparison used by every parity test.

Per tensor: max_i |g_i - o_i| / max(|o_i|, rms(o)).  The bound is 1e-4 for
fp32 layers (and for the fp32 routing weights of every layer) and 2e-2 for
bf16 layers.  The normwise error |g - o|_2 / |o|_2 is reported beside it.

Sums of stored values (the pre-reduced return rows and the combined output)
take each element's error relative to the magnitude of its summands,
max(|o_i|, sum |summands_i|, rms(o)): the summands are themselves rounded
results (a bf16 expert output may differ by one rounding step between two
correct implementations), and where they cancel the error of the sum is
bounded by their size, not by the sum's."""
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


def rel_err_sum(g, o, mag):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.maximum(np.abs(o), np.asarray(mag, np.float64)), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(g - o) / den))


def assert_close_sum(g, o, mag, dtype, what=""):
    e = rel_err_sum(g, o, mag)
    assert e <= TOL[dtype], (f"{what}: max rel err {e:.3e} (summand magnitudes) > {TOL[dtype]} "
                             f"(plain {rel_err(g, o):.3e}, normwise {norm_err(g, o):.3e})")
    return e
