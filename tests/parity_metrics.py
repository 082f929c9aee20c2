"""Error measures used by the parity tests.

A plain elementwise relative error is undefined where the reference is near
zero (a gated output passes through zero often), so the bound applied is

    err = max_i |g_i - r_i| / (|r_i| + rms(r))

over one output tensor: relative where |r_i| is large, relative to the
tensor's RMS where it is small.  The plain relative error over the elements
with |r_i| >= rms(r) and the normwise ||g - r|| / ||r|| are reported next to
it for information.
"""
import numpy as np


def as_f64(a):
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def scaled_max_err(got, ref):
    g, r = as_f64(got), as_f64(ref)
    if g.shape != r.shape:
        raise AssertionError("shape %s vs %s" % (g.shape, r.shape))
    if r.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    rms = float(np.sqrt(np.mean(r * r)))
    denom = np.abs(r) + rms
    denom = np.where(denom == 0, 1.0, denom)
    return float(np.max(np.abs(g - r) / denom))


def report(got, ref):
    g, r = as_f64(got), as_f64(ref)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    big = np.abs(r) >= rms
    rel = (float(np.max(np.abs(g[big] - r[big]) / np.abs(r[big])))
           if np.any(big) and rms > 0 else 0.0)
    nrm = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    return {"scaled_max": scaled_max_err(g, r), "rel_over_rms": rel,
            "normwise": nrm}
