"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Tolerances (the method's accuracy targets): fp32 inputs max-abs <= 1e-5; fp16 /
bf16 inputs max-abs <= 2e-2 and relative RMS <= 5e-3; the log-sum-exp within
1e-3 on finite rows, and -inf exactly where the oracle has no visible key.
"""

import numpy as np

TOL = {
    "f32": dict(max_abs=1e-5, rel_rms=None),
    "f16": dict(max_abs=2e-2, rel_rms=5e-3),
    "bf16": dict(max_abs=2e-2, rel_rms=5e-3),
}
LSE_TOL = 1e-3


def errors(o_gpu, o_ref, lse_gpu=None, lse_ref=None):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    d = o_gpu - o_ref
    out = {
        "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
        "rel_rms": float(np.linalg.norm(d) / max(np.linalg.norm(o_ref), 1e-300)) if d.size else 0.0,
        "nonfinite": int(np.count_nonzero(~np.isfinite(o_gpu))),
    }
    if lse_ref is not None:
        lg = np.asarray(lse_gpu, dtype=np.float64)
        lr = np.asarray(lse_ref, dtype=np.float64)
        fin = np.isfinite(lr)
        out["lse_max_abs"] = float(np.max(np.abs(lg[fin] - lr[fin]))) if fin.any() else 0.0
        out["lse_inf_mismatch"] = int(np.count_nonzero(np.isneginf(lr) != np.isneginf(lg)))
    return out


def assert_close(dtype, o_gpu, o_ref, lse_gpu=None, lse_ref=None, what=""):
    e = errors(o_gpu, o_ref, lse_gpu, lse_ref)
    tol = TOL[dtype]
    msg = "%s %s: %s" % (what, dtype, e)
    assert e["nonfinite"] == 0, msg
    assert e["max_abs"] <= tol["max_abs"], msg
    if tol["rel_rms"] is not None:
        assert e["rel_rms"] <= tol["rel_rms"], msg
    if lse_ref is not None:
        assert e["lse_inf_mismatch"] == 0, msg
        assert e["lse_max_abs"] <= LSE_TOL, msg
    return e


# Gradients (backward pass).  The GPU rounds P and dS to the input dtype
# before its MFMAs (relative error 2^-9 for bf16, 2^-12 for fp16 per element,
# random in sign), on top of the rounding of dO and O in the row sums; the
# result is compared by its relative RMS error and by its largest error
# relative to the largest reference value.
GRAD_TOL = {
    "f16": dict(max_rel=1.5e-2, rel_rms=5e-3),
    "bf16": dict(max_rel=3e-2, rel_rms=1e-2),
}


def grad_errors(g_gpu, g_ref):
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    g_ref = np.asarray(g_ref, dtype=np.float64)
    d = g_gpu - g_ref
    scale = max(float(np.max(np.abs(g_ref))) if g_ref.size else 0.0, 1e-30)
    return {
        "max_rel": float(np.max(np.abs(d))) / scale if d.size else 0.0,
        "rel_rms": float(np.linalg.norm(d) / max(np.linalg.norm(g_ref), 1e-300)) if d.size else 0.0,
        "nonfinite": int(np.count_nonzero(~np.isfinite(g_gpu))),
    }


def assert_grad_close(dtype, g_gpu, g_ref, what=""):
    e = grad_errors(g_gpu, g_ref)
    tol = GRAD_TOL[dtype]
    msg = "%s %s: %s" % (what, dtype, e)
    print("  ", msg, flush=True)
    assert e["nonfinite"] == 0, msg
    assert e["max_rel"] <= tol["max_rel"], msg
    assert e["rel_rms"] <= tol["rel_rms"], msg
    return e
