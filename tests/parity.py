"""Shared comparison helpers for the GPU parity tests (no attention arithmetic).

Tolerances are the ones fixed for this path: on O, max-abs error <= 2e-2 and
mean-abs error <= 2e-3; on the logsumexp, relative error <= 1e-3.  Both sides
see the same 16-bit inputs; the GPU output is compared against the oracle's
unrounded fp64 result.
"""
import json
import os

import numpy as np

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_REL = 1e-3


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    o_gpu = np.asarray(o_gpu, np.float64)
    lse_gpu = np.asarray(lse_gpu, np.float64)
    e = np.abs(o_gpu - o_ref)
    le = np.abs(lse_gpu - lse_ref) / np.maximum(np.abs(lse_ref), 1e-30)
    return {"o_max_abs": float(e.max()) if e.size else 0.0,
            "o_mean_abs": float(e.mean()) if e.size else 0.0,
            "lse_max_rel": float(le.max()) if le.size else 0.0,
            "finite": bool(np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)))}


def assert_parity(o_gpu, lse_gpu, o_ref, lse_ref, tag="", lse_abs=None):
    """lse_abs: for rows whose logsumexp is near 0 the relative bar is
    meaningless; pass an absolute bound to use max(rel, abs) per row."""
    err = errors(o_gpu, lse_gpu, o_ref, lse_ref)
    msg = "%s: %s" % (tag, err)
    assert err["finite"], msg
    assert err["o_max_abs"] <= O_MAX_ABS, msg
    assert err["o_mean_abs"] <= O_MEAN_ABS, msg
    if lse_abs is None:
        assert err["lse_max_rel"] <= LSE_REL, msg
    else:
        d = np.abs(np.asarray(lse_gpu, np.float64) - lse_ref)
        ok = (d <= LSE_REL * np.abs(lse_ref)) | (d <= lse_abs)
        assert np.all(ok), msg
    print(msg, flush=True)
    log = os.environ.get("FA2_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps(dict(err, case=tag)) + "\n")
    return err
