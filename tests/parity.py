"""Tolerances and comparison of GPU results against the fp64 oracle.

Bar for bf16/fp16 inputs with fp32 accumulation: max |O - O_ref| <= 2e-2,
rel-L2 = ||O - O_ref||_2 / ||O_ref||_2 <= 5e-3 over the checked set, and
max |lse - lse_ref| <= 1e-3.
"""
import numpy as np

O_MAX_ABS = 2e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


def report(o, ro, lse=None, rl=None):
    o = np.asarray(o, np.float64)
    ro = np.asarray(ro, np.float64)
    out = {"max_abs": float(np.abs(o - ro).max()) if o.size else 0.0,
           "rel_l2": float(np.linalg.norm(o - ro) / max(np.linalg.norm(ro), 1e-300)) if o.size else 0.0}
    if lse is not None:
        lse = np.asarray(lse, np.float64)
        rl = np.asarray(rl, np.float64)
        out["lse_max_abs"] = float(np.abs(lse - rl).max()) if lse.size else 0.0
    return out


def assert_close(o, ro, lse=None, rl=None, what="", o_max_abs=O_MAX_ABS, o_rel_l2=O_REL_L2,
                 lse_max_abs=LSE_MAX_ABS):
    assert np.isfinite(np.asarray(o)).all(), f"{what}: non-finite output"
    r = report(o, ro, lse, rl)
    print(f"{what}: {r}", flush=True)
    assert r["max_abs"] <= o_max_abs, (what, r)
    assert r["rel_l2"] <= o_rel_l2, (what, r)
    if lse is not None:
        assert r["lse_max_abs"] <= lse_max_abs, (what, r)
    return r
