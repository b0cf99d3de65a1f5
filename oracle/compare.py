"""Acceptance rule for GPU results against the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Gate: every element finite and |u - r| <= ATOL + RTOL * |r|, with r the
oracle's fp64 result rounded to the output type.  ATOL = 2e-3, RTOL = 2e-2
is the per-element tolerance of the hot path's target; the Devpost
"blackroom" page (section "What it does") states the looser-combined
either-or form |u - r| <= 0.002 or <= 0.02|r|, which is reported beside it.
The worklog's whole-output relative L2 measure (section "The actual error
rule, including what L2 means": error norm over reference norm) is reported,
not gated, by ``check``.

``check_rows`` is that section's whole rule, used where the weights are fp32
(the router, tolerance 0.01%): relative L2 over the whole output within the
tolerance; each row within five times it, against its own reference norm or
a tenth of the mean row norm, whichever is larger, with a small floor; the
sparse probe rows within 0.1% of their own norm; every value finite.  The
floor (1e-12) is this code's reading of "a small numerical floor".
"""
from __future__ import annotations

import numpy as np

ATOL = 2e-3
RTOL = 2e-2


def rel_l2(u, r) -> float:
    u = np.asarray(u, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = float(np.sqrt(np.sum(r * r)))
    num = float(np.sqrt(np.sum((u - r) ** 2)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def check(u, r, atol: float = ATOL, rtol: float = RTOL) -> dict:
    """Element-by-element comparison; returns a report dict with 'ok'."""
    u = np.asarray(u, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if u.shape != r.shape:
        return {"ok": False, "reason": "shape %s vs %s" % (u.shape, r.shape)}
    finite = np.isfinite(u)
    err = np.abs(u - r)
    bound = atol + rtol * np.abs(r)
    bad = ~(finite & (err <= bound))
    either_or = (err <= atol) | (err <= rtol * np.abs(r))
    rep = {
        "ok": bool(not bad.any()),
        "n": int(u.size),
        "n_bad": int(bad.sum()),
        "n_nonfinite": int((~finite).sum()),
        "max_abs_err": float(err[finite].max()) if finite.any() else float("nan"),
        "max_ratio": float((err / bound)[finite].max()) if finite.any() else float("nan"),
        "either_or_ok": bool(either_or.all() and finite.all()),
        "rel_l2": rel_l2(u, r) if finite.all() else float("inf"),
    }
    if bad.any():
        idx = np.argwhere(bad)[0]
        rep["first_bad"] = {"index": [int(i) for i in idx], "u": float(u[tuple(idx)]),
                            "r": float(r[tuple(idx)])}
    return rep


ROUTER_TOL = 1e-4
PROBE_TOL = 1e-3
ROW_FLOOR = 1e-12


def check_rows(u, r, tol: float = ROUTER_TOL, probe_rows=(), probe_tol: float = PROBE_TOL) -> dict:
    """The worklog's row rule for a 2-D output; returns a report with 'ok'."""
    u = np.asarray(u, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if u.shape != r.shape or u.ndim != 2:
        return {"ok": False, "reason": "shape %s vs %s" % (u.shape, r.shape)}
    if not np.isfinite(u).all():
        return {"ok": False, "reason": "non-finite output", "n_nonfinite": int((~np.isfinite(u)).sum())}
    whole = rel_l2(u, r)
    err_rows = np.sqrt(np.sum((u - r) ** 2, axis=1))
    ref_rows = np.sqrt(np.sum(r * r, axis=1))
    mean_norm = float(ref_rows.mean()) if ref_rows.size else 0.0
    den = np.maximum(np.maximum(ref_rows, 0.1 * mean_norm), ROW_FLOOR)
    row_ratio = err_rows / den if err_rows.size else np.zeros(0)
    probe = np.asarray(probe_rows, dtype=np.int64)
    probe_ratio = err_rows[probe] / np.maximum(ref_rows[probe], ROW_FLOOR) if probe.size else np.zeros(0)
    rep = {
        "rel_l2": whole,
        "max_row": float(row_ratio.max()) if row_ratio.size else 0.0,
        "max_probe": float(probe_ratio.max()) if probe_ratio.size else 0.0,
        "n_probe": int(probe.size),
    }
    rep["ok"] = bool(whole <= tol and rep["max_row"] <= 5 * tol and rep["max_probe"] <= probe_tol)
    return rep
