"""The five workloads at full size, through proj_run with the measured plan
(the plan the benchmark's graphs replay), against the oracle.

The two M = 16 workloads are compared on every element.  For the larger ones
the oracle computes sampled cells one by one: whole rows (every n-tile of
the output), whole columns (every m-tile) and random cells; in addition every
output element must be finite and the output statistics must be those of a
unit-variance projection.
"""
import sys

import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu


def _run(ctx, w):
    X, W, b = synth.workload_inputs(w)
    Y = out_tensor(w.M, w.N, w.out_dtype)
    dlp.proj_run(ctx, dev_bf16(X), dev_bf16(W), dev_bf16(b) if b is not None else None, w.epi, Y)
    u = host_f64(Y)
    return X, W, b, u


@pytest.mark.parametrize("idx", [0, 1])
def test_small_workloads_every_element(ctx, idx):
    w = synth.WORKLOADS[idx]
    print("workload", w.name, flush=True)
    X, W, b, u = _run(ctx, w)
    r, _ = oracle.reference(X, W, b, w.epi, w.out_dtype)
    rep = compare.check(u, r)
    print(w.name, dlp.proj_get_plan(ctx, w.M, w.N, w.K, w.epi, w.out_dtype), rep, flush=True)
    assert rep["ok"], rep


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_large_workloads_sampled(ctx, idx):
    w = synth.WORKLOADS[idx]
    print("workload", w.name, flush=True)
    X, W, b, u = _run(ctx, w)
    assert np.isfinite(u).all()
    rng = np.random.default_rng(100 + idx)
    full_rows = [0, w.M - 1, int(rng.integers(w.M))]
    full_cols = [0, w.N - 1, int(rng.integers(w.N))]
    rows = np.concatenate([np.repeat(full_rows, w.N), np.tile(np.arange(w.M), len(full_cols)),
                           rng.integers(0, w.M, 4000)])
    cols = np.concatenate([np.tile(np.arange(w.N), len(full_rows)), np.repeat(full_cols, w.M),
                           rng.integers(0, w.N, 4000)])
    s = oracle.proj_f64_at(X, W, rows, cols, b, w.epi)
    r = oracle.round_out(s, w.out_dtype)
    r = oracle.bf16_to_f64(r) if w.out_dtype == oracle.OUT_BF16 else r.astype(np.float64)
    rep = compare.check(u[rows, cols], r)
    print(w.name, dlp.proj_get_plan(ctx, w.M, w.N, w.K, w.epi, w.out_dtype), rep, flush=True)
    assert rep["ok"], rep
    # whole-output properties: projection of unit-variance rows by N(0, 1/K)
    # weights has unit variance (before GELU); GELU output mean is positive
    if w.epi & 2:
        assert 0.1 < u.mean() < 0.6
    else:
        assert abs(u.std() - 1.0) < 0.1
    sys.stdout.flush()
