"""The five workloads at full size, through proj_run with the measured plan
(the plan the benchmark's graphs replay), against the oracle on every
element of the output, with the acceptance rule |u - r| <= 2e-3 + 2e-2 |r|
and every value finite (worklog "How I made Muse's GPU projections 1.32x
faster in the Open Kernel Challenge", section "The actual error rule,
including what L2 means": the reference is computed in FP64 and converted to
the output type before the comparison).

The oracle takes seconds for the M = 64 and M = 8192 workloads and tens of
seconds for the M = 4096, K = 8192 one on the host's cores; the output is
copied back once and compared whole.
"""
import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4], ids=lambda i: synth.WORKLOADS[i].name)
def test_workload_every_element(ctx, idx):
    w = synth.WORKLOADS[idx]
    print("workload", w.name, flush=True)
    X, W, b = synth.workload_inputs(w)
    Y = out_tensor(w.M, w.N, w.out_dtype)
    dlp.proj_run(ctx, dev_bf16(X), dev_bf16(W), dev_bf16(b) if b is not None else None, w.epi, Y)
    u = host_f64(Y)
    del Y
    print(w.name, "plan", dlp.proj_get_plan(ctx, w.M, w.N, w.K, w.epi, w.out_dtype), flush=True)
    r, _ = oracle.reference(X, W, b, w.epi, w.out_dtype)
    assert u.shape == r.shape == (w.M, w.N)
    rep = compare.check(u, r)
    print(w.name, rep, flush=True)
    assert rep["ok"], rep
    assert rep["n"] == w.M * w.N
