"""proj_run_noalloc, the entry point for callers that cannot allocate device
memory, against proj_run: the same plan, its split-K partials in the
library's static per-GPU scratch instead of the context's workspace.

Plans are the untimed defaults (PROJ_TUNE=0), which split K for these
narrow shapes, so the scratch is what the partials go through.  Two calls in
a row, the second smaller (fewer rows, columns and k, bias, bf16 output),
each equal to proj_run's output bit for bit and within the acceptance rule
of the fp64 oracle; a shape whose plan's partials exceed the scratch is
refused with PROJ_ERR_NO_MEMORY and nothing enqueued."""
import re

import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor, require_gpu

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 2 << 20


def _splits(plan):
    """Workspace partials of a plan: its K-split count, 1 for plans without a
    split and for atomic splits (which add into Y and need no workspace)."""
    m = re.search(r"_s(\d+)(_atomic)?(?:_r\d+)?$", plan.split(" ")[0])
    return int(m.group(1)) if m and not m.group(2) else 1


def _inputs(M, N, K, bias, seed):
    X = synth.normal_bf16((M, K), 1.0, 7500 + seed)
    W = synth.normal_bf16((N, K), float(1 / np.sqrt(K)), 7600 + seed)
    b = synth.normal_bf16((N,), float(np.sqrt(0.02)), 7700 + seed) if bias else None
    return X, W, b


def test_noalloc_matches_proj_run_two_calls(monkeypatch):
    require_gpu()
    import torch
    monkeypatch.setenv("PROJ_TUNE", "0")
    c = dlp.proj_create(0)
    try:
        cases = [(16, 1024, 8192, dlp.EPI_NONE, dlp.OUT_F32),
                 (8, 512, 4096, dlp.EPI_BIAS, dlp.OUT_BF16)]   # the second call is smaller
        for seed, (M, N, K, epi, out) in enumerate(cases):
            print("noalloc call", seed, (M, N, K, epi, out), flush=True)
            X, W, b = _inputs(M, N, K, epi & 1, seed)
            Xd, Wd = dev_bf16(X), dev_bf16(W)
            bd = dev_bf16(b) if b is not None else None
            Yref = out_tensor(M, N, out)
            dlp.proj_run(c, Xd, Wd, bd, epi, Yref)
            plan = dlp.proj_get_plan(c, M, N, K, epi, out)
            S = _splits(plan)
            print("plan", plan, flush=True)
            assert S > 1 and S * M * N * 4 <= SCRATCH_BYTES, plan
            Y = out_tensor(M, N, out)
            dlp.proj_run_noalloc(c, Xd, Wd, bd, epi, Y)
            u, uref = host_f64(Y), host_f64(Yref)
            assert np.array_equal(u, uref), "noalloc differs from proj_run (same plan %s)" % plan
            r, _ = oracle.reference(X, W, b, epi, out)
            rep = compare.check(u, r)
            assert rep["ok"], rep
        # a shape with no cached plan: the default among plans that fit
        M, N, K = 16, 2048, 2048
        X, W, _ = _inputs(M, N, K, False, 5)
        Y = out_tensor(M, N, dlp.OUT_F32)
        dlp.proj_run_noalloc(c, dev_bf16(X), dev_bf16(W), None, dlp.EPI_NONE, Y)
        r, _ = oracle.reference(X, W, None, oracle.EPI_NONE, oracle.OUT_F32)
        assert compare.check(host_f64(Y), r)["ok"]
        with pytest.raises(dlp.ProjError):
            dlp.proj_get_plan(c, M, N, K, dlp.EPI_NONE, dlp.OUT_F32)   # nothing was cached
        # a cached plan whose partials (4 x 64 x 3072 x 4 bytes = 3 MiB)
        # exceed the scratch: refused, Y untouched
        M, N, K = 64, 3072, 1024
        X, W, _ = _inputs(M, N, K, False, 6)
        Xd, Wd = dev_bf16(X), dev_bf16(W)
        Y = out_tensor(M, N, dlp.OUT_F32)
        dlp.proj_run(c, Xd, Wd, None, dlp.EPI_NONE, Y)
        plan = dlp.proj_get_plan(c, M, N, K, dlp.EPI_NONE, dlp.OUT_F32)
        print("large plan", plan, flush=True)
        if _splits(plan) * M * N * 4 > SCRATCH_BYTES:
            Y2 = out_tensor(M, N, dlp.OUT_F32, fill=7.0)
            with pytest.raises(dlp.ProjError) as e:
                dlp.proj_run_noalloc(c, Xd, Wd, None, dlp.EPI_NONE, Y2)
            assert e.value.status == dlp.PROJ_ERR_NO_MEMORY
            assert "scratch" in str(e.value)
            torch.cuda.synchronize()
            assert bool((Y2 == 7.0).all())
    finally:
        dlp.proj_destroy(c)
