"""Status paths of the boundary on the GPU: the caller-bounded split-K
workspace (plans that do not fit are never chosen, a candidate that does
not fit is refused with PROJ_ERR_NO_MEMORY, also under stream capture), the
tuner's flush buffer released after tuning, and graphs of a destroyed
context refused instead of replayed."""
import re

import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor, require_gpu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

@pytest.fixture(autouse=True)
def _needs_gpu():
    require_gpu()


# the M = 16, K = 8192, N = 1024 fp32 projection: its best plans split K
M, N, K = 16, 1024, 8192


def _inputs(seed=0):
    X = synth.normal_bf16((M, K), 1.0, 7000 + seed)
    W = synth.normal_bf16((N, K), float(1 / np.sqrt(K)), 7100 + seed)
    return X, W


def _splits(name):
    """Workspace partials of a plan: its K-split count, 1 for plans without a
    split and for atomic splits (which add into Y and need no workspace)."""
    m = re.search(r"_s(\d+)(_atomic)?(?:_r\d+)?$", name)
    return int(m.group(1)) if m and not m.group(2) else 1


def _split_candidates():
    """(index, name) of every candidate that writes split-K partials."""
    out = []
    for i in range(dlp.proj_num_candidates(M, N, K, dlp.EPI_NONE, dlp.OUT_F32)):
        name = dlp.proj_candidate_name(M, N, K, dlp.EPI_NONE, dlp.OUT_F32, i)
        if _splits(name) > 1:
            out.append((i, name))
    return out


def test_zero_workspace_plans_without_splits_and_refuses_split_candidates():
    print("zero-workspace context", flush=True)
    c = dlp.proj_create(0, 0)
    try:
        X, W = _inputs()
        Xd, Wd = dev_bf16(X), dev_bf16(W)
        r, _ = oracle.reference(X, W, None, oracle.EPI_NONE, oracle.OUT_F32)
        # tuned plan: only candidates without partials were timed
        Y = out_tensor(M, N, oracle.OUT_F32)
        dlp.proj_run(c, Xd, Wd, None, dlp.EPI_NONE, Y)
        plan = dlp.proj_get_plan(c, M, N, K, dlp.EPI_NONE, dlp.OUT_F32)
        print("plan with no workspace:", plan, flush=True)
        assert _splits(plan.split(" ")[0]) == 1, plan
        rep = compare.check(host_f64(Y), r)
        assert rep["ok"], rep
        splits = _split_candidates()
        assert splits
        for i, name in splits:
            Y2 = out_tensor(M, N, oracle.OUT_F32, fill=7.0)
            with pytest.raises(dlp.ProjError) as e:
                dlp.proj_run_candidate(c, i, Xd, Wd, None, dlp.EPI_NONE, Y2)
            assert e.value.status == dlp.PROJ_ERR_NO_MEMORY, name
            assert "workspace" in str(e.value)
            torch.cuda.synchronize()
            assert bool((Y2 == 7.0).all()), name   # nothing was enqueued
        # under capture: refused the same way, nothing recorded
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        Y3 = out_tensor(M, N, oracle.OUT_F32, fill=7.0)
        status = None
        with torch.cuda.graph(g, stream=s):
            try:
                dlp.proj_run_candidate(c, splits[0][0], Xd, Wd, None, dlp.EPI_NONE, Y3, stream=s)
            except dlp.ProjError as err:
                status = err.status
        assert status == dlp.PROJ_ERR_NO_MEMORY
        g.replay()
        torch.cuda.synchronize()
        assert bool((Y3 == 7.0).all())
        # a shape first seen under capture takes a default plan that fits
        X4, W4 = synth.normal_bf16((M, 2048), 1.0, 7200), synth.normal_bf16((512, 2048), 0.02, 7201)
        X4d, W4d = dev_bf16(X4), dev_bf16(W4)
        Y4 = out_tensor(M, 512, oracle.OUT_F32)
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2, stream=s):
            dlp.proj_run(c, X4d, W4d, None, dlp.EPI_NONE, Y4, stream=s)
        plan4 = dlp.proj_get_plan(c, M, 512, 2048, dlp.EPI_NONE, dlp.OUT_F32)
        print("default plan with no workspace:", plan4, flush=True)
        assert plan4.endswith("(default)") and _splits(plan4.split(" ")[0]) == 1, plan4
        g2.replay()
        r4, _ = oracle.reference(X4, W4, None, oracle.EPI_NONE, oracle.OUT_F32)
        rep4 = compare.check(host_f64(Y4), r4)
        assert rep4["ok"], rep4
        del g, g2
    finally:
        dlp.proj_destroy(c)


def test_small_workspace_keeps_only_fitting_splits():
    """A 256 KiB workspace holds S = 4 partials of [16][1024] fp32 exactly:
    those run, S = 8 and S = 16 are refused."""
    print("256 KiB workspace context", flush=True)
    c = dlp.proj_create(0, 256 << 10)
    try:
        X, W = _inputs(1)
        Xd, Wd = dev_bf16(X), dev_bf16(W)
        r, _ = oracle.reference(X, W, None, oracle.EPI_NONE, oracle.OUT_F32)
        seen = set()
        for i, name in _split_candidates():
            S = _splits(name)
            Y = out_tensor(M, N, oracle.OUT_F32)
            if S * M * N * 4 <= 256 << 10:
                dlp.proj_run_candidate(c, i, Xd, Wd, None, dlp.EPI_NONE, Y)
                rep = compare.check(host_f64(Y), r)
                assert rep["ok"], (name, rep)
                seen.add("ran")
            else:
                with pytest.raises(dlp.ProjError) as e:
                    dlp.proj_run_candidate(c, i, Xd, Wd, None, dlp.EPI_NONE, Y)
                assert e.value.status == dlp.PROJ_ERR_NO_MEMORY, name
                seen.add("refused")
        assert seen == {"ran", "refused"}
        Y = out_tensor(M, N, oracle.OUT_F32)
        dlp.proj_run(c, Xd, Wd, None, dlp.EPI_NONE, Y)
        plan = dlp.proj_get_plan(c, M, N, K, dlp.EPI_NONE, dlp.OUT_F32).split(" ")[0]
        print("plan with 256 KiB:", plan, flush=True)
        S = _splits(plan)
        assert S * M * N * 4 <= 256 << 10, plan
        assert compare.check(host_f64(Y), r)["ok"]
    finally:
        dlp.proj_destroy(c)


def test_tuner_flush_buffer_is_released():
    """The 512 MiB buffer the tuner reads to flush the caches while it times
    a small shape is freed before the tuning call returns."""
    print("flush buffer release", flush=True)
    c = dlp.proj_create(0)
    try:
        X, W = _inputs(2)
        Xd, Wd = dev_bf16(X), dev_bf16(W)
        Y = out_tensor(M, N, oracle.OUT_F32)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        dlp.proj_tune(c, Xd, Wd, None, dlp.EPI_NONE, Y)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        print("free before %d after %d" % (free0, free1), flush=True)
        assert free0 - free1 < (256 << 20)
    finally:
        dlp.proj_destroy(c)


def test_graph_of_destroyed_context_is_not_replayed():
    """A graph records its context's workspace: after proj_destroy of that
    context the graph is refused (PROJ_ERR_DESTROYED), nothing is enqueued,
    and the graph can still be destroyed."""
    print("graph after context destroy", flush=True)
    c = dlp.proj_create(0)
    X, W = _inputs(3)
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    r, _ = oracle.reference(X, W, None, oracle.EPI_NONE, oracle.OUT_F32)
    Y = out_tensor(M, N, oracle.OUT_F32)
    s = torch.cuda.Stream()
    g = dlp.proj_graph_capture(c, [Xd], [Wd], None, [Y], dlp.EPI_NONE, stream=s)
    Y.fill_(7.0)
    dlp.proj_graph_launch(g, stream=s)
    s.synchronize()
    assert compare.check(host_f64(Y), r)["ok"]
    dlp.proj_destroy(c)
    Y.fill_(7.0)
    torch.cuda.synchronize()
    with pytest.raises(dlp.ProjError) as e:
        dlp.proj_graph_launch(g, stream=s)
    assert e.value.status == dlp.PROJ_ERR_DESTROYED
    s.synchronize()
    assert bool((Y == 7.0).all())
    dlp.proj_graph_destroy(g)
    with pytest.raises(dlp.ProjError) as e:
        dlp.proj_graph_launch(g, stream=s)
    assert e.value.status == dlp.PROJ_ERR_DESTROYED
