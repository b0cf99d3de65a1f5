"""HIP-graph capture and replay through the C ABI: a replay reads the X it
finds at replay time (worklog "How I made Muse's GPU projections 1.32x
faster in the Open Kernel Challenge", section "Fresh graph replay is a
correctness test too": [2,3] -> [5,8,5], then [3,1] -> [11,5,-3]), and
split-K partial sums are rebuilt by every replay."""
import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu


def test_replay_follows_fresh_input(ctx):
    import torch
    K = 32
    W = np.zeros((3, K))
    W[:, :2] = [[4, -1], [1, 2], [-2, 3]]
    X = np.zeros((1, K))
    X[0, :2] = [2, 3]
    Xd = dev_bf16(synth.values_to_bf16(X))
    Wd = dev_bf16(synth.values_to_bf16(W))
    Y = out_tensor(1, 3, oracle.OUT_F32)
    s = torch.cuda.Stream()
    g = dlp.proj_graph_capture(ctx, [Xd], [Wd], None, [Y], dlp.EPI_NONE, stream=s)
    try:
        dlp.proj_graph_launch(g, stream=s)
        s.synchronize()
        assert host_f64(Y).tolist() == [[5.0, 8.0, 5.0]]
        X[0, :2] = [3, 1]
        Xd.copy_(dev_bf16(synth.values_to_bf16(X)))
        torch.cuda.synchronize()
        dlp.proj_graph_launch(g, stream=s)
        s.synchronize()
        assert host_f64(Y).tolist() == [[11.0, 5.0, -3.0]]
    finally:
        dlp.proj_graph_destroy(g)


@pytest.mark.parametrize("shape", [(16, 1024, 8192), (16, 8192, 1024), (300, 640, 512),
                                   (1, 2304, 8192), (8, 1024, 4096), (130, 512, 1024)])
def test_graph_replays_match_oracle(ctx, shape):
    """Capture several calls over rotating buffers; replay with eager work
    and synchronisations in between, new X each time; check every replay."""
    import torch
    M, N, K = shape
    P = 3
    Ws = [synth.normal_bf16((N, K), 1.0 / np.sqrt(K), 50 + p) for p in range(P)]
    bs = [synth.normal_bf16((N,), 0.14, 60 + p) for p in range(P)]
    Xd = [dev_bf16(synth.normal_bf16((M, K), 1.0, 70 + p)) for p in range(P)]
    Wd = [dev_bf16(w) for w in Ws]
    bd = [dev_bf16(b) for b in bs]
    Ys = [out_tensor(M, N, oracle.OUT_BF16) for _ in range(P)]
    s = torch.cuda.Stream()
    g = dlp.proj_graph_capture(ctx, Xd, Wd, bd, Ys, dlp.EPI_BIAS, stream=s)
    try:
        for rep in range(4):
            Xs = [synth.normal_bf16((M, K), 1.0, 1000 * rep + p) for p in range(P)]
            for p in range(P):
                Xd[p].copy_(dev_bf16(Xs[p]))
            junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
            torch.cuda.synchronize()
            dlp.proj_graph_launch(g, stream=s)
            s.synchronize()
            del junk
            for p in range(P):
                r, _ = oracle.reference(Xs[p], Ws[p], bs[p], 1, 1)
                rep_ = compare.check(host_f64(Ys[p]), r)
                assert rep_["ok"], (rep, p, rep_)
    finally:
        dlp.proj_graph_destroy(g)
    plan = dlp.proj_get_plan(ctx, M, N, K, 1, 1)
    assert "tuned" in plan, plan


def test_capture_without_plan_uses_default(ctx, monkeypatch):
    """A first-seen shape under capture gets the untimed default plan."""
    import torch
    monkeypatch.setenv("PROJ_TUNE", "0")
    M, N, K = 16, 336, 2048
    X, W, b = synth.make_inputs(M, N, K, True, 21)
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    Y = out_tensor(M, N, oracle.OUT_BF16)
    s = torch.cuda.Stream()
    g = dlp.proj_graph_capture(ctx, [Xd], [Wd], [bd], [Y], dlp.EPI_BIAS, stream=s)
    try:
        for _ in range(3):
            dlp.proj_graph_launch(g, stream=s)
        s.synchronize()
    finally:
        dlp.proj_graph_destroy(g)
    assert "default" in dlp.proj_get_plan(ctx, M, N, K, 1, 1)
    r, _ = oracle.reference(X, W, b, 1, 1)
    assert compare.check(host_f64(Y), r)["ok"]


def test_tune_refused_under_capture_then_replaces_default(ctx):
    """Inside a stream capture, proj_tune returns PROJ_ERR_NOT_TUNED and
    enqueues nothing, while proj_run of a first-seen shape records the
    untimed default plan; the graph replays correctly.  Outside capture,
    proj_tune then replaces the default with a measured plan, and the
    result is the same within tolerance."""
    import torch
    M, N, K = 16, 272, 1536
    X, W, b = synth.make_inputs(M, N, K, True, 23)
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    Y = out_tensor(M, N, oracle.OUT_F32)
    L = dlp.lib()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = torch.cuda.current_stream().cuda_stream
        assert L.proj_tune(ctx, Xd.data_ptr(), Wd.data_ptr(), bd.data_ptr(), dlp.EPI_BIAS, M, N, K,
                           Y.data_ptr(), dlp.OUT_F32, st) == dlp.PROJ_ERR_NOT_TUNED
        assert L.proj_run(ctx, Xd.data_ptr(), Wd.data_ptr(), bd.data_ptr(), dlp.EPI_BIAS, M, N, K,
                          Y.data_ptr(), dlp.OUT_F32, st) == dlp.PROJ_OK
    r, _ = oracle.reference(X, W, b, oracle.EPI_BIAS, oracle.OUT_F32)
    for _ in range(3):
        Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert compare.check(host_f64(Y), r)["ok"]
    del g
    assert dlp.proj_get_plan(ctx, M, N, K, dlp.EPI_BIAS, dlp.OUT_F32).endswith("(default)")
    Y.fill_(float("nan"))
    dlp.proj_tune(ctx, Xd, Wd, bd, dlp.EPI_BIAS, Y)
    torch.cuda.synchronize()
    assert "tuned" in dlp.proj_get_plan(ctx, M, N, K, dlp.EPI_BIAS, dlp.OUT_F32)
    assert compare.check(host_f64(Y), r)["ok"]


def test_atomic_split_plans_replay_fresh_results(ctx):
    """Plans that zero Y with a kernel and add their split partials into it
    with atomics, captured in a graph: every replay, with eager work and a
    new X between replays, gives the oracle's result (no accumulation across
    replays, no memset node whose replays could go stale).  Integer inputs
    keep every order of the additions exact, so replays are compared bit for
    bit."""
    import torch
    M, N, K = 16, 1024, 8192
    names = [dlp.proj_candidate_name(M, N, K, dlp.EPI_BIAS, dlp.OUT_F32, i)
             for i in range(dlp.proj_num_candidates(M, N, K, dlp.EPI_BIAS, dlp.OUT_F32))]
    atomic = [(i, n) for i, n in enumerate(names) if "_atomic" in n]
    assert atomic
    W = synth.integer_bf16((N, K), -4, 4, 80)
    b = synth.integer_bf16((N,), -16, 16, 81)
    Wd, bd = dev_bf16(W), dev_bf16(b)
    Xd = dev_bf16(synth.integer_bf16((M, K), -4, 4, 82))
    Y = out_tensor(M, N, oracle.OUT_F32)
    s = torch.cuda.Stream()
    for i, name in atomic[::7] + atomic[-1:]:
        print("atomic plan in a graph:", name, flush=True)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            dlp.proj_run_candidate(ctx, i, Xd, Wd, bd, dlp.EPI_BIAS, Y, stream=s)
        for rep in range(4):
            X = synth.integer_bf16((M, K), -4, 4, 90 + rep)
            Xd.copy_(dev_bf16(X))
            Y.fill_(float(rep + 1))              # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            r, _ = oracle.reference(X, W, b, oracle.EPI_BIAS, oracle.OUT_F32)
            assert np.array_equal(host_f64(Y), r), (name, rep)
        del g
