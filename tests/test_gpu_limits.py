"""Long reductions at the kernels' addressing limits: K = 2^20 with inputs in
{-1, 0, 1}, so every fp32 partial sum is an exact integer below 2^24 and
every candidate plan must equal the oracle bit for bit.  The weights of one
16-row tile then span 32 MiB, and a split covers up to half a million
columns."""
import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

K_LONG = 1 << 20


@pytest.mark.parametrize("M,N", [(16, 48), (3, 40), (70, 20)])
def test_long_k_every_candidate_exact(ctx, M, N):
    print("long K", M, N, K_LONG, flush=True)
    X = synth.integer_bf16((M, K_LONG), -1, 1, 300 + M)
    W = synth.integer_bf16((N, K_LONG), -1, 1, 301 + N)
    b = synth.integer_bf16((N,), -100, 100, 302)
    r, _ = oracle.reference(X, W, b, oracle.EPI_BIAS, oracle.OUT_F32)
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    n = dlp.proj_num_candidates(M, N, K_LONG, dlp.EPI_BIAS, oracle.OUT_F32)
    for i in range(n):
        name = dlp.proj_candidate_name(M, N, K_LONG, dlp.EPI_BIAS, oracle.OUT_F32, i)
        if name.startswith("gemm"):
            continue   # one 256-row tile walking 2^20 columns alone: seconds per run
        Y = out_tensor(M, N, oracle.OUT_F32)
        dlp.proj_run_candidate(ctx, i, Xd, Wd, bd, dlp.EPI_BIAS, Y)
        u = host_f64(Y)
        bad = np.argwhere(u != r)
        assert bad.size == 0, "%s: first mismatch at %s: %r vs %r" % (name, bad[0], u[tuple(bad[0])],
                                                                     r[tuple(bad[0])])


def test_long_k_tuned_plan(ctx):
    """proj_run tunes a long-K shape without launching the hopeless GEMM
    tiles (their compute bound is far above the streaming plans' times), and
    the plan it keeps gives the exact result."""
    import time
    M, N = 16, 48
    X = synth.integer_bf16((M, K_LONG), -1, 1, 320)
    W = synth.integer_bf16((N, K_LONG), -1, 1, 321)
    r, _ = oracle.reference(X, W, None, oracle.EPI_NONE, oracle.OUT_F32)
    Y = out_tensor(M, N, oracle.OUT_F32)
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    torch.cuda.synchronize()
    t0 = time.time()
    dlp.proj_run(ctx, Xd, Wd, None, dlp.EPI_NONE, Y)
    torch.cuda.synchronize()
    dt = time.time() - t0
    plan = dlp.proj_get_plan(ctx, M, N, K_LONG, dlp.EPI_NONE, oracle.OUT_F32)
    print("long-K tuning took %.2f s, plan %s" % (dt, plan), flush=True)
    assert not plan.startswith("gemm"), plan
    assert dt < 30, dt
    assert np.array_equal(host_f64(Y), r)


def test_long_k_hilo_pair_exact(ctx):
    """A hi/lo pair of depth 2^20 (X rows of 2^19): weights a + b 2^-10 split
    exactly, and every candidate equals the oracle bit for bit."""
    M, N, K = 5, 24, 1 << 19
    X = synth.integer_bf16((M, K), -1, 1, 310)
    rng = np.random.default_rng(311)
    W = (rng.integers(-1, 2, (N, K)) + rng.integers(-1, 2, (N, K)) * 2.0 ** -10).astype(np.float32)
    r = oracle.round_out(oracle.proj_f64_w32(X, W), oracle.OUT_F32).astype(np.float64)
    Xd = dev_bf16(X)
    Whl = dlp.proj_prepare_hilo(ctx, torch.from_numpy(W).cuda())
    n = dlp.proj_num_candidates_hilo(M, N, K, dlp.EPI_NONE, oracle.OUT_F32)
    assert n > 0
    for i in range(n):
        name = dlp.proj_candidate_name_hilo(M, N, K, dlp.EPI_NONE, oracle.OUT_F32, i)
        if name.startswith("gemm"):
            continue   # see above
        Y = out_tensor(M, N, oracle.OUT_F32)
        dlp.proj_run_candidate_hilo(ctx, i, Xd, Whl, None, dlp.EPI_NONE, Y)
        assert np.array_equal(host_f64(Y), r), name
