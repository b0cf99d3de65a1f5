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
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor, require_gpu

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


# M = 512, N = 36864: 288 tiles of 256 x 256, 384 of 256 x 192 and 576 of
# 256 x 128, each a multiple of 8 and more than one per CU, so the
# persistent GEMM walks several tiles per workgroup through its XCD-
# contiguous renumbering; K = 8192 gives each tile 128 k-ranges of 64.
LK_M, LK_N, LK_K = 512, 36864, 8192


def test_k8192_every_candidate_exact_on_integers():
    """Every candidate plan at K = 8192 on a 512 x 36864 output, inputs in
    {-1, 0, 1} and an integer bias: all partial sums are integers below
    2^24, exact in fp32 in any order, so each plan must equal the oracle bit
    for bit -- fp32 output for every candidate, bf16 output (the staged
    16-byte store path of full GEMM tiles) for every GEMM candidate.  The
    context's workspace holds every split's partials."""
    require_gpu()
    print("K=8192 integer shape", LK_M, LK_N, LK_K, flush=True)
    X = synth.integer_bf16((LK_M, LK_K), -1, 1, 330)
    W = synth.integer_bf16((LK_N, LK_K), -1, 1, 331)
    b = synth.integer_bf16((LK_N,), -100, 100, 332)
    r32, s = oracle.reference(X, W, b, oracle.EPI_BIAS, oracle.OUT_F32)
    r16 = oracle.bf16_to_f64(oracle.round_out(s, oracle.OUT_BF16))
    assert np.array_equal(r32, s) and np.abs(s).max() < 2 ** 24
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    del W
    c = dlp.proj_create(0, 16 * LK_M * LK_N * 4)   # room for S = 16 partials
    try:
        Y32 = out_tensor(LK_M, LK_N, oracle.OUT_F32)
        Y16 = out_tensor(LK_M, LK_N, oracle.OUT_BF16)
        n = dlp.proj_num_candidates(LK_M, LK_N, LK_K, dlp.EPI_BIAS, oracle.OUT_F32)
        assert n > 0
        gemm_seen = 0
        for i in range(n):
            name = dlp.proj_candidate_name(LK_M, LK_N, LK_K, dlp.EPI_BIAS, oracle.OUT_F32, i)
            print(i, name, flush=True)
            Y32.fill_(float("nan"))
            dlp.proj_run_candidate(c, i, Xd, Wd, bd, dlp.EPI_BIAS, Y32)
            u = host_f64(Y32)
            bad = np.argwhere(u != r32)
            assert bad.size == 0, "%s fp32: first mismatch at %s: %r vs %r (%d bad)" % (
                name, bad[0], u[tuple(bad[0])], r32[tuple(bad[0])], len(bad))
            if not name.startswith("gemm"):
                continue
            gemm_seen += 1
            j = [dlp.proj_candidate_name(LK_M, LK_N, LK_K, dlp.EPI_BIAS, oracle.OUT_BF16, q)
                 for q in range(dlp.proj_num_candidates(LK_M, LK_N, LK_K, dlp.EPI_BIAS, oracle.OUT_BF16))].index(name)
            Y16.fill_(float("nan"))
            dlp.proj_run_candidate(c, j, Xd, Wd, bd, dlp.EPI_BIAS, Y16)
            u = host_f64(Y16)
            bad = np.argwhere(u != r16)
            assert bad.size == 0, "%s bf16: first mismatch at %s: %r vs %r (%d bad)" % (
                name, bad[0], u[tuple(bad[0])], r16[tuple(bad[0])], len(bad))
        assert gemm_seen >= 30
    finally:
        dlp.proj_destroy(c)
