"""fp32-weight projections through a bf16 high/low pair (the worklog's router
scheme, sections "Why the high-plus-low router scheme helped" and "The actual
error rule, including what L2 means"), against the oracle.

  - registration (proj_prepare_hilo) is bit-exact against the oracle's split;
  - integer inputs whose weights split exactly give bit-exact fp32 outputs;
  - every candidate plan, on shapes with ragged tiles, meets the element gate
    and the worklog's row rule at the router's 0.01% against the fp64 product
    with the fp32 weights themselves (not against H + L);
  - the six router shapes of the thirty-shape set, with sparse probe rows;
  - graph capture and replay of the tuned plan.
"""
import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def router_weights(N, K, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    W = rng.standard_normal((N, K), dtype=np.float32)
    W *= np.float32(1.0 / np.sqrt(K))
    return W


def reference_f32(X, W32, bias=None, epi=oracle.EPI_NONE, out_dtype=oracle.OUT_F32):
    s = oracle.proj_f64_w32(X, W32, bias, epi)
    r = oracle.round_out(s, out_dtype)
    if out_dtype == oracle.OUT_BF16:
        return oracle.bf16_to_f64(r)
    return r.astype(np.float64)


def whl_bits(Whl):
    torch.cuda.synchronize()
    return Whl.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("N,K", [(37, 200), (5, 1), (256, 8192)])
def test_prepare_bit_exact(ctx, N, K):
    print("prepare_hilo", N, K, flush=True)
    rng = np.random.default_rng(N * 7 + K)
    W = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-30, 30, (N, K)))).astype(np.float32)
    W.reshape(-1)[:4] = [1.00390625, -1.00390625, 0.0, 2.0 ** -140]   # page tie, zero, bf16 subnormal
    Whl = dlp.proj_prepare_hilo(ctx, dev_f32(W))
    hi, lo = oracle.hilo_split(W)
    assert np.array_equal(whl_bits(Whl), np.concatenate([hi, lo], axis=1))


def test_prepare_into_given_buffer_and_empty(ctx):
    W = router_weights(8, 64, 11)
    Whl = torch.full((8, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = dlp.proj_prepare_hilo(ctx, dev_f32(W), Whl)
    assert out.data_ptr() == Whl.data_ptr()
    hi, lo = oracle.hilo_split(W)
    assert np.array_equal(whl_bits(Whl), np.concatenate([hi, lo], axis=1))
    dlp.proj_prepare_hilo(ctx, torch.empty((0, 64), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        dlp.proj_prepare_hilo(ctx, dev_f32(W), torch.empty((8, 64), dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("M,N,K", [(16, 96, 256), (200, 130, 256), (3, 64, 128)])
def test_integer_bit_exact(ctx, M, N, K):
    """X in [-4, 4] and W = a + b 2^-10 (a in [-4, 4], b in [-3, 3]): the
    split is exact (H + L = W) and every fp32 partial sum is exact, so each
    candidate's fp32 output equals the oracle bit for bit."""
    print("hilo integer", M, N, K, flush=True)
    X = synth.integer_bf16((M, K), -4, 4, 700 + M)
    rng = np.random.default_rng(701 + N)
    W = (rng.integers(-4, 5, (N, K)) + rng.integers(-3, 4, (N, K)) * 2.0 ** -10).astype(np.float32)
    hi, lo = oracle.hilo_split(W)
    assert np.array_equal(oracle.bf16_to_f64(hi) + oracle.bf16_to_f64(lo), W.astype(np.float64))
    r = reference_f32(X, W)
    Xd, Whl = dev_bf16(X), dlp.proj_prepare_hilo(ctx, dev_f32(W))
    n = dlp.proj_num_candidates_hilo(M, N, K, dlp.EPI_NONE, oracle.OUT_F32)
    assert n >= 1
    for i in range(n):
        name = dlp.proj_candidate_name_hilo(M, N, K, dlp.EPI_NONE, oracle.OUT_F32, i)
        print("  candidate", name, flush=True)
        Y = out_tensor(M, N, oracle.OUT_F32)
        dlp.proj_run_candidate_hilo(ctx, i, Xd, Whl, None, dlp.EPI_NONE, Y)
        u = host_f64(Y)
        assert np.array_equal(u, r), (name, float(np.abs(u - r).max()))


CAND_SHAPES = [
    (1, 256, 8192), (5, 77, 512), (16, 300, 1024), (40, 200, 512), (64, 257, 640),
    (70, 333, 448), (260, 270, 192), (300, 256, 2048), (7, 50, 100),
]


@pytest.mark.parametrize("M,N,K", CAND_SHAPES)
def test_every_candidate(ctx, M, N, K):
    print("hilo candidates", M, N, K, flush=True)
    X = synth.with_probe_rows(synth.normal_bf16((M, K), 1.0, 800 + M), 801 + K)
    W = router_weights(N, K, 802 + N)
    r = reference_f32(X, W)
    Xd, Whl = dev_bf16(X), dlp.proj_prepare_hilo(ctx, dev_f32(W))
    probes = synth.probe_rows(M)
    n = dlp.proj_num_candidates_hilo(M, N, K, dlp.EPI_NONE, oracle.OUT_F32)
    for i in range(n):
        name = dlp.proj_candidate_name_hilo(M, N, K, dlp.EPI_NONE, oracle.OUT_F32, i)
        print("  candidate", name, flush=True)
        Y = out_tensor(M, N, oracle.OUT_F32)
        dlp.proj_run_candidate_hilo(ctx, i, Xd, Whl, None, dlp.EPI_NONE, Y)
        u = host_f64(Y)
        rep = compare.check(u, r)
        rows = compare.check_rows(u, r, compare.ROUTER_TOL, probes)
        assert rep["ok"] and rows["ok"], (name, rep, rows)


@pytest.mark.parametrize("epi,out_dtype", [(dlp.EPI_BIAS, oracle.OUT_F32), (dlp.EPI_BIAS_GELU_TANH, oracle.OUT_BF16),
                                           (dlp.EPI_GELU_TANH, oracle.OUT_F32)])
@pytest.mark.parametrize("M,N,K", [(16, 300, 1024), (260, 270, 192)])
def test_epilogues(ctx, M, N, K, epi, out_dtype):
    print("hilo epilogue", M, N, K, epi, out_dtype, flush=True)
    X = synth.normal_bf16((M, K), 1.0, 900 + M)
    W = router_weights(N, K, 901 + N)
    b = synth.normal_bf16((N,), float(np.sqrt(0.02)), 902)
    bias = b if epi in (dlp.EPI_BIAS, dlp.EPI_BIAS_GELU_TANH) else None
    r = reference_f32(X, W, bias, epi, out_dtype)
    Xd, Whl = dev_bf16(X), dlp.proj_prepare_hilo(ctx, dev_f32(W))
    bd = dev_bf16(b) if bias is not None else None
    n = dlp.proj_num_candidates_hilo(M, N, K, epi, out_dtype)
    for i in range(n):
        name = dlp.proj_candidate_name_hilo(M, N, K, epi, out_dtype, i)
        Y = out_tensor(M, N, out_dtype)
        dlp.proj_run_candidate_hilo(ctx, i, Xd, Whl, bd, epi, Y)
        u = host_f64(Y)
        rep = compare.check(u, r)
        assert rep["ok"], (name, rep)
        if out_dtype == oracle.OUT_F32:
            rows = compare.check_rows(u, r, compare.ROUTER_TOL)
            assert rows["ok"], (name, rows)


ROUTERS = [s for s in synth.sweep_shapes() if s.fp32_weights]


@pytest.mark.parametrize("shape", ROUTERS, ids=lambda s: s.name)
def test_router_shapes_tuned_plan(ctx, shape):
    print("router shape", shape.name, flush=True)
    X, W = synth.sweep_inputs(shape)
    X = synth.with_probe_rows(X, 7000 + shape.index)
    r = reference_f32(X, W)
    Xd, Whl = dev_bf16(X), dlp.proj_prepare_hilo(ctx, dev_f32(W))
    Y = out_tensor(shape.M, shape.N, oracle.OUT_F32)
    dlp.proj_run_hilo(ctx, Xd, Whl, None, dlp.EPI_NONE, Y)    # tunes, leaves the winner's result
    u1 = host_f64(Y)
    Y.fill_(float("nan"))
    dlp.proj_run_hilo(ctx, Xd, Whl, None, dlp.EPI_NONE, Y)    # the cached plan
    u2 = host_f64(Y)
    plan = dlp.proj_get_plan_hilo(ctx, shape.M, shape.N, shape.K, dlp.EPI_NONE, oracle.OUT_F32)
    for u in (u1, u2):
        rep = compare.check(u, r)
        rows = compare.check_rows(u, r, compare.ROUTER_TOL, synth.probe_rows(shape.M))
        print(shape.name, plan, rows, flush=True)
        assert rep["ok"] and rows["ok"], (plan, rep, rows)


def test_degenerate_and_errors(ctx):
    # K = 0: the empty sum, then the bias
    b = synth.normal_bf16((8,), 0.5, 1)
    Y = out_tensor(4, 8, oracle.OUT_F32)
    X = torch.empty((4, 0), dtype=torch.bfloat16, device="cuda")
    Whl = torch.empty((8, 0), dtype=torch.bfloat16, device="cuda")
    dlp.proj_run_hilo(ctx, X, Whl, dev_bf16(b), dlp.EPI_BIAS, Y)
    assert np.array_equal(host_f64(Y), np.tile(oracle.bf16_to_f64(b), (4, 1)))
    # M = 0 leaves Y untouched
    dlp.proj_run_hilo(ctx, torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                      torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda"), None, dlp.EPI_NONE,
                      torch.empty((0, 8), dtype=torch.float32, device="cuda"))
    # a bias epilogue without a bias is rejected
    with pytest.raises(RuntimeError):
        dlp.proj_run_hilo(ctx, torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda"),
                          torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda"), None, dlp.EPI_BIAS,
                          out_tensor(2, 8, oracle.OUT_F32))


def test_graph_replay(ctx):
    """The tuned plan captured in a torch CUDA graph; X is rewritten between
    replays and every replay is checked against the oracle."""
    M, N, K = 16, 256, 8192
    W = router_weights(N, K, 950)
    Whl = dlp.proj_prepare_hilo(ctx, dev_f32(W))
    X0 = synth.normal_bf16((M, K), 1.0, 951)
    Xd = dev_bf16(X0)
    Y = out_tensor(M, N, oracle.OUT_F32)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        dlp.proj_run_hilo(ctx, Xd, Whl, None, dlp.EPI_NONE, Y, stream=stream.cuda_stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            dlp.proj_run_hilo(ctx, Xd, Whl, None, dlp.EPI_NONE, Y, stream=stream.cuda_stream)
    for rep_i in range(3):
        X = synth.normal_bf16((M, K), 1.0, 960 + rep_i)
        Xd.copy_(dev_bf16(X))
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        u = host_f64(Y)
        r = reference_f32(X, W)
        rows = compare.check_rows(u, r, compare.ROUTER_TOL)
        assert compare.check(u, r)["ok"] and rows["ok"], (rep_i, rows)
