"""Seeded random shapes through the tuned entry points (the plan the tuner
keeps for each shape), against the oracle: token counts from 1 to 600 (the
GEMV, streaming, row-block and GEMM regimes), ragged N and K (including K not
a multiple of 8 and pointers off 16-byte alignment, which take the any-shape
kernel), every epilogue and both output types; then fp32 weights through the
hi/lo pair and bf16 weights through the packed layout."""
import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([rng.integers(1, 9), rng.integers(9, 65), rng.integers(65, 600)]))
        N = int(rng.integers(1, 700))
        K = int(rng.choice([8 * rng.integers(1, 256), rng.integers(1, 300)]))
        out.append((M, N, K, int(rng.integers(0, 4)), int(rng.integers(0, 2)), bool(rng.random() < 0.2)))
    return out


@pytest.mark.parametrize("M,N,K,epi,out,misaligned", _shapes(2024, 30),
                         ids=lambda v: str(v))
def test_random_shape_tuned_plan(ctx, M, N, K, epi, out, misaligned):
    print("random shape", M, N, K, epi, out, misaligned, flush=True)
    X, W, b = synth.make_inputs(M, N, K, True, 40 + M + N)
    bias = b if epi & 1 else None
    r, _ = oracle.reference(X, W, bias, epi, out)
    off = 1 if misaligned else 0    # one bf16 element: 2-byte aligned, not 16
    Xd, Wd = dev_bf16(X, off), dev_bf16(W, off)
    bd = dev_bf16(b) if bias is not None else None
    Y = out_tensor(M, N, out)
    dlp.proj_run(ctx, Xd, Wd, bd, epi, Y)
    rep = compare.check(host_f64(Y), r)
    if not rep["ok"]:
        try:
            plan = dlp.proj_get_plan(ctx, M, N, K, epi, out, aligned16=not misaligned and K % 8 == 0)
        except dlp.ProjError as e:
            plan = str(e)
        raise AssertionError((plan, rep))


def _router_shapes(seed, n):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 300)), int(rng.integers(1, 400)), int(64 * rng.integers(1, 64))) for _ in range(n)]


@pytest.mark.parametrize("M,N,K", _router_shapes(7, 8), ids=lambda v: str(v))
def test_random_hilo_shape(ctx, M, N, K):
    print("random hilo", M, N, K, flush=True)
    X = synth.normal_bf16((M, K), 1.0, 50 + M)
    W = (np.random.default_rng(51 + N).standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    r = oracle.round_out(oracle.proj_f64_w32(X, W), oracle.OUT_F32).astype(np.float64)
    Whl = dlp.proj_prepare_hilo(ctx, torch.from_numpy(W).cuda())
    Y = out_tensor(M, N, oracle.OUT_F32)
    dlp.proj_run_hilo(ctx, dev_bf16(X), Whl, None, dlp.EPI_NONE, Y)
    u = host_f64(Y)
    rows = compare.check_rows(u, r, compare.ROUTER_TOL)
    assert compare.check(u, r)["ok"] and rows["ok"], rows


def _packed_shapes(seed, n):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 513)), int(rng.integers(1, 600)), int(128 * rng.integers(1, 24)),
             int(rng.choice([1, 2, 4, 7]))) for _ in range(n)]


@pytest.mark.parametrize("M,N,K,tile16", _packed_shapes(11, 8), ids=lambda v: str(v))
def test_random_packed_shape(ctx, M, N, K, tile16):
    print("random packed", M, N, K, tile16, flush=True)
    X, W, b = synth.make_inputs(M, N, K, True, 60 + M)
    r, _ = oracle.reference(X, W, b, oracle.EPI_BIAS_GELU, oracle.OUT_BF16)
    Wp = dlp.proj_pack_weights(ctx, dev_bf16(W), tile16)
    Y = out_tensor(M, N, oracle.OUT_BF16)
    dlp.proj_run_packed(ctx, dev_bf16(X), Wp, tile16, dev_bf16(b), dlp.EPI_BIAS_GELU_TANH, Y, N)
    rep = compare.check(host_f64(Y), r)
    assert rep["ok"], rep
