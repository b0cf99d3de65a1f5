"""GPU parity on seeded random shapes, candidate by candidate: every plan the
planner offers for a shape (the validity rules, not a hand-picked list) is
run through the C ABI and compared with the fp64 oracle on every element.
(test_gpu_random_shapes.py runs the tuned entry points on other random
shapes.)

The shapes are drawn once from a fixed seed across the three regimes the
planner spans (up to 8 token rows, up to 64, up to 512), with N and K from a
handful to about two thousand, K sometimes not a multiple of 8, X sometimes
not 16-byte aligned, every epilogue and both output types.  Inputs are
N(0, 1) X and N(0, 1/K) W, so the bar is |u - r| <= 2e-3 + 2e-2 |r|.
"""
import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu


def _cases(n=60, seed=20240611):
    rng = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        regime = len(out) % 3
        M = int(rng.randint(1, 9)) if regime == 0 else int(rng.randint(9, 65)) if regime == 1 else \
            int(rng.randint(65, 513))
        N = int(np.exp(rng.uniform(np.log(3), np.log(2100))))
        K = int(np.exp(rng.uniform(np.log(8), np.log(2100))))
        if rng.rand() < 0.75:
            K = max(8, K // 8 * 8)       # the aligned kernels' K rule
        if M * N * K > 3e8:              # keeps the oracle at a fraction of a second
            continue
        epi = int(rng.randint(0, 4))
        out_t = int(rng.randint(0, 2))
        off = 1 if rng.rand() < 0.15 else 0
        out.append((M, N, K, epi, out_t, off))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "M%d_N%d_K%d_e%d_o%d_x%d" % c)
def test_every_candidate_on_random_shape(ctx, case):
    M, N, K, epi, out, off = case
    print("random shape", case, flush=True)
    X, W, b = synth.make_inputs(M, N, K, True, 7000 + M + N + K)
    r, _ = oracle.reference(X, W, b, epi, out)
    Xd, Wd, bd = dev_bf16(X, offset_elems=off), dev_bf16(W), dev_bf16(b)
    aligned = off == 0 and K % 8 == 0
    n = dlp.proj_num_candidates(M, N, K, epi, out, aligned)
    assert n >= 1
    for i in range(n):
        name = dlp.proj_candidate_name(M, N, K, epi, out, i, aligned)
        Y = out_tensor(M, N, out)
        dlp.proj_run_candidate(ctx, i, Xd, Wd, bd if epi & 1 else None, epi, Y)
        rep = compare.check(host_f64(Y), r)
        assert rep["ok"], (case, name, rep)
    # and the plan the tuner keeps for it
    Y = out_tensor(M, N, out)
    dlp.proj_run(ctx, Xd, Wd, bd if epi & 1 else None, epi, Y)
    rep = compare.check(host_f64(Y), r)
    assert rep["ok"], (case, dlp.proj_get_plan(ctx, M, N, K, epi, out, aligned), rep)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "M%d_N%d_K%d_e%d_o%d_x%d" % c)
def test_every_candidate_exact_on_random_integer_shape(ctx, case):
    """The same shapes with integer inputs in [-8, 8] (bias in [-64, 64]):
    every partial sum is an exact integer below 2^24, so every candidate must
    equal the oracle bit for bit (GELU left out: it is not exact), which a
    tolerance would not guarantee for, say, one k-term dropped at large K."""
    M, N, K, epi, out, off = case
    epi &= 1
    print("random integer shape", case, flush=True)
    X = synth.integer_bf16((M, K), -8, 8, 7300 + M)
    W = synth.integer_bf16((N, K), -8, 8, 7301 + N)
    b = synth.integer_bf16((N,), -64, 64, 7302 + K)
    r, _ = oracle.reference(X, W, b, epi, out)
    Xd, Wd, bd = dev_bf16(X, offset_elems=off), dev_bf16(W), dev_bf16(b)
    aligned = off == 0 and K % 8 == 0
    n = dlp.proj_num_candidates(M, N, K, epi, out, aligned)
    for i in range(n):
        name = dlp.proj_candidate_name(M, N, K, epi, out, i, aligned)
        Y = out_tensor(M, N, out)
        dlp.proj_run_candidate(ctx, i, Xd, Wd, bd if epi else None, epi, Y)
        u = host_f64(Y)
        bad = np.argwhere(u != r)
        assert bad.size == 0, "%s %s: %d mismatches, first at %s: %r vs %r" % (
            case, name, len(bad), bad[0], u[tuple(bad[0])], r[tuple(bad[0])])


def _packed_cases(n=15, seed=20240612):
    rng = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        regime = len(out) % 3
        M = int(rng.randint(1, 17)) if regime == 0 else int(rng.randint(17, 65)) if regime == 1 else \
            int(rng.randint(65, 513))
        N = int(np.exp(rng.uniform(np.log(3), np.log(2100))))
        K = 128 * int(rng.randint(1, 17))
        if M * N * K > 3e8:
            continue
        tile16 = int(rng.choice([1, 2, 4, 7]))
        out.append((M, N, K, tile16, int(rng.randint(0, 4)), int(rng.randint(0, 2))))
    return out


PACKED_CASES = _packed_cases()


@pytest.mark.parametrize("case", PACKED_CASES, ids=lambda c: "M%d_N%d_K%d_t%d_e%d_o%d" % c)
def test_every_packed_candidate_on_random_shape(ctx, case):
    """The same on weights registered in the packed tile layout."""
    from tests.test_gpu_packed import run_all_packed
    M, N, K, tile16, epi, out = case
    print("random packed shape", case, flush=True)
    X, W, b = synth.make_inputs(M, N, K, True, 7100 + M + N + K)
    r, _ = oracle.reference(X, W, b, epi, out)
    for name, u in run_all_packed(ctx, X, W, b if epi & 1 else None, epi, out, tile16):
        rep = compare.check(u, r)
        assert rep["ok"], (case, name, rep)


def _hilo_cases(n=12, seed=20240613):
    rng = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        regime = len(out) % 3
        M = int(rng.randint(1, 17)) if regime == 0 else int(rng.randint(17, 257)) if regime == 1 else \
            int(rng.randint(257, 700))
        N = int(np.exp(rng.uniform(np.log(3), np.log(1500))))
        K = 8 * int(np.exp(rng.uniform(np.log(1), np.log(260))))
        if M * N * K > 2e8:
            continue
        out.append((M, N, K, int(rng.randint(0, 4)), int(rng.randint(0, 2))))
    return out


HILO_CASES = _hilo_cases()


@pytest.mark.parametrize("case", HILO_CASES, ids=lambda c: "M%d_N%d_K%d_e%d_o%d" % c)
def test_every_hilo_candidate_on_random_shape(ctx, case):
    """fp32 weights registered as a bf16 high/low pair: every candidate
    against the product with the fp32 weights themselves; with fp32 output
    and no GELU also the router's per-row rule at 0.01%."""
    from tests.test_gpu_hilo import dev_f32, reference_f32, router_weights
    M, N, K, epi, out = case
    print("random hi/lo shape", case, flush=True)
    X = synth.normal_bf16((M, K), 1.0, 7200 + M)
    W = router_weights(N, K, 7201 + N + K)
    b = synth.normal_bf16((N,), float(np.sqrt(0.02)), 7202)
    bias = b if epi & 1 else None
    r = reference_f32(X, W, bias, epi, out)
    Xd, Whl = dev_bf16(X), dlp.proj_prepare_hilo(ctx, dev_f32(W))
    bd = dev_bf16(b) if bias is not None else None
    n = dlp.proj_num_candidates_hilo(M, N, K, epi, out)
    assert n >= 1
    for i in range(n):
        name = dlp.proj_candidate_name_hilo(M, N, K, epi, out, i)
        Y = out_tensor(M, N, out)
        dlp.proj_run_candidate_hilo(ctx, i, Xd, Whl, bd, epi, Y)
        u = host_f64(Y)
        rep = compare.check(u, r)
        assert rep["ok"], (case, name, rep)
        if out == oracle.OUT_F32 and not epi & 2:
            rows = compare.check_rows(u, r, compare.ROUTER_TOL)
            assert rows["ok"], (case, name, rows)
