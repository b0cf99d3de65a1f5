"""Identities the pages and the mathematics fix, checked on the GPU path for
every kernel variant: worked examples, the transposed product, linearity,
power-of-two scaling, one-hot probes, and fresh results on repeated calls
(split-K partials must not leak between calls)."""
import json
import os

import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def names(M, N, K, epi=0, out=0):
    return [dlp.proj_candidate_name(M, N, K, epi, out, i) for i in range(dlp.proj_num_candidates(M, N, K, epi, out))]


def run(ctx, i, X, W, M, N, K, bias=None, epi=0, out=0):
    Y = out_tensor(M, N, out)
    dlp.proj_run_candidate(ctx, i, X, W, bias, epi, Y, M=M, N=N, K=K)
    return host_f64(Y)


def pad_k(a, K):
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros((a.shape[0], K))
    out[:, :a.shape[1]] = a
    return out


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["projections"], ids=lambda c: c["name"])
def test_worked_examples_every_variant(ctx, case):
    """The pages' worked examples, zero-padded to K = 32 so the vector
    kernels take them (zero terms change no sum), on every variant."""
    X = synth.values_to_bf16(pad_k(case["X"], 32))
    W = synth.values_to_bf16(pad_k(case["W"], 32))
    M, N = X.shape[0], W.shape[0]
    want = np.array(case["Y"], dtype=np.float64)
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    for out in (oracle.OUT_F32, oracle.OUT_BF16):
        for i, nm in enumerate(names(M, N, 32, 0, out)):
            assert np.array_equal(run(ctx, i, Xd, Wd, M, N, 32, out=out), want), nm
    # and through the generic kernel at the pages' own K
    X0, W0 = synth.values_to_bf16(case["X"]), synth.values_to_bf16(case["W"])
    Y = out_tensor(M, N, oracle.OUT_F32)
    dlp.proj_run(ctx, dev_bf16(X0), dev_bf16(W0), None, 0, Y)
    assert np.array_equal(host_f64(Y), want)


def test_transposed_product_every_variant(ctx):
    """Y^T = W . X^T: swapping the operands gives the transposed result."""
    M, N, K = 48, 64, 512
    X = synth.integer_bf16((M, K), -8, 8, 1)
    W = synth.integer_bf16((N, K), -8, 8, 2)
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    ref = oracle.proj_f64(X, W)
    for i, nm in enumerate(names(N, M, K)):
        YT = run(ctx, i, Wd, Xd, N, M, K)
        assert np.array_equal(YT.T, ref), nm


def test_linearity_every_variant(ctx):
    M, N, K = 16, 80, 1024
    A = synth.integer_bf16((M, K), -4, 4, 3)
    B = synth.integer_bf16((M, K), -4, 4, 4)
    S = synth.values_to_bf16(oracle.bf16_to_f64(A) + oracle.bf16_to_f64(B))
    W = synth.integer_bf16((N, K), -8, 8, 5)
    Wd = dev_bf16(W)
    for i, nm in enumerate(names(M, N, K)):
        ya = run(ctx, i, dev_bf16(A), Wd, M, N, K)
        yb = run(ctx, i, dev_bf16(B), Wd, M, N, K)
        ys = run(ctx, i, dev_bf16(S), Wd, M, N, K)
        assert np.array_equal(ys, ya + yb), nm


def test_power_of_two_scaling_every_variant(ctx):
    """T(4X) = 4 T(X) bit for bit on random inputs: power-of-two scaling
    commutes with every fp32 rounding, so any fixed summation order keeps
    it -- split partials are combined in split order, not arrival order.
    Plans that add their partials into Y with atomics have no fixed order
    and are left out (their exactness is checked on integer inputs)."""
    M, N, K = 16, 96, 2048
    X, W, _ = synth.make_inputs(M, N, K, False, 11)
    X4 = synth.values_to_bf16(oracle.bf16_to_f64(X) * 4.0)
    Wd = dev_bf16(W)
    for i, nm in enumerate(names(M, N, K)):
        if "_atomic" in nm:
            continue
        y1 = run(ctx, i, dev_bf16(X), Wd, M, N, K)
        y4 = run(ctx, i, dev_bf16(X4), Wd, M, N, K)
        assert np.array_equal(y4, 4.0 * y1), nm
        assert np.array_equal(run(ctx, i, dev_bf16(X), Wd, M, N, K), y1), nm + " not reproducible"


def test_one_hot_probe_every_variant(ctx):
    """A token row equal to 2^j at feature k returns 2^j W[:, k] exactly."""
    M, N, K = 4, 64, 256
    W = synth.normal_bf16((N, K), 1.0, 12)
    Wd64 = oracle.bf16_to_f64(W)
    X = np.zeros((M, K))
    X[0, 0], X[1, 31], X[2, 200], X[3, K - 1] = 1.0, 8.0, 0.25, 2.0 ** -10
    Xb = synth.values_to_bf16(X)
    want = np.stack([Wd64[:, 0], 8 * Wd64[:, 31], 0.25 * Wd64[:, 200], 2.0 ** -10 * Wd64[:, K - 1]])
    for i, nm in enumerate(names(M, N, K)):
        assert np.array_equal(run(ctx, i, dev_bf16(Xb), dev_bf16(W), M, N, K), want), nm


def test_repeated_calls_give_fresh_results(ctx):
    """Call each split-K variant repeatedly with different inputs into the
    same Y: no result may accumulate into or leak from the previous call
    (with fp32 output this covers the plans that zero Y and add their
    partials into it with atomics)."""
    import torch
    M, N, K = 16, 128, 4096
    W = synth.integer_bf16((N, K), -8, 8, 13)
    Wd = dev_bf16(W)
    for out in (oracle.OUT_BF16, oracle.OUT_F32):
        nms = names(M, N, K, 1, out)
        if out == oracle.OUT_F32:
            assert any("_atomic" in nm for nm in nms)
        for i, nm in enumerate(nms):
            Y = out_tensor(M, N, out)
            for rep in range(3):
                X = synth.integer_bf16((M, K), -8, 8, 100 + rep)
                b = synth.integer_bf16((N,), -8, 8, 200 + rep)
                r, _ = oracle.reference(X, W, b, 1, out)
                dlp.proj_run_candidate(ctx, i, dev_bf16(X), Wd, dev_bf16(b), 1, Y, M=M, N=N, K=K)
                torch.cuda.synchronize()
                assert np.array_equal(host_f64(Y), r), (nm, rep)
