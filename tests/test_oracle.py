"""Pins for the fp64 oracle: what the pages and the mathematics fix, checked
against things other than the oracle itself (page values, exact rational
arithmetic, numpy's float64 matmul, torch's float64 GELU, IEEE bit layouts).

Each test names what a plausible mistake in the oracle would look like and
why it would fail here.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import compare

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def bits(values):
    return synth.values_to_bf16(values)


# ---------------------------------------------------------------- page values

@pytest.mark.parametrize("case", golden()["projections"], ids=lambda c: c["name"])
def test_worked_examples_exact(case):
    """Worked examples printed on the worklog (dropped terms, a wrong sign or a
    transposed operand all change these integers)."""
    X, W = bits(case["X"]), bits(case["W"])
    Y = oracle.proj_f64(X, W)
    assert Y.tolist() == [[float(v) for v in row] for row in case["Y"]]
    # both output roundings keep exact small integers
    assert oracle.round_out(Y, oracle.OUT_F32).astype(np.float64).tolist() == Y.tolist()
    assert oracle.bf16_to_f64(oracle.round_out(Y, oracle.OUT_BF16)).tolist() == Y.tolist()


def test_reduction_split_partials():
    """The 17 + 53 = 70 split: the sum over a K-range is the oracle on that
    slice, and the slices add to the whole."""
    case = [c for c in golden()["projections"] if c["name"] == "reduction_seventy"][0]
    X, W = np.array(case["X"]), np.array(case["W"])
    total = 0.0
    for part in case["split_partials"]:
        a, b = part["k"]
        v = oracle.proj_f64(bits(X[:, a:b]), bits(W[:, a:b]))[0, 0]
        assert v == part["value"]
        total += v
    assert total == case["Y"][0][0]


def test_storage_and_transpose_identity():
    """Row-major offsets n*K + k, and Y^T = W . X^T (swapping the operands of
    the oracle transposes its result exactly, term by term)."""
    g = golden()["storage"]
    W = np.array(g["W"])
    assert W.reshape(-1).tolist() == g["flat"]
    assert np.ascontiguousarray(W.T).reshape(-1).tolist() == g["transpose_copy_flat"]
    rng = np.random.default_rng(7)
    X = synth.normal_bf16((5, 37), 1.0, 11)
    Wb = synth.normal_bf16((9, 37), 0.2, 12)
    Y = oracle.proj_f64(X, Wb)
    YT = oracle.proj_f64(Wb, X)
    assert np.array_equal(Y.T, YT)
    del rng


def test_rel_l2_page_example():
    g = golden()["rel_l2"]
    assert abs(compare.rel_l2(g["u"], g["r"]) - g["value"]) < 1e-12


# ------------------------------------------------------- sums vs independent

def test_matches_numpy_float64_matmul():
    """numpy's float64 matmul is an independent library routine; bf16 inputs
    make every product exact in double, so the only difference is summation
    order: bounded by K * 2^-53 * sum|x w|."""
    for seed, (M, N, K) in enumerate([(1, 1, 1), (3, 5, 7), (16, 33, 64), (17, 31, 96), (64, 48, 129)]):
        X = synth.normal_bf16((M, K), 1.0, 100 + seed)
        W = synth.normal_bf16((N, K), 1.0 / math.sqrt(K), 200 + seed)
        Xd, Wd = oracle.bf16_to_f64(X), oracle.bf16_to_f64(W)
        ref = Xd @ Wd.T
        mag = np.abs(Xd) @ np.abs(Wd).T
        got = oracle.proj_f64(X, W, nthreads=3)
        assert np.all(np.abs(got - ref) <= 2 * K * 2.0 ** -53 * mag + 1e-300)


def test_exact_rational_brute_force_tiny():
    """Pure-Python exact rationals on tiny shapes: the oracle's double result
    is the correctly rounded sum to within K ulps."""
    X = synth.normal_bf16((3, 6), 1.0, 31)
    W = synth.normal_bf16((4, 6), 0.5, 32)
    b = synth.normal_bf16((4,), 0.1, 33)
    Xd, Wd, bd = oracle.bf16_to_f64(X), oracle.bf16_to_f64(W), oracle.bf16_to_f64(b)
    got = oracle.proj_f64(X, W, b, oracle.EPI_BIAS)
    for m in range(3):
        for n in range(4):
            exact = sum(Fraction(Xd[m, k]) * Fraction(Wd[n, k]) for k in range(6)) + Fraction(bd[n])
            mag = sum(abs(Fraction(Xd[m, k]) * Fraction(Wd[n, k])) for k in range(6)) + abs(Fraction(bd[n]))
            assert abs(Fraction(got[m, n]) - exact) <= Fraction(8 * 2 ** -53) * mag


def test_integer_inputs_exact_with_bias():
    """Integer inputs: every partial sum is exact in double, so the oracle
    equals numpy's result (and the bias is added once, not per split)."""
    X = synth.integer_bf16((7, 300), -8, 8, 41)
    W = synth.integer_bf16((11, 300), -8, 8, 42)
    b = synth.integer_bf16((11,), -100, 100, 43)
    Xd, Wd, bd = oracle.bf16_to_f64(X), oracle.bf16_to_f64(W), oracle.bf16_to_f64(b)
    assert np.array_equal(oracle.proj_f64(X, W, b, oracle.EPI_BIAS), Xd @ Wd.T + bd)
    assert np.array_equal(oracle.proj_f64(X, W), Xd @ Wd.T)


def test_linearity_and_power_of_two_scaling():
    """T(a + b) = T(a) + T(b) on integers, and T(2^j X) = 2^j T(X) exactly
    (power-of-two scaling commutes with every rounding in range)."""
    A = synth.integer_bf16((4, 50), -8, 8, 51)
    B = synth.integer_bf16((4, 50), -8, 8, 52)
    W = synth.integer_bf16((6, 50), -8, 8, 53)
    S = bits(oracle.bf16_to_f64(A) + oracle.bf16_to_f64(B))
    assert np.array_equal(oracle.proj_f64(S, W), oracle.proj_f64(A, W) + oracle.proj_f64(B, W))
    X = synth.normal_bf16((4, 64), 1.0, 54)
    W2 = synth.normal_bf16((6, 64), 0.125, 55)
    X8 = bits(oracle.bf16_to_f64(X) * 8.0)
    assert np.array_equal(oracle.proj_f64(X8, W2), 8.0 * oracle.proj_f64(X, W2))


def test_one_hot_probe_selects_weight_column():
    """A row that is 2^j at feature k and zero elsewhere returns 2^j W[:, k]."""
    K, N = 40, 13
    W = synth.normal_bf16((N, K), 1.0, 61)
    Wd = oracle.bf16_to_f64(W)
    X = np.zeros((3, K))
    X[0, 5] = 4.0
    X[1, 0] = 0.5
    X[2, K - 1] = 1.0
    Y = oracle.proj_f64(bits(X), W)
    assert np.array_equal(Y[0], 4.0 * Wd[:, 5])
    assert np.array_equal(Y[1], 0.5 * Wd[:, 0])
    assert np.array_equal(Y[2], Wd[:, K - 1])


def test_sampled_cells_equal_dense():
    X = synth.normal_bf16((9, 70), 1.0, 71)
    W = synth.normal_bf16((21, 70), 0.1, 72)
    b = synth.normal_bf16((21,), 0.1, 73)
    for epi in range(4):
        dense = oracle.proj_f64(X, W, b, epi)
        rows = np.array([0, 8, 3, 3, 5])
        cols = np.array([0, 20, 7, 8, 19])
        assert np.array_equal(oracle.proj_f64_at(X, W, rows, cols, b, epi), dense[rows, cols])


def test_degenerate_shapes():
    """K = 0: the empty sum is 0, so Y = epilogue(bias or 0).  M or N = 0:
    an empty result."""
    b = bits([1.5, -2.0, 0.25])
    X = np.zeros((2, 0), dtype=np.uint16)
    W = np.zeros((3, 0), dtype=np.uint16)
    assert oracle.proj_f64(X, W).tolist() == [[0.0] * 3] * 2
    assert oracle.proj_f64(X, W, b, oracle.EPI_BIAS).tolist() == [[1.5, -2.0, 0.25]] * 2
    g = oracle.proj_f64(X, W, b, oracle.EPI_BIAS_GELU)
    assert np.array_equal(g[0], oracle.gelu_tanh(np.array([1.5, -2.0, 0.25])))
    assert oracle.proj_f64(np.zeros((0, 4), np.uint16), synth.normal_bf16((3, 4), 1, 1)).shape == (0, 3)
    with pytest.raises(ValueError):
        oracle.proj_f64(np.zeros((2, 4), np.uint16), np.zeros((3, 5), np.uint16))
    with pytest.raises(ValueError):
        oracle.proj_f64(np.zeros((2, 4), np.uint16), np.zeros((3, 4), np.uint16), None, oracle.EPI_BIAS)


# ------------------------------------------------------------------ bf16 codec

def _bf16_from_fields(b: int) -> float:
    """bf16 decode written from the layout (1 sign, 8 exponent, 7 fraction
    bits), independent of any bit reinterpretation."""
    s = -1.0 if b >> 15 else 1.0
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    if e == 0xFF:
        return s * math.inf if f == 0 else math.nan
    if e == 0:
        return s * math.ldexp(f / 128.0, -126)
    return s * math.ldexp(1.0 + f / 128.0, e - 127)


def test_decode_all_bf16_patterns():
    allb = np.arange(65536, dtype=np.uint16)
    got = oracle.bf16_to_f64(allb)
    ref = np.array([_bf16_from_fields(int(b)) for b in allb])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_page_values():
    g = golden()["bf16"]
    # consecutive values and their spacing on [1, 2)
    c = g["consecutive"]
    assert c[1] - c[0] == g["spacing_1_2"] == c[2] - c[1]
    enc = oracle.f64_to_bf16(np.array(c))
    assert oracle.bf16_to_f64(enc).tolist() == c
    assert int(enc[1]) - int(enc[0]) == 1 and int(enc[2]) - int(enc[1]) == 1
    # the halfway value goes to the even neighbour; its residual is exact
    tie = oracle.bf16_to_f64(oracle.f64_to_bf16(np.array([g["tie_input"]])))[0]
    assert tie == g["tie_result"]
    res = g["tie_input"] - tie
    assert res == g["tie_residual"]
    assert oracle.bf16_to_f64(oracle.f64_to_bf16(np.array([res])))[0] == res


def test_bf16_direct_rounding_avoids_double_rounding():
    """Just above a tie in double, but exactly a tie once rounded to fp32:
    direct rounding must go up; a detour through fp32 would go to even."""
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle.bf16_to_f64(oracle.f64_to_bf16(np.array([x])))[0] == 1.0078125
    assert oracle.bf16_to_f64(oracle.f64_to_bf16(np.array([-x])))[0] == -1.0078125


def _bf16_rne_bit_trick(a32: np.ndarray) -> np.ndarray:
    """The usual integer formulation for fp32 -> bf16 RNE, with NaN kept quiet."""
    u = a32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a32)
    r[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return r


def test_bf16_encode_vs_bit_trick_on_fp32_inputs():
    """For inputs that are already fp32 values, direct RNE from double equals
    the integer fp32 -> bf16 formulation.  Every upper half (all exponents and
    fractions, both signs) with low halves on and around the rounding
    boundary."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFF,
                     0x1234, 0x7FFE, 0x8002, 0xC000], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).reshape(-1)
    a32 = pats.view(np.float32)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns widen quietly
        got = oracle.f64_to_bf16(a32.astype(np.float64))
    ref = _bf16_rne_bit_trick(a32)
    nan = np.isnan(a32)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7FC0) == 0x7FC0)   # quiet NaN stays NaN


def _nearest_bf16_exact(x: float) -> float:
    """Brute force with exact rationals: the nearest bf16 value to x, ties to
    the neighbour with an even fraction field."""
    if x == 0:
        return x
    a = abs(x)
    e = math.frexp(a)[1]
    q = max((e - 1) - 7, -133)
    unit = Fraction(2) ** q
    lo = (Fraction(a) / unit).__floor__()
    cands = [lo, lo + 1]
    best = None
    for c in cands:
        d = abs(Fraction(a) - c * unit)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    v = best[1] * unit
    if v >= Fraction(2) ** 128:
        return math.copysign(math.inf, x)
    return math.copysign(float(v), x)


def test_bf16_encode_vs_exact_rationals_on_doubles():
    rng = np.random.default_rng(5)
    xs = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.integers(-140, 128, 3000)),
        np.exp2(rng.uniform(-134, -120, 500)),          # subnormal bf16 region
        (1 + np.arange(0, 256) / 256.0) * 2.0 ** 5,     # exact ties at 2^5
        np.array([3.3895313892515355e38, 3.3961775292304173e38, 3.4e38, 1e39]),
    ])
    got = oracle.bf16_to_f64(oracle.f64_to_bf16(xs))
    ref = np.array([_nearest_bf16_exact(float(x)) for x in xs])
    assert np.array_equal(got, ref)


def test_fp32_rounding_vs_numpy():
    xs = np.random.default_rng(9).standard_normal(10000) * 1e3
    assert np.array_equal(oracle.round_out(xs, oracle.OUT_F32), xs.astype(np.float32))


# ------------------------------------------------------------------------ GELU

def test_gelu_tanh_vs_torch_float64():
    """torch's tanh-approximate GELU in float64 is an independent library
    routine; a mistyped constant (sqrt(2/pi), 0.044715, the 0.5) fails here."""
    torch = pytest.importorskip("torch")
    xs = np.linspace(-8, 8, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(xs), approximate="tanh").numpy()
    assert np.max(np.abs(oracle.gelu_tanh(xs) - ref)) < 1e-14


def test_gelu_identities_and_limits():
    xs = np.linspace(-6, 6, 2001)
    g = oracle.gelu_tanh(xs)
    gm = oracle.gelu_tanh(-xs)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.max(np.abs((g - gm) - xs)) < 1e-14          # odd-part identity
    big = np.array([20.0, 50.0])
    assert np.array_equal(oracle.gelu_tanh(big), big)
    assert np.all(np.abs(oracle.gelu_tanh(-big)) < 1e-300 + 1e-12)
    # close to the exact (erf) GELU everywhere, as an approximation must be
    erf = np.array([0.5 * x * (1 + math.erf(x / math.sqrt(2))) for x in xs])
    assert np.max(np.abs(g - erf)) < 1e-3


def test_epilogue_order_bias_then_gelu():
    X = synth.integer_bf16((3, 20), -3, 3, 81)
    W = synth.integer_bf16((5, 20), -3, 3, 82)
    b = synth.integer_bf16((5,), -4, 4, 83)
    plain = oracle.bf16_to_f64(X) @ oracle.bf16_to_f64(W).T
    bd = oracle.bf16_to_f64(b)
    assert np.array_equal(oracle.proj_f64(X, W, b, oracle.EPI_BIAS_GELU), oracle.gelu_tanh(plain + bd))
    assert np.array_equal(oracle.proj_f64(X, W, b, oracle.EPI_GELU), oracle.gelu_tanh(plain))


# -------------------------------------------- fp32 weights and the hi/lo pair

def test_hilo_page_example():
    """The halfway weight of the worklog's hi/lo section: the high part goes
    to the even neighbour 1.0 and the low part holds the residual exactly."""
    g = golden()["bf16"]
    hi, lo = oracle.hilo_split(np.array([g["tie_input"], -g["tie_input"]], np.float32))
    assert oracle.bf16_to_f64(hi).tolist() == [g["tie_result"], -g["tie_result"]]
    assert oracle.bf16_to_f64(lo).tolist() == [g["tie_residual"], -g["tie_residual"]]
    # 1.0 is 0x3F80; 2^-8 has biased exponent 119 and no fraction: 0x3B80
    assert hi.tolist() == [0x3F80, 0xBF80] and lo.tolist() == [0x3B80, 0xBB80]


def _hilo_weights():
    rng = np.random.default_rng(81)
    normal = rng.standard_normal(20000).astype(np.float32) * np.float32(1 / 90.5)
    scaled = (rng.standard_normal(5000) * np.exp2(rng.integers(-120, 120, 5000))).astype(np.float32)
    # exact bf16 ties and their neighbours: low 16 bits at 0x8000 +- 1
    top = rng.integers(0, 65536, 3000).astype(np.uint32) << 16
    ties = (top[:, None] | np.array([0x7FFF, 0x8000, 0x8001], np.uint32)).reshape(-1).view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) < 3e38)]
    tiny = (rng.standard_normal(2000) * 2.0 ** -130).astype(np.float32)   # bf16 subnormal range
    special = np.array([0.0, -0.0, 1.0, -2.0, 2.0 ** -126, 2.0 ** -149, 65504.0], np.float32)
    return np.concatenate([normal, scaled, ties, tiny, special])


def test_hilo_vs_bit_trick():
    """Independent formulation: the integer RNE on float32 bits for both
    parts, with the residual taken in numpy float32 (where it is exact)."""
    w = _hilo_weights()
    hi, lo = oracle.hilo_split(w)
    ref_hi = _bf16_rne_bit_trick(w)
    r32 = w - (ref_hi.astype(np.uint32) << 16).view(np.float32)
    ref_lo = _bf16_rne_bit_trick(r32)
    assert np.array_equal(hi, ref_hi)
    assert np.array_equal(lo, ref_lo)


def test_hilo_error_bounds():
    """Two roundings of unit roundoff 2^-8: |lo| <= 2^-8 |w| and
    |w - (hi + lo)| <= 2^-16 |w| for weights in the normal range; lo is zero
    exactly when w is itself a bf16 value; signs agree."""
    w = _hilo_weights()
    w = w[(np.abs(w) >= 2.0 ** -100) | (w == 0)]
    hi, lo = oracle.hilo_split(w)
    wd, hd, ld = w.astype(np.float64), oracle.bf16_to_f64(hi), oracle.bf16_to_f64(lo)
    assert np.all(np.abs(ld) <= 2.0 ** -8 * np.abs(wd))
    assert np.all(np.abs(wd - (hd + ld)) <= 2.0 ** -16 * np.abs(wd))
    is_bf16 = (w.view(np.uint32) & 0xFFFF) == 0
    assert np.array_equal(ld == 0, is_bf16)
    assert np.all(np.signbit(hd[wd != 0]) == np.signbit(wd[wd != 0]))


def test_hilo_recovers_constructed_pairs():
    """w = h + l, with h a bf16 value and l a bf16 value small enough that
    h is w's nearest bf16 value (|l| < 2^-9 of h's binade) and large enough
    that w is exact in fp32: the split returns (h, l) bit for bit.  A swapped
    pair or a residual of the wrong sign fails here."""
    rng = np.random.default_rng(82)
    n = 4000
    e = rng.integers(-40, 40, n)
    h = np.ldexp(1 + rng.integers(0, 128, n) / 128.0, e) * rng.choice([-1.0, 1.0], n)
    el = e - rng.integers(10, 17, n)
    l = np.ldexp(1 + rng.integers(0, 128, n) / 128.0, el) * rng.choice([-1.0, 1.0], n)
    w = (h + l).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), h + l)      # exact in fp32 by construction
    hi, lo = oracle.hilo_split(w)
    assert np.array_equal(oracle.bf16_to_f64(hi), h)
    assert np.array_equal(oracle.bf16_to_f64(lo), l)


def test_w32_matches_numpy_float64_matmul():
    """fp32 weights: bf16 x fp32 products are exact in double, so numpy's
    float64 matmul differs only by summation order."""
    for seed, (M, N, K) in enumerate([(1, 1, 1), (3, 5, 7), (16, 33, 64), (9, 20, 200)]):
        X = synth.normal_bf16((M, K), 1.0, 300 + seed)
        W = (np.random.default_rng(400 + seed).standard_normal((N, K)) / math.sqrt(K)).astype(np.float32)
        Xd, Wd = oracle.bf16_to_f64(X), W.astype(np.float64)
        ref = Xd @ Wd.T
        mag = np.abs(Xd) @ np.abs(Wd).T
        got = oracle.proj_f64_w32(X, W, nthreads=2)
        assert np.all(np.abs(got - ref) <= 2 * K * 2.0 ** -53 * mag + 1e-300)


def test_w32_exact_rationals_and_bias():
    X = synth.normal_bf16((2, 5), 1.0, 91)
    W = (np.random.default_rng(92).standard_normal((3, 5))).astype(np.float32)
    b = synth.normal_bf16((3,), 0.5, 93)
    Xd, bd = oracle.bf16_to_f64(X), oracle.bf16_to_f64(b)
    got = oracle.proj_f64_w32(X, W, b, oracle.EPI_BIAS)
    for m in range(2):
        for n in range(3):
            terms = [Fraction(Xd[m, k]) * Fraction(float(W[n, k])) for k in range(5)]
            exact = sum(terms) + Fraction(bd[n])
            mag = sum(abs(t) for t in terms) + abs(Fraction(bd[n]))
            assert abs(Fraction(got[m, n]) - exact) <= Fraction(8 * 2 ** -53) * mag
    gg = oracle.proj_f64_w32(X, W, b, oracle.EPI_BIAS_GELU)
    assert np.array_equal(gg, oracle.gelu_tanh(got))


def test_w32_agrees_with_bf16_oracle_on_bf16_weights():
    """Weights that are bf16 values give the same doubles through either
    weight format (same products, same order)."""
    X = synth.normal_bf16((6, 130), 1.0, 94)
    Wb = synth.normal_bf16((7, 130), 0.1, 95)
    W32 = oracle.bf16_to_f64(Wb).astype(np.float32)
    assert np.array_equal(oracle.proj_f64_w32(X, W32), oracle.proj_f64(X, Wb))


def test_hilo_product_meets_router_tolerance():
    """The scheme itself: X (hi + lo)^T, computed exactly by the bf16 oracle
    on the paired layout [hi | lo] with X repeated, differs from the fp32
    reference by at most 2^-16 sum |x w| per cell, far inside the router's
    0.01% relative L2."""
    M, N, K = 8, 64, 512
    X = synth.normal_bf16((M, K), 1.0, 96)
    W = (np.random.default_rng(97).standard_normal((N, K)) / math.sqrt(K)).astype(np.float32)
    hi, lo = oracle.hilo_split(W)
    pair = oracle.proj_f64(np.concatenate([X, X], axis=1), np.concatenate([hi, lo], axis=1))
    ref = oracle.proj_f64_w32(X, W)
    mag = np.abs(oracle.bf16_to_f64(X)) @ np.abs(W.astype(np.float64)).T
    assert np.all(np.abs(pair - ref) <= 2.0 ** -16 * mag * (1 + 1e-9))
    assert compare.rel_l2(pair, ref) < 1e-5


# ------------------------------------------------------------------ comparator

def test_comparator_rule():
    r = np.array([0.0, 1.0, -10.0, 100.0])
    ok = r + np.array([2e-3, 2.2e-2 * 0.999, -0.202 * 0.999, 2.002 * 0.999])
    assert compare.check(ok, r)["ok"]
    bad = r.copy()
    bad[3] += 2.1
    rep = compare.check(bad, r)
    assert not rep["ok"] and rep["n_bad"] == 1
    assert not compare.check(np.array([np.nan, 1, -10, 100.0]), r)["ok"]
    assert not compare.check(np.array([np.inf, 1, -10, 100.0]), r)["ok"]


def test_row_rule():
    """The worklog's row rule: whole-output relative L2 within the
    tolerance, each row within five times it against max(own norm, a tenth
    of the mean row norm), sparse probe rows within 0.1%."""
    g = golden()["rel_l2"]
    r = np.array([g["r"]], dtype=np.float64)
    u = np.array([g["u"]], dtype=np.float64)
    assert abs(compare.check_rows(u, r, tol=1.0)["rel_l2"] - g["value"]) < 1e-12
    assert compare.check_rows(u, r, tol=0.0101)["ok"]
    assert not compare.check_rows(u, r, tol=0.0099)["ok"]
    rng = np.random.default_rng(3)
    r = rng.standard_normal((100, 64))
    u = r * (1 + 1e-6)
    assert compare.check_rows(u, r)["ok"]
    # one bad row hidden in a good average: 6e-4 relative on a single row
    bad = u.copy()
    bad[5] = r[5] * (1 + 6e-4)
    rep = compare.check_rows(bad, r)
    assert rep["rel_l2"] <= compare.ROUTER_TOL and not rep["ok"]
    # a near-zero row is judged against a tenth of the mean row norm
    r2 = r.copy()
    r2[9] = 1e-9
    u2 = r2.copy()
    u2[9] += 1e-5
    assert compare.check_rows(u2, r2)["ok"]
    # probe rows: 0.1% of their own norm
    u3 = r.copy()
    u3[7] = r[7] * (1 + 2e-4)
    assert compare.check_rows(u3, r, tol=1e-3, probe_rows=[7])["ok"]
    u3[7] = r[7] * (1 + 2e-3)
    assert not compare.check_rows(u3, r, tol=1e-2, probe_rows=[7])["ok"]
    assert not compare.check_rows(np.full((2, 2), np.nan), np.ones((2, 2)))["ok"]
    assert not compare.check_rows(np.ones((2, 3)), np.ones((2, 2)))["ok"]
