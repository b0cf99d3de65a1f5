"""The seeded input generator: deterministic, shaped and scaled as stated."""
import numpy as np

import synth


def test_deterministic_and_distinct_seeds():
    a = synth.normal_bf16((4, 300), 1.0, 5)
    b = synth.normal_bf16((4, 300), 1.0, 5)
    c = synth.normal_bf16((4, 300), 1.0, 6)
    assert a.dtype == np.uint16 and a.shape == (4, 300)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_chunked_draw_equals_single_draw():
    n = (1 << 20) + 12345
    got = synth.normal_bf16((n,), 0.5, 77)
    rng = np.random.Generator(np.random.PCG64(77))
    x = rng.standard_normal(size=n, dtype=np.float32) * np.float32(0.5)
    assert np.array_equal(got, synth.f32_to_bf16_bits(x))


def test_workload_scales():
    X, W, b = synth.make_inputs(16, 512, 4096, True, 1)
    f = lambda u: (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(f(X).std() - 1.0) < 0.02
    assert abs(f(W).std() * np.sqrt(4096) - 1.0) < 0.02
    assert abs(f(b).std() - np.sqrt(0.02)) < 0.02
    assert [w.M for w in synth.WORKLOADS] == [16, 16, 64, 8192, 4096]
    assert synth.WORKLOADS[0].alg_bytes() == 17104896
    assert synth.WORKLOADS[4].alg_flops() == 549755813888


def test_bf16_rounding_of_inputs():
    # halfway cases go to the even neighbour
    v = np.array([1.00390625, 1.01171875, -1.00390625], dtype=np.float32)
    assert synth.f32_to_bf16_bits(v).tolist() == [0x3F80, 0x3F82, 0xBF80]


def test_sweep_shapes_follow_the_table():
    shapes = synth.sweep_shapes()
    assert len(shapes) == 30
    assert sorted({s.M for s in shapes}) == [1, 8, 16, 32, 128, 256]
    fam = {(s.family, s.M): s for s in shapes}
    for M in synth.SWEEP_LOADS:
        assert (fam[("qkv_gate", M)].N, fam[("qkv_gate", M)].K) == (2304, 8192)
        assert (fam[("output", M)].N, fam[("output", M)].K) == (8192, 1024)
        assert (fam[("pooler", M)].N, fam[("pooler", M)].K) == (4096, 8192)
        # the worklog's thirty-shape timing table: 1 / 1,024 / 4,096 and
        # 8 / 1,024 / 4,096; every other load 8,192 / 4,096
        assert fam[("unpooler", M)].K == 4096 and fam[("unpooler", M)].N == (1024 if M in (1, 8) else 8192)
        r = fam[("router", M)]
        assert (r.N, r.K, r.fp32_weights) == (256, 8192, True)
    assert [fam[("unpooler", M)].N for M in (1, 8, 16, 32, 128, 256)] == [1024, 1024, 8192, 8192, 8192, 8192]
    X, W = synth.sweep_inputs(fam[("router", 1)])
    assert X.dtype == np.uint16 and W.dtype == np.float32 and W.shape == (256, 8192)
    assert abs(W.std() * np.sqrt(8192) - 1.0) < 0.02
