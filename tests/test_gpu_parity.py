"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle,
element by element.

* integer-valued inputs make every fp32 partial sum exact in any order, so
  every kernel variant must match the oracle bit for bit (fp32 and bf16
  outputs, with bias);
* random N(0, .) inputs are compared with |u - r| <= 2e-3 + 2e-2 |r|;
* every candidate plan of a shape is run (not only the tuned winner), at
  sizes that span several tiles and a ragged tail.
"""
import ctypes

import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu

EPIS = [oracle.EPI_NONE, oracle.EPI_BIAS, oracle.EPI_GELU, oracle.EPI_BIAS_GELU]


def run_candidate(ctx, i, Xd, Wd, bd, epi, M, N, K, out):
    Y = out_tensor(M, N, out)
    dlp.proj_run_candidate(ctx, i, Xd, Wd, bd if epi & 1 else None, epi, Y, M=M, N=N, K=K)
    return host_f64(Y)


def candidate_names(M, N, K, epi, out, aligned=True):
    n = dlp.proj_num_candidates(M, N, K, epi, out, aligned)
    return [dlp.proj_candidate_name(M, N, K, epi, out, i, aligned) for i in range(n)]


# shapes that span several tiles of every family and have ragged tails
INT_SHAPES = [
    (16, 200, 256),    # N not a multiple of 16
    (5, 77, 96),       # M < 16
    (5, 77, 512),      # M < 16, whole stages (buffer-resource copy path)
    (33, 130, 264),    # 3 m-tiles of 16, K % 32 == 8 (partial k-step)
    (64, 256, 1024),
    (1, 48, 4104),     # one token row, K % 32 == 8, many k-steps
    (300, 520, 512),   # large-M family, ragged M and N
    (257, 129, 128),
    (300, 256, 64),    # large-M family, a single 64-wide k-range
    (130, 200, 1024),  # streaming kernel in row blocks: the last holds 2 rows
    (385, 96, 512),    # 4 row blocks of 128 (7 of 64), the last holds 1 row
]


@pytest.mark.parametrize("shape", INT_SHAPES, ids=lambda s: "M%d_N%d_K%d" % s)
def test_every_candidate_bit_exact_on_integers(ctx, shape):
    M, N, K = shape
    X = synth.integer_bf16((M, K), -8, 8, 10 + M)
    W = synth.integer_bf16((N, K), -8, 8, 20 + N)
    b = synth.integer_bf16((N,), -64, 64, 30 + K)
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    for epi in (oracle.EPI_NONE, oracle.EPI_BIAS):
        for out in (oracle.OUT_F32, oracle.OUT_BF16):
            r, _ = oracle.reference(X, W, b if epi & 1 else None, epi, out)
            names = candidate_names(M, N, K, epi, out)
            assert names
            for i, name in enumerate(names):
                u = run_candidate(ctx, i, Xd, Wd, bd, epi, M, N, K, out)
                bad = np.argwhere(u != r)
                assert bad.size == 0, "%s epi=%d out=%d: first mismatch at %s: %r vs %r" % (
                    name, epi, out, bad[0], u[tuple(bad[0])], r[tuple(bad[0])])


RAND_SHAPES = [(16, 1040, 2048), (64, 200, 1024), (17, 64, 512), (520, 384, 640),
               (3, 1000, 2056),   # register-streaming GEMV: ragged chunk count (257 per row), N % 16 == 8
               (8, 300, 4096)]    # GEMV at its largest token count


@pytest.mark.parametrize("shape", RAND_SHAPES, ids=lambda s: "M%d_N%d_K%d" % s)
def test_every_candidate_within_tolerance_random(ctx, shape):
    M, N, K = shape
    X, W, b = synth.make_inputs(M, N, K, True, 7)
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    for epi in EPIS:
        out = oracle.OUT_BF16 if epi & 2 else oracle.OUT_F32
        r, _ = oracle.reference(X, W, b if epi & 1 else None, epi, out)
        for i, name in enumerate(candidate_names(M, N, K, epi, out)):
            u = run_candidate(ctx, i, Xd, Wd, bd, epi, M, N, K, out)
            rep = compare.check(u, r)
            assert rep["ok"], "%s epi=%d: %s" % (name, epi, rep)


def test_persistent_tile_walk(ctx):
    """More 256-row tiles than CUs, so persistent workgroups walk several
    tiles with the LDS ring running on across them; a ragged last tile row
    takes the element-wise epilogue between full tiles.  Integer inputs:
    every large-M candidate bit-exact; then GELU within tolerance."""
    M, N, K = 4196, 4352, 128
    X = synth.integer_bf16((M, K), -8, 8, 41)
    W = synth.integer_bf16((N, K), -8, 8, 42)
    b = synth.integer_bf16((N,), -64, 64, 43)
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    for epi, out in ((oracle.EPI_NONE, oracle.OUT_BF16), (oracle.EPI_BIAS, oracle.OUT_BF16),
                     (oracle.EPI_BIAS, oracle.OUT_F32)):
        r, _ = oracle.reference(X, W, b if epi & 1 else None, epi, out)
        names = candidate_names(M, N, K, epi, out)
        assert any(n.startswith("gemmpp64p") for n in names)
        for i, name in enumerate(names):
            u = run_candidate(ctx, i, Xd, Wd, bd, epi, M, N, K, out)
            bad = np.argwhere(u != r)
            assert bad.size == 0, "%s epi=%d out=%d: %d mismatches, first at %s: %r vs %r" % (
                name, epi, out, len(bad), bad[0], u[tuple(bad[0])], r[tuple(bad[0])])
    Xr, Wr, br = synth.make_inputs(M, N, K, True, 44)
    Xd, Wd, bd = dev_bf16(Xr), dev_bf16(Wr), dev_bf16(br)
    r, _ = oracle.reference(Xr, Wr, br, oracle.EPI_BIAS_GELU, oracle.OUT_BF16)
    for i, name in enumerate(candidate_names(M, N, K, oracle.EPI_BIAS_GELU, oracle.OUT_BF16)):
        if not name.startswith("gemmpp64"):
            continue
        u = run_candidate(ctx, i, Xd, Wd, bd, oracle.EPI_BIAS_GELU, M, N, K, oracle.OUT_BF16)
        rep = compare.check(u, r)
        assert rep["ok"], "%s: %s" % (name, rep)


def test_split_k_item_walk(ctx):
    """K-split candidates with more (tile, split) items than CUs, so
    persistent workgroups walk several items whose k-ranges differ; ragged
    last tile row and column.  Integer inputs: bit-exact (partials and their
    reduction are exact); then GELU with random inputs within tolerance."""
    # 3 x 31 tiles of 256 x 256 (ragged), 4 splits: 372 items; four fp32
    # partials fit the 64 MiB workspace
    M, N, K = 520, 7700, 512
    X = synth.integer_bf16((M, K), -8, 8, 51)
    W = synth.integer_bf16((N, K), -8, 8, 52)
    b = synth.integer_bf16((N,), -64, 64, 53)
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    for epi, out in ((oracle.EPI_BIAS, oracle.OUT_BF16), (oracle.EPI_NONE, oracle.OUT_F32)):
        r, _ = oracle.reference(X, W, b if epi & 1 else None, epi, out)
        names = candidate_names(M, N, K, epi, out)
        split = [(i, n) for i, n in enumerate(names) if "_s" in n and n.startswith("gemm")]
        assert any(n.endswith("_s4") for _, n in split)
        for i, name in split:
            u = run_candidate(ctx, i, Xd, Wd, bd, epi, M, N, K, out)
            bad = np.argwhere(u != r)
            assert bad.size == 0, "%s epi=%d out=%d: %d mismatches, first at %s: %r vs %r" % (
                name, epi, out, len(bad), bad[0], u[tuple(bad[0])], r[tuple(bad[0])])
    Xr, Wr, br = synth.make_inputs(M, N, K, True, 54)
    Xd, Wd, bd = dev_bf16(Xr), dev_bf16(Wr), dev_bf16(br)
    r, _ = oracle.reference(Xr, Wr, br, oracle.EPI_BIAS_GELU, oracle.OUT_BF16)
    for i, name in enumerate(candidate_names(M, N, K, oracle.EPI_BIAS_GELU, oracle.OUT_BF16)):
        if "_s" not in name or not name.startswith("gemm"):
            continue
        u = run_candidate(ctx, i, Xd, Wd, bd, oracle.EPI_BIAS_GELU, M, N, K, oracle.OUT_BF16)
        rep = compare.check(u, r)
        assert rep["ok"], "%s: %s" % (name, rep)


@pytest.mark.parametrize("M", [1, 15, 16, 17, 63, 64, 65, 127, 128, 129])
def test_token_counts_around_tile_edges(ctx, M):
    """Tuned plan (proj_run) at token counts on both sides of tile edges."""
    N, K = 272, 1024
    X, W, b = synth.make_inputs(M, N, K, True, 3)
    r, _ = oracle.reference(X, W, b, oracle.EPI_BIAS, oracle.OUT_BF16)
    Y = out_tensor(M, N, oracle.OUT_BF16)
    dlp.proj_run(ctx, dev_bf16(X), dev_bf16(W), dev_bf16(b), dlp.EPI_BIAS, Y)
    rep = compare.check(host_f64(Y), r)
    assert rep["ok"], rep


@pytest.mark.parametrize("M", [2047, 2048, 2049])
@pytest.mark.parametrize("N,epi,out", [(777, oracle.EPI_BIAS_GELU, oracle.OUT_BF16),
                                       (3072, oracle.EPI_BIAS, oracle.OUT_F32)],
                         ids=["N777_gelu_bf16", "N3072_bias_f32"])
def test_large_token_counts_around_tile_edges(ctx, M, N, epi, out):
    """Tuned plan (proj_run) on the large-M path at token counts on both sides
    of a 256-row tile edge, with an odd N (rows of Y not 16-byte aligned, a
    ragged last column tile) and with whole column tiles."""
    K = 1024
    X, W, b = synth.make_inputs(M, N, K, True, 60 + M)
    r, _ = oracle.reference(X, W, b, epi, out)
    Y = out_tensor(M, N, out)
    dlp.proj_run(ctx, dev_bf16(X), dev_bf16(W), dev_bf16(b), epi, Y)
    rep = compare.check(host_f64(Y), r)
    assert rep["ok"], (M, N, dlp.proj_get_plan(ctx, M, N, K, epi, out), rep)


def test_generic_path_unaligned_and_odd_k(ctx):
    """K % 8 != 0 and a 2-byte-offset X both route to the generic kernel and
    stay within tolerance."""
    for (M, N, K, off) in [(7, 33, 100, 0), (16, 64, 256, 1), (3, 5, 7, 1)]:
        X, W, b = synth.make_inputs(M, N, K, True, 5)
        r, _ = oracle.reference(X, W, b, oracle.EPI_BIAS_GELU, oracle.OUT_F32)
        Y = out_tensor(M, N, oracle.OUT_F32)
        Xd = dev_bf16(X, offset_elems=off)
        dlp.proj_run(ctx, Xd, dev_bf16(W), dev_bf16(b), dlp.EPI_BIAS_GELU_TANH, Y)
        rep = compare.check(host_f64(Y), r)
        assert rep["ok"], (M, N, K, off, rep)


def test_degenerate_sizes(ctx):
    import torch
    # M == 0 or N == 0: nothing is written
    Y = out_tensor(4, 4, oracle.OUT_F32, fill=7.0)
    W = dev_bf16(synth.normal_bf16((4, 32), 1.0, 1))
    X0 = dev_bf16(np.zeros((0, 32), np.uint16))
    dlp.proj_run(ctx, X0, W, None, 0, Y, M=0, N=4, K=32)
    assert torch.all(Y == 7.0).item()
    # K == 0: the empty sum, so Y = epilogue(bias)
    b = synth.values_to_bf16([1.5, -2.0, 0.25])
    Y = out_tensor(2, 3, oracle.OUT_F32)
    Xe = dev_bf16(np.zeros((2, 0), np.uint16))
    We = dev_bf16(np.zeros((3, 0), np.uint16))
    dlp.proj_run(ctx, Xe, We, dev_bf16(b), dlp.EPI_BIAS, Y, M=2, N=3, K=0)
    assert host_f64(Y).tolist() == [[1.5, -2.0, 0.25]] * 2
    dlp.proj_run(ctx, Xe, We, dev_bf16(b), dlp.EPI_BIAS_GELU_TANH, Y, M=2, N=3, K=0)
    r = oracle.round_out(oracle.gelu_tanh(np.array([1.5, -2.0, 0.25])), oracle.OUT_F32)
    assert compare.check(host_f64(Y)[0], r.astype(np.float64))["ok"]


def test_invalid_arguments_are_rejected(ctx):
    import torch
    W = dev_bf16(synth.normal_bf16((4, 32), 1.0, 1))
    X = dev_bf16(synth.normal_bf16((2, 32), 1.0, 2))
    Y = out_tensor(2, 4, oracle.OUT_F32)
    L = dlp.lib()
    args = lambda epi=0, M=2, out=0, bias=None, Yp=Y.data_ptr(): (
        ctx, X.data_ptr(), W.data_ptr(), bias, epi, M, 4, 32, Yp, out, None)
    assert L.proj_run(*args(M=-1)) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_run(*args(epi=7)) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_run(*args(out=5)) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_run(*args(epi=1)) == dlp.PROJ_ERR_INVALID_ARG        # bias missing
    assert L.proj_run(*args(Yp=None)) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_run(*args(Yp=Y.data_ptr() + 2)) == dlp.PROJ_ERR_INVALID_ARG  # fp32 Y misaligned
    assert b"bias" in L.proj_last_error(ctx) or L.proj_last_error(ctx)
    # Y sharing memory with an input (the plan measurement writes Y repeatedly)
    assert L.proj_run(*args(Yp=X.data_ptr())) == dlp.PROJ_ERR_INVALID_ARG
    assert b"overlaps" in L.proj_last_error(ctx)
    assert L.proj_run(*args(Yp=W.data_ptr() + 64)) == dlp.PROJ_ERR_INVALID_ARG
    b = dev_bf16(synth.normal_bf16((4,), 1.0, 3))
    assert L.proj_run(*args(epi=1, bias=b.data_ptr(), Yp=b.data_ptr())) == dlp.PROJ_ERR_INVALID_ARG
    big = torch.zeros(4096, dtype=torch.float32, device="cuda")   # disjoint halves of one allocation
    Xb = big[:32].view(torch.bfloat16)                              # 2 x 32 bf16 in the first 128 bytes
    assert L.proj_run(ctx, Xb.data_ptr(), W.data_ptr(), None, 0, 2, 4, 32, big[1024:].data_ptr(), 0,
                      None) == dlp.PROJ_OK
    torch.cuda.synchronize()


def test_nonfinite_inputs_propagate(ctx):
    M, N, K = 16, 64, 512
    X, W, _ = synth.make_inputs(M, N, K, False, 9)
    X = X.copy()
    X[3, 100] = 0x7FC0           # NaN
    X[5, 7] = 0x7F80             # +inf
    Y = out_tensor(M, N, oracle.OUT_F32, fill=0.0)
    dlp.proj_run(ctx, dev_bf16(X), dev_bf16(W), None, 0, Y)
    u = host_f64(Y)
    assert np.isnan(u[3]).all()
    assert (~np.isfinite(u[5])).all()
    others = [m for m in range(M) if m not in (3, 5)]
    assert np.isfinite(u[others]).all()


def test_destroyed_handles_are_reported():
    """A destroyed context or graph keeps a marker, so using it again, or
    destroying it a second time, returns PROJ_ERR_DESTROYED."""
    import torch
    L = dlp.lib()
    c = dlp.proj_create(0)
    X = dev_bf16(synth.normal_bf16((2, 32), 1.0, 4))
    W = dev_bf16(synth.normal_bf16((4, 32), 1.0, 5))
    Y = out_tensor(2, 4, oracle.OUT_F32)
    s = torch.cuda.Stream()
    g = dlp.proj_graph_capture(c, [X], [W], None, [Y], dlp.EPI_NONE, stream=s)
    dlp.proj_graph_launch(g, stream=s)
    s.synchronize()
    assert L.proj_graph_destroy(g) == dlp.PROJ_OK
    assert L.proj_graph_destroy(g) == dlp.PROJ_ERR_DESTROYED
    assert L.proj_graph_launch(g, None) == dlp.PROJ_ERR_DESTROYED
    assert L.proj_destroy(c) == dlp.PROJ_OK
    assert L.proj_destroy(c) == dlp.PROJ_ERR_DESTROYED
    assert L.proj_run(c, X.data_ptr(), W.data_ptr(), None, 0, 2, 4, 32, Y.data_ptr(), 0, None) == \
        dlp.PROJ_ERR_DESTROYED
    buf = ctypes.create_string_buffer(64)
    assert L.proj_get_plan(c, 2, 4, 32, 0, 0, 1, buf, 64) == dlp.PROJ_ERR_DESTROYED
    assert L.proj_last_error(c) == b""


def test_read_probe_reads_only(ctx):
    """The read floor probe: whole and ragged sizes (fewer chunks than one
    slab, a partial last slab) run and leave the buffer as it was; a
    misaligned buffer or size is rejected."""
    import torch
    buf = torch.arange(1 << 20, dtype=torch.float32, device="cuda")   # 4 MiB
    ref = buf.clone()
    L = dlp.lib()
    dlp.proj_read_probe(ctx, buf)
    for n in (16, 48, 4096 + 16, 3 * 2048 * 16 + 32, (1 << 22) - 16):
        assert L.proj_read_probe(ctx, buf.data_ptr(), n, None) == dlp.PROJ_OK
    assert L.proj_read_probe(ctx, buf.data_ptr(), 0, None) == dlp.PROJ_OK
    assert L.proj_read_probe(ctx, buf.data_ptr() + 4, 64, None) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_read_probe(ctx, buf.data_ptr(), 20, None) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_read_probe(ctx, None, 64, None) == dlp.PROJ_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)


def test_project_helper_allocates_and_matches(ctx):
    """dlp.project (allocates Y): bias + GELU to bf16 by default, fp32 on
    request, both within tolerance of the oracle; no bias means no bias."""
    import torch
    M, N, K = 16, 520, 1024
    X, W, b = synth.make_inputs(M, N, K, True, 17)
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    Y = dlp.project(ctx, Xd, Wd, bd, gelu=True)
    assert Y.dtype == torch.bfloat16 and tuple(Y.shape) == (M, N)
    r, _ = oracle.reference(X, W, b, oracle.EPI_BIAS_GELU, oracle.OUT_BF16)
    assert compare.check(host_f64(Y), r)["ok"]
    Y32 = dlp.project(ctx, Xd, Wd, out_dtype=dlp.OUT_F32)
    assert Y32.dtype == torch.float32
    r32, _ = oracle.reference(X, W, None, oracle.EPI_NONE, oracle.OUT_F32)
    assert compare.check(host_f64(Y32), r32)["ok"]


def test_two_contexts_on_two_streams(ctx):
    """Each context owns its split-K workspace, so split plans of two
    contexts may run at the same time on two streams.  A four-way split
    candidate runs 20 times on each of two contexts, interleaved across two
    streams; both results match the oracle bit for bit on integer inputs."""
    import torch
    M, N, K = 16, 1024, 8192
    names = candidate_names(M, N, K, oracle.EPI_NONE, oracle.OUT_F32)
    split = [i for i, x in enumerate(names) if x.startswith("stream_") and x.endswith("_s4")]
    assert split
    i = split[0]
    c2 = dlp.proj_create(0)
    try:
        runs = []
        for seed in (61, 71):
            X = synth.integer_bf16((M, K), -8, 8, seed)
            W = synth.integer_bf16((N, K), -8, 8, seed + 1)
            r = oracle.reference(X, W, None, oracle.EPI_NONE, oracle.OUT_F32)[0]
            runs.append((dev_bf16(X), dev_bf16(W), out_tensor(M, N, oracle.OUT_F32), r))
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        for _ in range(20):
            for c, (Xd, Wd, Y, _r), s in ((ctx, runs[0], s1), (c2, runs[1], s2)):
                dlp.proj_run_candidate(ctx=c, index=i, X=Xd, W=Wd, bias=None, epilogue=dlp.EPI_NONE, Y=Y,
                                       stream=s)
        torch.cuda.synchronize()
        for Xd, Wd, Y, r in runs:
            assert np.array_equal(host_f64(Y), r)
    finally:
        dlp.proj_destroy(c2)


@pytest.mark.parametrize("shape", [(8, 96, 512), (40, 96, 256), (300, 192, 128)],
                         ids=lambda s: "M%d_N%d_K%d" % s)
def test_nonfinite_inputs_propagate_every_candidate(ctx, shape):
    """IEEE propagation through every kernel family: a NaN in a row of X
    makes that row of Y all NaN, an infinity makes it all non-finite (inf
    or NaN, by the signs met), with bias and GELU too; other rows stay
    finite."""
    M, N, K = shape
    X, W, b = synth.make_inputs(M, N, K, True, 31)
    X = X.copy()
    X[3, K // 3] = 0x7FC0        # NaN
    X[5, 7] = 0x7F80             # +inf
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    others = [m for m in range(M) if m not in (3, 5)]
    for epi in (oracle.EPI_NONE, oracle.EPI_BIAS_GELU):
        for i, name in enumerate(candidate_names(M, N, K, epi, oracle.OUT_BF16)):
            u = run_candidate(ctx, i, Xd, Wd, bd, epi, M, N, K, oracle.OUT_BF16)
            assert np.isnan(u[3]).all(), name
            assert (~np.isfinite(u[5])).all(), name
            assert np.isfinite(u[others]).all(), name
