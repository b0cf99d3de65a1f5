"""bf16 weights registered in the packed tile layout (worklog, section
"Weight packing and library descriptors solve related but different
problems"): the packing is a bit-exact re-layout, and every plan that reads
packed weights matches the oracle as the row-major path does.

The expected packed array is built here with numpy from the layout's
definition (include/proj.h): tiles of R rows, each as K/128 blocks of
[R rows][128 columns], rows past N zero."""
import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def packed_reference(W: np.ndarray, tile16: int) -> np.ndarray:
    N, K = W.shape
    R = 16 * tile16
    tiles = -(-N // R)
    padded = np.zeros((tiles * R, K), dtype=np.uint16)
    padded[:N] = W
    return padded.reshape(tiles, R, K // 128, 128).transpose(0, 2, 1, 3).reshape(-1)


def bits_of(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


@pytest.mark.parametrize("N,K,tile16", [(100, 256, 1), (100, 256, 7), (300, 1024, 2), (8192, 1024, 4), (37, 128, 2)])
def test_pack_is_the_layout(ctx, N, K, tile16):
    print("pack", N, K, tile16, flush=True)
    rng = np.random.default_rng(N + K + tile16)
    W = rng.integers(0, 65536, (N, K)).astype(np.uint16)
    W[(W & 0x7F80) == 0x7F80] = 0x3F80          # keep the bits finite (pattern check only)
    Wp = dlp.proj_pack_weights(ctx, dev_bf16(W), tile16)
    assert Wp.numel() * 2 == dlp.proj_packed_bytes(N, K, tile16)
    assert np.array_equal(bits_of(Wp), packed_reference(W, tile16))


def run_all_packed(ctx, X, W, b, epi, out, tile16):
    M, K = X.shape
    N = W.shape[0]
    Xd, bd = dev_bf16(X), (dev_bf16(b) if b is not None else None)
    Wp = dlp.proj_pack_weights(ctx, dev_bf16(W), tile16)
    n = dlp.proj_num_candidates_packed(M, N, K, tile16, epi, out)
    assert n > 0
    for i in range(n):
        name = dlp.proj_candidate_name_packed(M, N, K, tile16, epi, out, i)
        Y = out_tensor(M, N, out)
        dlp.proj_run_candidate_packed(ctx, i, Xd, Wp, tile16, bd, epi, Y, N)
        yield name, host_f64(Y)


INT_CASES = [
    (16, 200, 256, 1),     # ragged last tile
    (5, 77, 512, 2),       # M < 16
    (64, 250, 1024, 7),    # 112-row tiles, ragged
    (130, 200, 1024, 4),   # row blocks, the last holding 2 rows
    (33, 130, 384, 2),     # K = 3 x 128
]


@pytest.mark.parametrize("M,N,K,tile16", INT_CASES)
def test_every_packed_candidate_bit_exact_on_integers(ctx, M, N, K, tile16):
    print("packed integer", M, N, K, tile16, flush=True)
    X = synth.integer_bf16((M, K), -8, 8, 40 + M)
    W = synth.integer_bf16((N, K), -8, 8, 41 + N)
    b = synth.integer_bf16((N,), -64, 64, 42)
    for epi, out in ((oracle.EPI_NONE, oracle.OUT_F32), (oracle.EPI_BIAS, oracle.OUT_BF16)):
        r, _ = oracle.reference(X, W, b if epi & 1 else None, epi, out)
        for name, u in run_all_packed(ctx, X, W, b if epi & 1 else None, epi, out, tile16):
            bad = np.argwhere(u != r)
            assert bad.size == 0, "%s epi=%d: first mismatch at %s" % (name, epi, bad[0])


def test_packed_random_with_gelu(ctx):
    M, N, K, tile16 = 16, 1040, 2048, 2
    X, W, b = synth.make_inputs(M, N, K, True, 7)
    r, _ = oracle.reference(X, W, b, oracle.EPI_BIAS_GELU, oracle.OUT_BF16)
    for name, u in run_all_packed(ctx, X, W, b, oracle.EPI_BIAS_GELU, oracle.OUT_BF16, tile16):
        rep = compare.check(u, r)
        assert rep["ok"], (name, rep)


@pytest.mark.parametrize("M,N,K,tile16", [(64, 2048, 4096, 7), (16, 4096, 8192, 2), (200, 1024, 2048, 4)])
def test_tuned_packed_plan(ctx, M, N, K, tile16):
    """proj_run_packed tunes, caches and reruns; results agree with the
    oracle and with the row-major path."""
    print("packed tuned", M, N, K, tile16, flush=True)
    X, W, b = synth.make_inputs(M, N, K, True, 8)
    r, _ = oracle.reference(X, W, b, oracle.EPI_BIAS, oracle.OUT_BF16)
    Xd, Wd, bd = dev_bf16(X), dev_bf16(W), dev_bf16(b)
    Wp = dlp.proj_pack_weights(ctx, Wd, tile16)
    for _ in range(2):
        Y = out_tensor(M, N, oracle.OUT_BF16)
        dlp.proj_run_packed(ctx, Xd, Wp, tile16, bd, dlp.EPI_BIAS, Y, N)
        rep = compare.check(host_f64(Y), r)
        assert rep["ok"], rep
    plan = dlp.proj_get_plan_packed(ctx, M, N, K, tile16, dlp.EPI_BIAS, oracle.OUT_BF16)
    assert plan.startswith("stream_") and ("_nt%d_" % tile16) in plan, plan


def test_packed_errors(ctx):
    W = dev_bf16(synth.integer_bf16((64, 256), -2, 2, 1))
    Wp = dlp.proj_pack_weights(ctx, W, 2)
    X = dev_bf16(synth.integer_bf16((600, 256), -2, 2, 2))
    with pytest.raises(dlp.ProjError) as e:         # above the streaming kernel's 512 rows
        dlp.proj_run_packed(ctx, X, Wp, 2, None, dlp.EPI_NONE, out_tensor(600, 64, oracle.OUT_F32), 64)
    assert e.value.status == dlp.PROJ_ERR_UNSUPPORTED
    with pytest.raises(dlp.ProjError):              # no tile of 48 rows
        dlp.proj_run_packed(ctx, X[:16], Wp, 3, None, dlp.EPI_NONE, out_tensor(16, 64, oracle.OUT_F32), 64)
    with pytest.raises(ValueError):                 # K not a multiple of 128
        dlp.proj_pack_weights(ctx, dev_bf16(synth.integer_bf16((8, 200), -2, 2, 3)), 1)


def test_packed_graph_replays(ctx):
    """The tuned packed plan captured in a torch CUDA graph over two buffer
    sets; every replay, with new X and eager work in between, matches the
    oracle."""
    M, N, K, tile16 = 16, 2048, 4096, 2
    Ws = [synth.normal_bf16((N, K), 1.0 / np.sqrt(K), 90 + p) for p in range(2)]
    bs = [synth.normal_bf16((N,), 0.14, 92 + p) for p in range(2)]
    Wps = [dlp.proj_pack_weights(ctx, dev_bf16(w), tile16) for w in Ws]
    bd = [dev_bf16(b) for b in bs]
    Xd = [dev_bf16(synth.normal_bf16((M, K), 1.0, 94 + p)) for p in range(2)]
    Ys = [out_tensor(M, N, oracle.OUT_BF16) for _ in range(2)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for p in range(2):
            dlp.proj_run_packed(ctx, Xd[p], Wps[p], tile16, bd[p], dlp.EPI_BIAS, Ys[p], N, stream=s)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for p in range(2):
                dlp.proj_run_packed(ctx, Xd[p], Wps[p], tile16, bd[p], dlp.EPI_BIAS, Ys[p], N, stream=s)
    for rep in range(3):
        Xs = [synth.normal_bf16((M, K), 1.0, 500 + 10 * rep + p) for p in range(2)]
        for p in range(2):
            Xd[p].copy_(dev_bf16(Xs[p]))
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        del junk
        for p in range(2):
            r, _ = oracle.reference(Xs[p], Ws[p], bs[p], oracle.EPI_BIAS, oracle.OUT_BF16)
            rep_ = compare.check(host_f64(Ys[p]), r)
            assert rep_["ok"], (rep, p, rep_)
