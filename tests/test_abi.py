"""The C ABI library loads, exports every symbol include/proj.h declares, and
its host-side logic (argument checks, status strings, candidate lists) works
without a GPU.  No compute calls here."""
import ctypes
import os
import re

import pytest

import dense_linear_projection_amd as dlp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "proj.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(proj_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("proj_create", "proj_run", "proj_destroy"):
        assert required in names
    assert sorted(dlp.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    L = dlp.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings():
    assert dlp.proj_status_string(0) == "ok"
    for s in range(1, 7):
        assert dlp.proj_status_string(s) not in ("ok", "unknown status")
    assert dlp.proj_status_string(99) == "unknown status"


def test_null_handles_rejected_before_any_hip_call():
    L = dlp.lib()
    assert L.proj_run(None, None, None, None, 0, 1, 1, 1, None, 0, None) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_tune(None, None, None, None, 0, 1, 1, 1, None, 0, None) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_destroy(None) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_create(None, 0, 0) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_graph_launch(None, None) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_graph_destroy(None) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_read_probe(None, None, 64, None) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_prepare_hilo(None, None, 1, 1, None, None) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_pack_weights(None, None, 16, 128, 2, None, None) == dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_graph_capture(None, 1, None, None, None, None, 0, 1, 1, 1, 0, None, None) == \
        dlp.PROJ_ERR_INVALID_ARG
    assert L.proj_last_error(None) == b""


def test_candidate_lists_are_host_logic():
    # small M: weight-streaming variants with several split counts + GEMMs
    n = dlp.proj_num_candidates(16, 8192, 8192, dlp.EPI_BIAS, dlp.OUT_BF16)
    names = [dlp.proj_candidate_name(16, 8192, 8192, dlp.EPI_BIAS, dlp.OUT_BF16, i) for i in range(n)]
    assert any(x.startswith("stream_mt1") for x in names)
    assert any(x.endswith("_s1") for x in names) and any(x.endswith("_s4") for x in names)
    assert any(x.startswith("gemm_") for x in names)
    assert len(set(names)) == len(names)          # every candidate is a distinct variant
    # large M: only the tiled GEMMs
    big = [dlp.proj_candidate_name(4096, 8192, 8192, 3, 1, i)
           for i in range(dlp.proj_num_candidates(4096, 8192, 8192, 3, 1))]
    assert big and all(x.startswith("gemm") for x in big)
    # misaligned operands or K % 8 != 0: the generic kernel only
    assert dlp.proj_num_candidates(16, 64, 100, 0, 0) >= 1
    assert dlp.proj_candidate_name(16, 64, 64, 0, 0, 0, aligned16=False) == "generic"
    assert dlp.proj_num_candidates(0, 64, 64, 0, 0) == 0
    with pytest.raises(dlp.ProjError):
        dlp.proj_candidate_name(16, 64, 64, 0, 0, 10 ** 6)


def test_create_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(dlp.ProjError) as e:
        dlp.proj_create(0)
    assert e.value.status in (dlp.PROJ_ERR_HIP, dlp.PROJ_ERR_INVALID_ARG)


def test_packed_layout_host_rules():
    """Packed-weight sizes and candidate lists are host logic: tiles of
    16 * tile16 rows padded with zero rows, K a multiple of 128, only the
    streaming kernel's tile heights, and no plan above 512 token rows."""
    assert dlp.proj_packed_bytes(100, 256, 1) == 7 * 16 * 256 * 2
    assert dlp.proj_packed_bytes(100, 256, 7) == 1 * 112 * 256 * 2
    assert dlp.proj_packed_bytes(8192, 8192, 2) == 8192 * 8192 * 2
    assert dlp.proj_packed_bytes(0, 256, 2) == 0
    assert dlp.proj_packed_bytes(100, 200, 2) == -1      # K not a multiple of 128
    assert dlp.proj_packed_bytes(100, 256, 3) == -1      # no streaming tile of 48 rows
    assert dlp.proj_packed_bytes(-1, 256, 2) == -1
    n = dlp.proj_num_candidates_packed(16, 8192, 8192, 2, dlp.EPI_BIAS, dlp.OUT_BF16)
    names = [dlp.proj_candidate_name_packed(16, 8192, 8192, 2, dlp.EPI_BIAS, dlp.OUT_BF16, i) for i in range(n)]
    assert n > 0 and all(x.startswith("stream_mt1_nt2_") for x in names)
    assert dlp.proj_num_candidates_packed(513, 8192, 8192, 2, 0, 0) == 0
    assert dlp.proj_num_candidates_packed(16, 8192, 8192, 3, 0, 0) == 0
    assert dlp.proj_num_candidates_packed(16, 8192, 8200, 2, 0, 0) == 0
    assert dlp.proj_num_candidates_packed(16, 8192, 8192, 2, 0, 0, aligned16=False) == 0
    # 384 = 3 x 128: the 256-column stage variants are not offered
    names = [dlp.proj_candidate_name_packed(200, 300, 384, 4, 0, 0, i)
             for i in range(dlp.proj_num_candidates_packed(200, 300, 384, 4, 0, 0))]
    assert names and not any("_k256_" in x for x in names)
    assert all(re.match(r"stream_mt(4|8)_nt4_", x) for x in names)


def test_offset_limits_in_candidate_lists():
    """Variants whose buffer-resource offsets would pass 32 (GEMV: 31) bits
    are not offered: at K = 2^26 a packed 32-row tile spans 2^32 bytes and a
    16-row GEMV workgroup 2^31 bytes."""
    K = 1 << 26
    assert dlp.proj_num_candidates_packed(16, 1024, K, 2, 0, 0) == 0
    assert dlp.proj_num_candidates_packed(16, 1024, K, 1, 0, 0) > 0
    n = dlp.proj_num_candidates(1, 1024, K, 0, 0)
    gemv = [x for x in (dlp.proj_candidate_name(1, 1024, K, 0, 0, i) for i in range(n)) if x.startswith("gemv")]
    assert gemv and not any("_r16_" in x for x in gemv)
    n = dlp.proj_num_candidates(1, 1024, 1 << 20, 0, 0)
    assert any("_r16_" in dlp.proj_candidate_name(1, 1024, 1 << 20, 0, 0, i) for i in range(n))


def test_candidate_lists_hold_validity_rules_only():
    """The candidate list carries no device or workspace threshold: every K
    split that leaves each split at least two 64-wide k-ranges is listed for
    the persistent GEMM, however many tiles the shape has, and streaming
    splits are listed even where their fp32 partials exceed any default
    workspace (a context keeps only those that fit its own bound)."""
    def names(M, N, K, epi=0, out=1):
        return [dlp.proj_candidate_name(M, N, K, epi, out, i)
                for i in range(dlp.proj_num_candidates(M, N, K, epi, out))]
    qkv = names(8192, 3072, 1024, 1, 1)                  # 512 tiles of 256 x 192, K / 64 = 16
    for S in (2, 4, 8):
        assert "gemmpp64p_256x192x64_w4x2_g4_s%d" % S in qkv
    assert "gemmpp64p_256x192x64_w4x2_g4_s16" not in qkv    # a split would hold one k-range
    ffn = names(4096, 8192, 8192, 3, 1)                  # 512 tiles of 256 x 256, K / 64 = 128
    assert "gemmpp64p_256x256x64_w4x2_g4_s16" in ffn
    wide = names(64, 131072, 8192)                       # S = 16 partials: 512 MiB
    assert any(x.startswith("stream_mt4_") and x.endswith("_s16") for x in wide)
