"""The host side of the C ABI under AddressSanitizer (CPU only, no GPU).

csrc/proj.cpp -- argument checks, candidate enumeration, plan-file parsing,
status strings -- is rebuilt with AddressSanitizer on its host half only
(the device half of a HIP build is never sanitized here), linked with the
library's other objects into a separate libproj_asan.so, and a C program
built with the sanitizer drives the host paths: candidate lists and names
over many shapes and every epilogue / output / alignment combination, packed
sizes, every NULL / destroyed / invalid-argument path, and proj_create
without a GPU (which must fail with a status, also with a plan file set).
Any heap or stack error aborts the program with a report.
"""
import os
import subprocess

import pytest

import dense_linear_projection_amd as dlp
from dense_linear_projection_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "proj.h"

static const long long shapes[][3] = {
    {1, 1, 1}, {1, 256, 8192}, {5, 77, 96}, {16, 1024, 8192}, {16, 8192, 8192}, {64, 28672, 8192},
    {8192, 3072, 1024}, {4096, 8192, 8192}, {300, 520, 512}, {513, 100, 200}, {7, 50, 100},
    {1, 1024, 1 << 26}, {64, 131072, 8192}, {0, 10, 10}, {10, 0, 10}, {10, 10, 0}};

int main(void) {
    char name[256];
    long long total = 0;
    for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int epi = 0; epi < 4; ++epi)
            for (int out = 0; out < 2; ++out)
                for (int al = 0; al < 2; ++al) {
                    const long long M = shapes[s][0], N = shapes[s][1], K = shapes[s][2];
                    int n = proj_num_candidates(M, N, K, epi, out, al);
                    for (int i = 0; i < n; ++i) {
                        if (proj_candidate_name(M, N, K, epi, out, al, i, name, sizeof name) != PROJ_OK) return 10;
                        if (strlen(name) == 0) return 11;
                    }
                    if (n > 0 && proj_candidate_name(M, N, K, epi, out, al, n, name, sizeof name) == PROJ_OK)
                        return 12;
                    if (n > 0 && proj_candidate_name(M, N, K, epi, out, al, 0, name, 4) == PROJ_OK) return 13;
                    total += n;
                    int nh = proj_num_candidates_hilo(M, N, K, epi, out, al);
                    for (int i = 0; i < nh; ++i)
                        if (proj_candidate_name_hilo(M, N, K, epi, out, al, i, name, sizeof name) != PROJ_OK)
                            return 14;
                    for (int t = 0; t < 9; ++t) {
                        int np = proj_num_candidates_packed(M, N, K, t, epi, out, al);
                        for (int i = 0; i < np; ++i)
                            if (proj_candidate_name_packed(M, N, K, t, epi, out, al, i, name, sizeof name) !=
                                PROJ_OK)
                                return 15;
                        (void)proj_packed_bytes(N, K, t);
                    }
                }
    if (proj_run(NULL, NULL, NULL, NULL, 0, 1, 1, 1, NULL, 0, NULL) != PROJ_ERR_INVALID_ARG) return 20;
    if (proj_run_noalloc(NULL, NULL, NULL, NULL, 0, 1, 1, 1, NULL, 0, NULL) != PROJ_ERR_INVALID_ARG) return 21;
    if (proj_destroy(NULL) != PROJ_ERR_INVALID_ARG) return 22;
    if (proj_graph_launch(NULL, NULL) != PROJ_ERR_INVALID_ARG) return 23;
    if (proj_get_plan(NULL, 1, 1, 1, 0, 0, 1, name, sizeof name) != PROJ_ERR_INVALID_ARG) return 24;
    if (proj_read_probe(NULL, NULL, 16, NULL) != PROJ_ERR_INVALID_ARG) return 25;
    for (int st = -1; st < 9; ++st)
        if (!proj_status_string(st)) return 26;
    if (strcmp(proj_last_error(NULL), "") != 0) return 27;
    proj_ctx *ctx = NULL;
    proj_status s = proj_create(&ctx, 0, (size_t)64 << 20);
    if (s == PROJ_OK) proj_destroy(ctx);   /* a GPU host: the host paths above still ran */
    printf("%lld|%s\n", total, proj_status_string(s));
    return 0;
}
"""


def test_host_paths_under_address_sanitizer(tmp_path):
    if not os.path.exists(dlp.LIB_PATH):
        pytest.skip("libproj.so is not built")
    objs = [os.path.join(_build.BUILD, os.path.splitext(x)[0] + ".o") for x in _build.SOURCES if x != "proj.cpp"]
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    if not all(os.path.exists(o) for o in objs) or not os.path.exists(clang):
        pytest.skip("library objects or ROCm's clang missing")
    hipcc = _build.hipcc()
    flags = [f for f in _build.FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    proj_o = str(tmp_path / "proj_asan.o")
    # the sanitizer applies to the host half of the translation unit only
    subprocess.run([hipcc] + flags + ["-Xarch_host", "-fsanitize=address", "-x", "hip", "-c",
                                      os.path.join(_build.CSRC, "proj.cpp"), "-o", proj_o],
                   check=True, capture_output=True)
    lib = str(tmp_path / "libproj_asan.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-o", lib, proj_o] + objs, check=True, capture_output=True)
    src = tmp_path / "drive.c"
    src.write_text(C_SRC)
    exe = str(tmp_path / "drive")
    # the driver is built by the same compiler family, so one sanitizer
    # runtime serves both
    subprocess.run([clang, "-std=c99", "-g", "-fsanitize=address", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", exe, lib, "-Wl,-rpath," + str(tmp_path)], check=True, capture_output=True)
    env = dict(os.environ)
    # the HIP runtime's own start-up allocations are not ours to report
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["PROJ_PLAN_FILE"] = str(tmp_path / "plans.txt")
    (tmp_path / "plans.txt").write_text("proj-plan 1 gfx950_cu256 16 1024 8192 0 0 1 0 0 x 1.0\nnot a plan\n")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    total, status = r.stdout.strip().splitlines()[-1].split("|")
    assert int(total) > 1000
    assert "AddressSanitizer" not in r.stderr
