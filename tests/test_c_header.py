"""The boundary is usable from C: include/proj.h compiles as C99 with all
warnings as errors, and a C program links against libproj.so and calls its
host-side functions (status strings, candidate lists, packed sizes, argument
checks).  No GPU is needed: proj_create reports its absence with a status."""
import os
import subprocess

import pytest

import dense_linear_projection_amd as dlp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "proj.h"

int main(void) {
    if (strcmp(proj_status_string(PROJ_OK), "ok") != 0) return 1;
    if (proj_num_candidates(16, 8192, 8192, PROJ_EPI_BIAS, PROJ_OUT_BF16, 1) <= 0) return 2;
    char name[128];
    if (proj_candidate_name(16, 8192, 8192, PROJ_EPI_BIAS, PROJ_OUT_BF16, 1, 0, name, sizeof name) != PROJ_OK)
        return 3;
    if (proj_packed_bytes(100, 256, 1) != 7 * 16 * 256 * 2) return 4;
    if (proj_packed_bytes(100, 200, 1) != -1) return 5;
    if (proj_run(NULL, NULL, NULL, NULL, 0, 1, 1, 1, NULL, 0, NULL) != PROJ_ERR_INVALID_ARG) return 6;
    proj_ctx *ctx = NULL;
    proj_status s = proj_create(&ctx, 0, (size_t)64 << 20);
    if (s == PROJ_OK) proj_destroy(ctx);
    printf("%s|%s\n", name, proj_status_string(s));
    return 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path):
    lib = dlp.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("libproj.so is not built")
    src = tmp_path / "use_proj.c"
    src.write_text(C_SRC)
    exe = tmp_path / "use_proj"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), lib, "-Wl,-rpath," + os.path.dirname(lib)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, (out.returncode, out.stdout, out.stderr)
    name, status = out.stdout.strip().split("|")
    assert name.startswith(("stream_", "gemv_", "gemm")), name
    assert status   # "ok" on a GPU host, a failure status without one
