"""The optional plan file (PROJ_PLAN_FILE): a tuned plan is appended as one
line keyed by device and shape, and a context created later loads it, so
the shape runs its measured plan without tuning again; lines that do not
name a candidate of their key are skipped.  PROJ_LOG reports decisions."""
import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor, require_gpu

pytestmark = pytest.mark.gpu


def test_plan_file_round_trip(tmp_path, monkeypatch, capfd):
    require_gpu()
    path = tmp_path / "plans.txt"
    monkeypatch.setenv("PROJ_PLAN_FILE", str(path))
    monkeypatch.setenv("PROJ_LOG", "1")
    M, N, K = 16, 512, 2048
    X = synth.normal_bf16((M, K), 1.0, 7800)
    W = synth.normal_bf16((N, K), float(1 / np.sqrt(K)), 7801)
    r, _ = oracle.reference(X, W, None, oracle.EPI_NONE, oracle.OUT_BF16)
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    c1 = dlp.proj_create(0)
    try:
        Y = out_tensor(M, N, oracle.OUT_BF16)
        dlp.proj_run(c1, Xd, Wd, None, dlp.EPI_NONE, Y)
        plan = dlp.proj_get_plan(c1, M, N, K, dlp.EPI_NONE, dlp.OUT_BF16)
    finally:
        dlp.proj_destroy(c1)
    lines = path.read_text().splitlines()
    print(lines, flush=True)
    assert len(lines) == 1
    f = lines[0].split()
    assert f[:2] == ["proj-plan", "1"] and f[2].startswith("gfx950")
    assert [int(x) for x in f[3:10]] == [M, N, K, dlp.EPI_NONE, dlp.OUT_BF16, 1, 0]
    assert f[11] == plan.split(" ")[0]
    # a line for another device and a line naming no candidate are skipped
    with open(path, "a") as fh:
        fh.write("proj-plan 1 gfx000_cu1 %d %d %d 0 1 1 0 0 %s 1.0\n" % (M, N, K, f[11]))
        fh.write("proj-plan 1 %s 16 1024 2048 0 1 1 0 0 no_such_plan 1.0\n" % f[2])
    c2 = dlp.proj_create(0)
    try:
        loaded = dlp.proj_get_plan(c2, M, N, K, dlp.EPI_NONE, dlp.OUT_BF16)   # before any call
        assert loaded.split(" ")[0] == f[11] and "tuned" in loaded, loaded
        with pytest.raises(dlp.ProjError):
            dlp.proj_get_plan(c2, M, 1024, K, dlp.EPI_NONE, dlp.OUT_BF16)
        Y = out_tensor(M, N, oracle.OUT_BF16)
        dlp.proj_run(c2, Xd, Wd, None, dlp.EPI_NONE, Y)
        assert compare.check(host_f64(Y), r)["ok"]
        assert len(path.read_text().splitlines()) == 3   # nothing tuned again
    finally:
        dlp.proj_destroy(c2)
    err = capfd.readouterr().err
    assert "proj: " in err and "tuned" in err and "loaded" in err
