"""The worklog's thirty-shape set (bf16-weight shapes) through proj_run with
the measured plan, against the oracle on every element.  Token counts 1, 8,
16, 32 go to the weight-streaming kernel (M = 1 and 8 below its 16-row
tile), 128 and 256 to the tiled GEMMs."""
import numpy as np
import pytest

import dense_linear_projection_amd as dlp
import oracle
import synth
from oracle import compare
from tests.gpu_helpers import dev_bf16, host_f64, out_tensor

pytestmark = pytest.mark.gpu

SHAPES = [s for s in synth.sweep_shapes() if not s.fp32_weights]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_sweep_shape_every_element(ctx, shape):
    print("sweep shape", shape.name, flush=True)
    X, W = synth.sweep_inputs(shape)
    Y = out_tensor(shape.M, shape.N, oracle.OUT_BF16)
    dlp.proj_run(ctx, dev_bf16(X), dev_bf16(W), None, dlp.EPI_NONE, Y)
    u = host_f64(Y)
    r, _ = oracle.reference(X, W, None, oracle.EPI_NONE, oracle.OUT_BF16)
    rep = compare.check(u, r)
    print(shape.name, dlp.proj_get_plan(ctx, shape.M, shape.N, shape.K, dlp.EPI_NONE, oracle.OUT_BF16), rep,
          flush=True)
    assert rep["ok"], rep
