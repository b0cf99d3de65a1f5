"""Seeded synthetic inputs for the dense projection workloads.

This module only draws numbers: it holds none of the projection's arithmetic
(no products, sums, bias, GELU or output rounding), so both the oracle side
and the GPU side can take their inputs from it without sharing method code.

Recipe (the same for every workload):
  - X[M, K] ~ N(0, 1), W[N, K] ~ N(0, 1/K) (variance 1/K, so each output is
    of unit scale), bias[N] ~ N(0, 0.02) (variance 0.02, std ~0.141);
  - numbers come from numpy's PCG64 generator seeded per tensor, drawn as
    float32 normals, scaled, then rounded to the nearest bf16 with ties to
    even; the bf16 bit patterns (uint16) are what both sides receive;
  - seeds: X = 1000 + i, W = 2000 + i, bias = 3000 + i for workload i, plus
    an optional offset for rotated copies.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

EPI_NONE, EPI_BIAS, EPI_GELU, EPI_BIAS_GELU = 0, 1, 2, 3
OUT_F32, OUT_BF16 = 0, 1


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    M: int
    N: int
    K: int
    epi: int
    out_dtype: int

    @property
    def has_bias(self) -> bool:
        return self.epi in (EPI_BIAS, EPI_BIAS_GELU)

    def alg_bytes(self) -> int:
        """Bytes the projection must move at minimum: X, W, bias read once,
        Y written once."""
        out_b = 4 if self.out_dtype == OUT_F32 else 2
        return (2 * self.M * self.K + 2 * self.N * self.K
                + (2 * self.N if self.has_bias else 0) + out_b * self.M * self.N)

    def alg_flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The five workloads, sized as the hot-path targets state them.
WORKLOADS = [
    Workload(0, "proj_m16_k8192_n1024_f32", 16, 1024, 8192, EPI_NONE, OUT_F32),
    Workload(1, "decode_m16_k8192_n8192_bias_bf16", 16, 8192, 8192, EPI_BIAS, OUT_BF16),
    Workload(2, "ffn_up_m64_k8192_n28672_bf16", 64, 28672, 8192, EPI_NONE, OUT_BF16),
    Workload(3, "qkv_m8192_k1024_n3072_bias_bf16", 8192, 3072, 1024, EPI_BIAS, OUT_BF16),
    Workload(4, "prefill_ffn_m4096_k8192_n8192_bias_gelu_bf16", 4096, 8192, 8192,
             EPI_BIAS_GELU, OUT_BF16),
]


# The thirty-shape set of the worklog (section "The same calculation shows up
# in different sizes"): six loads -- decode with 1, 16 or 32 token rows,
# verification with 8, 128 or 256 -- times five projection families.  The
# projections have no bias (the worklog's plain Y = X W^T); bf16 weights give
# bf16 outputs.  The router's weights are fp32 and its output fp32.  The
# unpooler's smaller output slice (N = 1024) applies to the loads of 1 and 8
# token rows only; the other four loads use N = 8192 (the thirty-shape timing
# table under "What actually ran in the winning version?").
SWEEP_LOADS = (1, 16, 32, 8, 128, 256)


@dataclass(frozen=True)
class SweepShape:
    index: int
    family: str
    M: int
    N: int
    K: int
    fp32_weights: bool

    @property
    def name(self) -> str:
        return "%s_m%d_n%d_k%d" % (self.family, self.M, self.N, self.K)

    def alg_bytes(self) -> int:
        """X and W read once (W in its stored format), Y written once."""
        w_b = 4 if self.fp32_weights else 2
        y_b = 4 if self.fp32_weights else 2
        return 2 * self.M * self.K + w_b * self.N * self.K + y_b * self.M * self.N

    def alg_flops(self) -> int:
        return 2 * self.M * self.N * self.K


def sweep_shapes():
    out = []
    for M in SWEEP_LOADS:
        fams = [("qkv_gate", 2304, 8192, False), ("output", 8192, 1024, False), ("pooler", 4096, 8192, False),
                ("unpooler", 1024 if M in (1, 8) else 8192, 4096, False), ("router", 256, 8192, True)]
        for fam, N, K, f32w in fams:
            out.append(SweepShape(len(out), fam, M, N, K, f32w))
    return out


def sweep_inputs(s: SweepShape, offset: int = 0):
    """(X, W) for a sweep shape: X bf16 bits ~ N(0, 1); W ~ N(0, 1/K) as bf16
    bits, or as float32 values for fp32-weight shapes.  Seeds 5000 + index
    (X) and 6000 + index (W)."""
    X = normal_bf16((s.M, s.K), 1.0, 5000 + s.index + offset)
    if not s.fp32_weights:
        return X, normal_bf16((s.N, s.K), float(1.0 / np.sqrt(s.K)), 6000 + s.index + offset)
    rng = np.random.Generator(np.random.PCG64(6000 + s.index + offset))
    W = rng.standard_normal((s.N, s.K), dtype=np.float32)
    W *= np.float32(1.0 / np.sqrt(s.K))
    return X, W


def probe_rows(M: int):
    """Rows that carry a sparse probe: one row in eight (rows 7, 15, ...),
    so there is at least one from M = 8 up (worklog, section "The actual
    error rule, including what L2 means")."""
    return list(range(7, M, 8))


PROBE_NNZ = 8


def with_probe_rows(X: np.ndarray, seed: int) -> np.ndarray:
    """A copy of bf16 bits X whose probe rows are replaced by sparse rows:
    PROBE_NNZ distinct positions holding N(0, 1) values, zeros elsewhere."""
    X = np.array(X, dtype=np.uint16, copy=True)
    M, K = X.shape
    rng = np.random.Generator(np.random.PCG64(seed))
    for m in probe_rows(M):
        X[m, :] = 0
        nnz = min(PROBE_NNZ, K)
        cols = rng.choice(K, size=nnz, replace=False)
        X[m, cols] = f32_to_bf16_bits(rng.standard_normal(nnz, dtype=np.float32))
    return X


def f32_to_bf16_bits(a: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Round float32 samples to bf16 bit patterns (nearest, ties to even).
    Only used to produce inputs; the samples must be finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.isfinite(a).all():
        raise ValueError("input samples must be finite")
    u = a.view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF            # finite values never carry past bit 31 here
    r += u
    r >>= 16
    if out is None:
        return r.astype(np.uint16)
    out[...] = r
    return out


_CHUNK = 1 << 20


def normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    """bf16 bits of N(0, std^2) samples, drawn in row-major order.  Drawn in
    fixed-size pieces to bound temporary memory; the stream is the same as
    one single draw of the whole array."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    buf = np.empty(min(_CHUNK, max(flat.size, 1)), dtype=np.float32)
    for at in range(0, flat.size, _CHUNK):
        n = min(_CHUNK, flat.size - at)
        b = buf[:n]
        rng.standard_normal(out=b, dtype=np.float32)
        if std != 1.0:
            b *= np.float32(std)
        f32_to_bf16_bits(b, flat[at:at + n])
    return out


def make_inputs(M: int, N: int, K: int, has_bias: bool, index: int, offset: int = 0):
    """(X, W, bias) as uint16 bf16 bit arrays; bias is None without a bias."""
    X = normal_bf16((M, K), 1.0, 1000 + index + offset)
    W = normal_bf16((N, K), float(1.0 / np.sqrt(K)) if K > 0 else 1.0, 2000 + index + offset)
    b = normal_bf16((N,), float(np.sqrt(0.02)), 3000 + index + offset) if has_bias else None
    return X, W, b


def workload_inputs(w: Workload, offset: int = 0):
    return make_inputs(w.M, w.N, w.K, w.has_bias, w.index, offset)


def integer_bf16(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """Small integers in [lo, hi] as bf16 bits (exact in bf16 for |v| <= 256)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(v)


def values_to_bf16(values) -> np.ndarray:
    """bf16 bits of given float values (used for hand-written fixtures)."""
    return f32_to_bf16_bits(np.asarray(values, dtype=np.float32))
