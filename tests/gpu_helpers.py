"""Shared helpers for the GPU tests: device transfer of bf16 bit arrays,
read-back, and a per-session library context."""
import numpy as np
import pytest

try:
    import torch
except Exception:  # pragma: no cover
    torch = None

import oracle


def gpu_available() -> bool:
    return torch is not None and torch.cuda.is_available()


def require_gpu():
    if not gpu_available():
        pytest.skip("needs a GPU")


def dev_bf16(bits: np.ndarray, offset_elems: int = 0):
    """uint16 bf16 bits -> contiguous bf16 device tensor.  With offset_elems
    > 0 the tensor is a view starting that many elements into a larger
    allocation (to test unaligned pointers)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    flat = torch.from_numpy(bits.reshape(-1).view(np.int16).copy())
    if offset_elems:
        pad = torch.zeros(flat.numel() + offset_elems, dtype=torch.int16)
        pad[offset_elems:] = flat
        t = pad.cuda()[offset_elems:]
    else:
        t = flat.cuda()
    return t.view(torch.bfloat16).reshape(bits.shape)


def host_f64(Y) -> np.ndarray:
    """Device output (fp32 or bf16) -> float64 numpy, exactly."""
    torch.cuda.synchronize()
    if Y.dtype == torch.bfloat16:
        bits = Y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return oracle.bf16_to_f64(bits)
    return Y.float().cpu().numpy().astype(np.float64)


def out_tensor(M, N, out_dtype, fill=float("nan")):
    dt = torch.float32 if out_dtype == oracle.OUT_F32 else torch.bfloat16
    return torch.full((M, N), fill, dtype=dt, device="cuda")


def rounded_reference(X, W, bias, epi, out_dtype):
    r, s = oracle.reference(X, W, bias, epi, out_dtype)
    return r, s
