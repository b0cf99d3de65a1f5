"""MI355X-native dense projection Y = X . W^T (+ bias) (-> GELU tanh).

A thin ctypes binding over ``libproj.so`` (C ABI declared in
``include/proj.h``).  Every step of the projection runs in the library's HIP
kernels; this module only turns torch tensors and streams into pointers and
sizes, and status codes into exceptions.  PyTorch provides device memory and
streams.  There is no fallback: if the library is not built, importing the
binding's entry points raises.

Names mirror the C ABI: ``proj_create``, ``proj_run``, ``proj_destroy``,
``proj_tune``, ``proj_get_plan``, ``proj_num_candidates``,
``proj_candidate_name``, ``proj_run_candidate``, ``proj_graph_capture``,
``proj_graph_launch``, ``proj_graph_destroy``, ``proj_status_string``, and
for fp32 weights held as a bf16 high/low pair ``proj_prepare_hilo``,
``proj_run_hilo``, ``proj_get_plan_hilo``, ``proj_num_candidates_hilo``,
``proj_candidate_name_hilo``, ``proj_run_candidate_hilo``, and for bf16
weights registered in the packed tile layout ``proj_packed_bytes``,
``proj_pack_weights``, ``proj_run_packed``, ``proj_get_plan_packed``,
``proj_num_candidates_packed``, ``proj_candidate_name_packed``,
``proj_run_candidate_packed``, the measured read floor
``proj_read_probe``, and ``proj_run_noalloc`` (proj_run with no device
allocation).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libproj.so")

PROJ_OK = 0
PROJ_ERR_INVALID_ARG = 1
PROJ_ERR_UNSUPPORTED = 2
PROJ_ERR_HIP = 3
PROJ_ERR_NO_MEMORY = 4
PROJ_ERR_NOT_TUNED = 5
PROJ_ERR_DESTROYED = 6

EPI_NONE, EPI_BIAS, EPI_GELU_TANH, EPI_BIAS_GELU_TANH = 0, 1, 2, 3
OUT_F32, OUT_BF16 = 0, 1

EXPORTS = ["proj_create", "proj_run", "proj_tune", "proj_destroy", "proj_status_string",
           "proj_last_error", "proj_get_plan", "proj_num_candidates", "proj_candidate_name",
           "proj_run_candidate", "proj_graph_capture", "proj_graph_launch", "proj_graph_destroy",
           "proj_prepare_hilo", "proj_run_hilo", "proj_get_plan_hilo", "proj_num_candidates_hilo",
           "proj_candidate_name_hilo", "proj_run_candidate_hilo", "proj_packed_bytes", "proj_pack_weights",
           "proj_run_packed", "proj_get_plan_packed", "proj_num_candidates_packed", "proj_candidate_name_packed",
           "proj_run_candidate_packed", "proj_read_probe", "proj_run_noalloc"]


class ProjError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d)%s" % (_status_text(status), status,
                                               ": " + message if message else ""))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libproj.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libproj.so is not built: run `python -m dense_linear_projection_amd._build` "
                           "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, ci, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int
    run_args = [vp, vp, vp, vp, ci, i64, i64, i64, vp, ci, vp]
    sig = {
        "proj_create": ([ctypes.POINTER(vp), ci, ctypes.c_size_t], st),
        "proj_run": (run_args, st),
        "proj_tune": (run_args, st),
        "proj_destroy": ([vp], st),
        "proj_status_string": ([ci], ctypes.c_char_p),
        "proj_last_error": ([vp], ctypes.c_char_p),
        "proj_get_plan": ([vp, i64, i64, i64, ci, ci, ci, ctypes.c_char_p, ctypes.c_size_t], st),
        "proj_num_candidates": ([i64, i64, i64, ci, ci, ci], ci),
        "proj_candidate_name": ([i64, i64, i64, ci, ci, ci, ci, ctypes.c_char_p, ctypes.c_size_t], st),
        "proj_run_candidate": ([vp, ci, vp, vp, vp, ci, i64, i64, i64, vp, ci, vp], st),
        "proj_graph_capture": ([vp, ci, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                ctypes.POINTER(vp), ci, i64, i64, i64, ci, vp, ctypes.POINTER(vp)], st),
        "proj_graph_launch": ([vp, vp], st),
        "proj_graph_destroy": ([vp], st),
        "proj_prepare_hilo": ([vp, vp, i64, i64, vp, vp], st),
        "proj_run_hilo": (run_args, st),
        "proj_get_plan_hilo": ([vp, i64, i64, i64, ci, ci, ci, ctypes.c_char_p, ctypes.c_size_t], st),
        "proj_num_candidates_hilo": ([i64, i64, i64, ci, ci, ci], ci),
        "proj_candidate_name_hilo": ([i64, i64, i64, ci, ci, ci, ci, ctypes.c_char_p, ctypes.c_size_t], st),
        "proj_run_candidate_hilo": ([vp, ci, vp, vp, vp, ci, i64, i64, i64, vp, ci, vp], st),
        "proj_packed_bytes": ([i64, i64, ci], i64),
        "proj_pack_weights": ([vp, vp, i64, i64, ci, vp, vp], st),
        "proj_run_packed": ([vp, vp, vp, ci, vp, ci, i64, i64, i64, vp, ci, vp], st),
        "proj_get_plan_packed": ([vp, i64, i64, i64, ci, ci, ci, ci, ctypes.c_char_p, ctypes.c_size_t], st),
        "proj_num_candidates_packed": ([i64, i64, i64, ci, ci, ci, ci], ci),
        "proj_candidate_name_packed": ([i64, i64, i64, ci, ci, ci, ci, ci, ctypes.c_char_p, ctypes.c_size_t], st),
        "proj_run_candidate_packed": ([vp, ci, vp, vp, ci, vp, ci, i64, i64, i64, vp, ci, vp], st),
        "proj_read_probe": ([vp, vp, ctypes.c_size_t, vp], st),
        "proj_run_noalloc": (run_args, st),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes, f.restype = args, res
    _lib = L
    return L


def _status_text(s: int) -> str:
    try:
        return lib().proj_status_string(int(s)).decode()
    except Exception:  # library not loadable: still describe the code
        return "status"


def _check(status: int, ctx=None) -> None:
    if status != PROJ_OK:
        msg = ""
        if ctx is not None:
            try:
                msg = lib().proj_last_error(ctx).decode()
            except Exception:
                msg = ""
        raise ProjError(status, msg)


# ------------------------------------------------------------- marshalling

def _ptr(t):
    """Device pointer of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must be on a GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous (row-major)")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _out_dtype(Y, out_dtype):
    if out_dtype is not None:
        return int(out_dtype)
    import torch
    if Y.dtype == torch.float32:
        return OUT_F32
    if Y.dtype == torch.bfloat16:
        return OUT_BF16
    raise ValueError("Y must be float32 or bfloat16")


def _check_operands(X, W, bias, Y):
    import torch
    for name, t in (("X", X), ("W", W), ("bias", bias)):
        if t is not None and not isinstance(t, int) and t.dtype != torch.bfloat16:
            raise ValueError("%s must be bfloat16" % name)
    if Y is not None and not isinstance(Y, int) and Y.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("Y must be float32 or bfloat16")


# ------------------------------------------------------------------ the ABI

DEFAULT_WORKSPACE_BYTES = 64 << 20


def proj_create(device: int = 0, max_workspace_bytes: int = DEFAULT_WORKSPACE_BYTES) -> int:
    """Create a context on `device` whose split-K workspace is
    max_workspace_bytes (plans whose fp32 partials need more are not used)."""
    h = ctypes.c_void_p()
    _check(lib().proj_create(ctypes.byref(h), int(device), int(max_workspace_bytes)))
    return h.value


def proj_destroy(ctx: int) -> None:
    _check(lib().proj_destroy(ctx))


def proj_status_string(status: int) -> str:
    return lib().proj_status_string(int(status)).decode()


def _shape(X, W, M, N, K):
    if M is None:
        M = X.shape[0]
    if N is None:
        N = W.shape[0]
    if K is None:
        K = X.shape[1] if X.dim() == 2 else 0
    return int(M), int(N), int(K)


def proj_run(ctx, X, W, bias, epilogue, Y, M=None, N=None, K=None, out_dtype=None, stream=None) -> None:
    """Enqueue Y = epilogue(X . W^T [+ bias]) on `stream` (default: torch's
    current stream).  X bf16 [M, K], W bf16 [N, K], bias bf16 [N] or None,
    Y float32 / bfloat16 [M, N]; all contiguous device tensors."""
    _check_operands(X, W, bias, Y)
    M, N, K = _shape(X, W, M, N, K)
    _check(lib().proj_run(ctx, _ptr(X), _ptr(W), _ptr(bias), int(epilogue), M, N, K, _ptr(Y),
                          _out_dtype(Y, out_dtype), _stream(stream)), ctx)


def proj_run_noalloc(ctx, X, W, bias, epilogue, Y, M=None, N=None, K=None, out_dtype=None, stream=None) -> None:
    """proj_run without any device allocation: split-K partials go to the
    library's static per-GPU scratch (2 MiB)."""
    _check_operands(X, W, bias, Y)
    M, N, K = _shape(X, W, M, N, K)
    _check(lib().proj_run_noalloc(ctx, _ptr(X), _ptr(W), _ptr(bias), int(epilogue), M, N, K, _ptr(Y),
                                  _out_dtype(Y, out_dtype), _stream(stream)), ctx)


def proj_tune(ctx, X, W, bias, epilogue, Y, M=None, N=None, K=None, out_dtype=None, stream=None) -> None:
    _check_operands(X, W, bias, Y)
    M, N, K = _shape(X, W, M, N, K)
    _check(lib().proj_tune(ctx, _ptr(X), _ptr(W), _ptr(bias), int(epilogue), M, N, K, _ptr(Y),
                           _out_dtype(Y, out_dtype), _stream(stream)), ctx)


def proj_get_plan(ctx, M, N, K, epilogue, out_dtype, aligned16=True) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().proj_get_plan(ctx, int(M), int(N), int(K), int(epilogue), int(out_dtype),
                               1 if aligned16 else 0, buf, 256), ctx)
    return buf.value.decode()


def proj_num_candidates(M, N, K, epilogue, out_dtype, aligned16=True) -> int:
    return int(lib().proj_num_candidates(int(M), int(N), int(K), int(epilogue), int(out_dtype),
                                         1 if aligned16 else 0))


def proj_candidate_name(M, N, K, epilogue, out_dtype, index, aligned16=True) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().proj_candidate_name(int(M), int(N), int(K), int(epilogue), int(out_dtype),
                                     1 if aligned16 else 0, int(index), buf, 256))
    return buf.value.decode()


def proj_run_candidate(ctx, index, X, W, bias, epilogue, Y, M=None, N=None, K=None, out_dtype=None,
                       stream=None) -> None:
    _check_operands(X, W, bias, Y)
    M, N, K = _shape(X, W, M, N, K)
    _check(lib().proj_run_candidate(ctx, int(index), _ptr(X), _ptr(W), _ptr(bias), int(epilogue), M, N, K,
                                    _ptr(Y), _out_dtype(Y, out_dtype), _stream(stream)), ctx)


# ---------------------------------------------- fp32 weights, high/low pair

def proj_prepare_hilo(ctx, W, Whl=None, stream=None):
    """Register fp32 weights W [N, K] (device float32 tensor) as the bf16
    pair Whl [N, 2K] = [H | L] (allocated here if not given); returns Whl."""
    import torch
    if W.dtype != torch.float32 or W.dim() != 2:
        raise ValueError("W must be a float32 [N, K] tensor")
    N, K = W.shape
    if Whl is None:
        Whl = torch.empty((N, 2 * K), dtype=torch.bfloat16, device=W.device)
    elif Whl.dtype != torch.bfloat16 or tuple(Whl.shape) != (N, 2 * K):
        raise ValueError("Whl must be bfloat16 [N, 2K]")
    _check(lib().proj_prepare_hilo(ctx, _ptr(W), int(N), int(K), _ptr(Whl), _stream(stream)), ctx)
    return Whl


def _shape_hilo(X, Whl, M, N, K):
    if M is None:
        M = X.shape[0]
    if N is None:
        N = Whl.shape[0]
    if K is None:
        K = X.shape[1]
    return int(M), int(N), int(K)


def proj_run_hilo(ctx, X, Whl, bias, epilogue, Y, M=None, N=None, K=None, out_dtype=None, stream=None) -> None:
    """Enqueue Y = epilogue(X . H^T + X . L^T [+ bias]) for X bf16 [M, K] and
    a registered pair Whl bf16 [N, 2K]."""
    _check_operands(X, Whl, bias, Y)
    M, N, K = _shape_hilo(X, Whl, M, N, K)
    _check(lib().proj_run_hilo(ctx, _ptr(X), _ptr(Whl), _ptr(bias), int(epilogue), M, N, K, _ptr(Y),
                               _out_dtype(Y, out_dtype), _stream(stream)), ctx)


def proj_get_plan_hilo(ctx, M, N, K, epilogue, out_dtype, aligned16=True) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().proj_get_plan_hilo(ctx, int(M), int(N), int(K), int(epilogue), int(out_dtype),
                                    1 if aligned16 else 0, buf, 256), ctx)
    return buf.value.decode()


def proj_num_candidates_hilo(M, N, K, epilogue, out_dtype, aligned16=True) -> int:
    return int(lib().proj_num_candidates_hilo(int(M), int(N), int(K), int(epilogue), int(out_dtype),
                                              1 if aligned16 else 0))


def proj_candidate_name_hilo(M, N, K, epilogue, out_dtype, index, aligned16=True) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().proj_candidate_name_hilo(int(M), int(N), int(K), int(epilogue), int(out_dtype),
                                          1 if aligned16 else 0, int(index), buf, 256))
    return buf.value.decode()


def proj_run_candidate_hilo(ctx, index, X, Whl, bias, epilogue, Y, M=None, N=None, K=None, out_dtype=None,
                            stream=None) -> None:
    _check_operands(X, Whl, bias, Y)
    M, N, K = _shape_hilo(X, Whl, M, N, K)
    _check(lib().proj_run_candidate_hilo(ctx, int(index), _ptr(X), _ptr(Whl), _ptr(bias), int(epilogue), M, N, K,
                                         _ptr(Y), _out_dtype(Y, out_dtype), _stream(stream)), ctx)


def proj_packed_bytes(N, K, tile16) -> int:
    """Bytes of the packed array for W [N, K] in tiles of 16 * tile16 rows
    (-1 if that packing is not offered)."""
    return int(lib().proj_packed_bytes(int(N), int(K), int(tile16)))


def proj_pack_weights(ctx, W, tile16, Wp=None, stream=None):
    """Pack bf16 W [N, K] into the tile layout (Wp allocated here if not
    given: a flat bf16 tensor of proj_packed_bytes / 2 elements); returns Wp."""
    import torch
    if W.dtype != torch.bfloat16 or W.dim() != 2:
        raise ValueError("W must be a bfloat16 [N, K] tensor")
    N, K = W.shape
    nbytes = proj_packed_bytes(N, K, tile16)
    if nbytes < 0:
        raise ValueError("no packing for N=%d K=%d tile16=%d" % (N, K, tile16))
    if Wp is None:
        Wp = torch.empty((nbytes // 2,), dtype=torch.bfloat16, device=W.device)
    elif Wp.dtype != torch.bfloat16 or Wp.numel() * 2 < nbytes:
        raise ValueError("Wp must be bfloat16 with at least %d bytes" % nbytes)
    _check(lib().proj_pack_weights(ctx, _ptr(W), int(N), int(K), int(tile16), _ptr(Wp), _stream(stream)), ctx)
    return Wp


def proj_run_packed(ctx, X, Wp, tile16, bias, epilogue, Y, N, M=None, K=None, out_dtype=None, stream=None) -> None:
    """Enqueue Y = epilogue(X . W^T [+ bias]) with W given packed (Wp from
    proj_pack_weights with the same tile16); N is W's row count."""
    _check_operands(X, Wp, bias, Y)
    M = int(X.shape[0] if M is None else M)
    K = int(X.shape[1] if K is None else K)
    _check(lib().proj_run_packed(ctx, _ptr(X), _ptr(Wp), int(tile16), _ptr(bias), int(epilogue), M, int(N), K,
                                 _ptr(Y), _out_dtype(Y, out_dtype), _stream(stream)), ctx)


def proj_get_plan_packed(ctx, M, N, K, tile16, epilogue, out_dtype, aligned16=True) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().proj_get_plan_packed(ctx, int(M), int(N), int(K), int(tile16), int(epilogue), int(out_dtype),
                                      1 if aligned16 else 0, buf, 256), ctx)
    return buf.value.decode()


def proj_num_candidates_packed(M, N, K, tile16, epilogue, out_dtype, aligned16=True) -> int:
    return int(lib().proj_num_candidates_packed(int(M), int(N), int(K), int(tile16), int(epilogue), int(out_dtype),
                                                1 if aligned16 else 0))


def proj_candidate_name_packed(M, N, K, tile16, epilogue, out_dtype, index, aligned16=True) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().proj_candidate_name_packed(int(M), int(N), int(K), int(tile16), int(epilogue), int(out_dtype),
                                            1 if aligned16 else 0, int(index), buf, 256))
    return buf.value.decode()


def proj_run_candidate_packed(ctx, index, X, Wp, tile16, bias, epilogue, Y, N, M=None, K=None, out_dtype=None,
                              stream=None) -> None:
    _check_operands(X, Wp, bias, Y)
    M = int(X.shape[0] if M is None else M)
    K = int(X.shape[1] if K is None else K)
    _check(lib().proj_run_candidate_packed(ctx, int(index), _ptr(X), _ptr(Wp), int(tile16), _ptr(bias),
                                           int(epilogue), M, int(N), K, _ptr(Y), _out_dtype(Y, out_dtype),
                                           _stream(stream)), ctx)


def proj_graph_capture(ctx, Xs, Ws, biases, Ys, epilogue, out_dtype=None, stream=None) -> int:
    """Capture len(Xs) calls (call i on Xs[i], Ws[i], biases[i], Ys[i]) into
    one instantiated HIP graph; returns its handle.  `stream` must not be the
    legacy default stream."""
    n = len(Xs)
    if not (len(Ws) == n and len(Ys) == n and (biases is None or len(biases) == n)):
        raise ValueError("buffer lists differ in length")
    for i in range(n):
        _check_operands(Xs[i], Ws[i], biases[i] if biases else None, Ys[i])
    M, N, K = _shape(Xs[0], Ws[0], None, None, None)
    arr = ctypes.c_void_p * n
    xs = arr(*[_ptr(t) for t in Xs])
    ws = arr(*[_ptr(t) for t in Ws])
    bs = arr(*[_ptr(t) for t in biases]) if biases else None
    ys = arr(*[_ptr(t) for t in Ys])
    g = ctypes.c_void_p()
    _check(lib().proj_graph_capture(ctx, n, xs, ws, bs, ys, int(epilogue), M, N, K,
                                    _out_dtype(Ys[0], out_dtype), _stream(stream), ctypes.byref(g)), ctx)
    return g.value


def proj_read_probe(ctx, buf, stream=None) -> None:
    """Enqueue one plain streaming read of the whole of tensor `buf` (its
    bytes a multiple of 16): the measured read floor to time beside
    proj_run on the same buffers."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().proj_read_probe(ctx, _ptr(buf), nbytes, _stream(stream)), ctx)


def proj_graph_launch(graph, stream=None) -> None:
    _check(lib().proj_graph_launch(graph, _stream(stream)))


def proj_graph_destroy(graph) -> None:
    _check(lib().proj_graph_destroy(graph))


# ------------------------------------------------------------ convenience

def project(ctx, X, W, bias=None, gelu=False, out_dtype=None, stream=None):
    """Allocate Y with torch and run the projection; returns Y."""
    import torch
    epi = (EPI_BIAS if bias is not None else EPI_NONE) | (EPI_GELU_TANH if gelu else 0)
    dt = torch.bfloat16 if out_dtype in (None, OUT_BF16, torch.bfloat16) else torch.float32
    Y = torch.empty((X.shape[0], W.shape[0]), dtype=dt, device=X.device)
    proj_run(ctx, X, W, bias, epi, Y, stream=stream)
    return Y
