"""Python binding of libfk, the exact batched Lloyd k-means library for MI355X.

Argument marshalling only: shapes, dtypes, data pointers and the stream of
torch tensors are passed to the C ABI declared in include/fk.h, and a
non-zero status raises FKError.  Every step of the computation runs in the
library's HIP kernels; torch only owns the device memory and the stream.

Importing this package loads libfk.so and fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfk.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python exact_lloyd_means_amd/build.py` "
        "(or __graft_entry__.build()) first")

lib = ctypes.CDLL(LIB_PATH)

FK_F32, FK_F16, FK_BF16 = 0, 1, 2
FK_OK, FK_EINVAL, FK_EUNSUPPORTED, FK_EWORKSPACE, FK_EHIP, FK_EHOST = 0, -1, -2, -3, -4, -5
FK_DETERMINISTIC = 1

DTYPES = {torch.float32: FK_F32, torch.float16: FK_F16, torch.bfloat16: FK_BF16}


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("d", ctypes.c_int64), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


_P = ctypes.c_void_p
_PP = ctypes.POINTER(Problem)
_SIG = {
    "fk_abi_version": ([], ctypes.c_int),
    "fk_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "fk_last_error": ([], ctypes.c_char_p),
    "fk_workspace_size": ([_PP, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "fk_workspace_bytes": ([_PP, ctypes.c_int64], ctypes.c_size_t),
    "fk_centroid_bias": ([_PP, _P, _P, _P], ctypes.c_int),
    "fk_assign": ([_PP, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "fk_assign_with_bias": ([_PP, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "fk_sort_labels": ([_PP, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "fk_update": ([_PP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "fk_update_bias": ([_PP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "fk_update_bias_noalloc": ([_PP, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "fk_lloyd": ([_PP, _P, _P, _P, _P, ctypes.c_int, ctypes.c_float,
                  ctypes.POINTER(ctypes.c_int), _P, ctypes.c_size_t, _P], ctypes.c_int),
    "fk_lloyd_streamed": ([_PP, _P, ctypes.c_int64, _P, _P, _P, ctypes.c_int, _P, ctypes.c_size_t,
                           _P, _P], ctypes.c_int),
    "fk_error_count": ([_PP, _P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int64), _P],
                       ctypes.c_int),
    # include/fk_baseline.h
    "fk_baseline_scores": ([_PP, _P, _P, _P, _P, _P], ctypes.c_int),
    "fk_baseline_argmin": ([_PP, _P, _P, _P], ctypes.c_int),
    "fk_baseline_update_scatter": ([_PP, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    # include/fk_tune.h
    "fk_assign_variant": ([_PP, _P, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int64, _P],
                          ctypes.c_int),
}
for _name, (_args, _res) in _SIG.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class FKError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.fk_status_str(status).decode()
        detail = lib.fk_last_error().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail else ""))


def _check(status: int, where: str) -> None:
    if status != FK_OK:
        raise FKError(status, where)


def problem(B: int, N: int, K: int, d: int, dtype, deterministic: bool = False) -> Problem:
    code = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return Problem(B, N, K, d, code, FK_DETERMINISTIC if deterministic else 0)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libfk must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _want(t, name: str, dtype, shape, device=None, optional: bool = False) -> None:
    """Raise ValueError unless t is a tensor of this dtype (one dtype or a
    tuple of them), exactly this shape and, when device is given, on that
    device.  The kernels index every buffer by (B, N, K, d) alone, so a
    tensor of the wrong type or size would be read or written out of
    bounds; these checks run before anything reaches the library."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    dtypes = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(x) for x in dtypes)}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _device(t: torch.Tensor, name: str) -> torch.device:
    """Device of the tensor every other argument must share."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    return t.device


def _need_gpu(dev: torch.device) -> None:
    # checked after dtypes and shapes, so those errors name the argument
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on the GPU, got {dev}")


def _want_ws(ws, dev) -> None:
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError("ws must be a 1-D uint8 tensor (see workspace())")
    if ws.device != dev:
        raise ValueError(f"ws is on {ws.device}, expected {dev}")
    if not ws.is_contiguous():
        raise ValueError("ws must be contiguous")


_FLOATS = (torch.float32, torch.float16, torch.bfloat16)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _problem_from(X: torch.Tensor, K: int, deterministic: bool = False) -> Problem:
    if not isinstance(X, torch.Tensor):
        raise TypeError("X must be a torch tensor")
    if X.dim() != 3:
        raise ValueError("X must be (B, N, d)")
    if X.dtype not in _FLOATS:
        raise ValueError(f"X must be float32, float16 or bfloat16, got {X.dtype}")
    B, N, d = X.shape
    return problem(B, N, K, d, X.dtype, deterministic)


def abi_version() -> int:
    return lib.fk_abi_version()


def workspace_size(p: Problem, chunk_points: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.fk_workspace_size(ctypes.byref(p), chunk_points, ctypes.byref(n)),
           "fk_workspace_size")
    return n.value


def workspace(p: Problem, device=None, chunk_points: int = 0) -> torch.Tensor:
    """A caller-owned device workspace of the required size (allocated by torch)."""
    return torch.empty(workspace_size(p, chunk_points), dtype=torch.uint8,
                       device=device or "cuda")


def fk_centroid_bias(C: torch.Tensor, bias: torch.Tensor, stream=None) -> None:
    dev = _device(C, "C")
    if C.dim() != 3:
        raise ValueError("C must be (B, K, d)")
    B, K, d = C.shape
    _want(C, "C", _FLOATS, (B, K, d), dev)
    _want(bias, "bias", torch.float32, (B, K), dev)
    _need_gpu(dev)
    p = problem(B, 1, K, d, C.dtype)
    _check(lib.fk_centroid_bias(ctypes.byref(p), _ptr(C), _ptr(bias), _stream(stream)),
           "fk_centroid_bias")


def _assign_args(X, C, labels, min_dist):
    dev = _device(X, "X")
    if not isinstance(C, torch.Tensor) or C.dim() != 3:
        raise ValueError("C must be a (B, K, d) tensor")
    p = _problem_from(X, C.shape[1])
    _want(X, "X", X.dtype, (p.B, p.N, p.d), dev)
    _want(C, "C", X.dtype, (p.B, p.K, p.d), dev)
    _want(labels, "labels", torch.int32, (p.B, p.N), dev)
    _want(min_dist, "min_dist", torch.float32, (p.B, p.N), dev, optional=True)
    return p, dev


def fk_assign(X: torch.Tensor, C: torch.Tensor, labels: torch.Tensor,
              min_dist: torch.Tensor | None = None, ws: torch.Tensor | None = None,
              stream=None) -> None:
    p, dev = _assign_args(X, C, labels, min_dist)
    _want_ws(ws, dev)
    _need_gpu(dev)
    ws = workspace(p, dev) if ws is None else ws
    _check(lib.fk_assign(ctypes.byref(p), _ptr(X), _ptr(C), _ptr(labels), _ptr(min_dist),
                         _ptr(ws), ws.numel(), _stream(stream)), "fk_assign")


def fk_assign_with_bias(X: torch.Tensor, C: torch.Tensor, bias: torch.Tensor,
                        labels: torch.Tensor, min_dist: torch.Tensor | None = None,
                        stream=None) -> None:
    p, dev = _assign_args(X, C, labels, min_dist)
    _want(bias, "bias", torch.float32, (p.B, p.K), dev)
    _need_gpu(dev)
    _check(lib.fk_assign_with_bias(ctypes.byref(p), _ptr(X), _ptr(C), _ptr(bias), _ptr(labels),
                                   _ptr(min_dist), _stream(stream)), "fk_assign_with_bias")


def fk_sort_labels(labels: torch.Tensor, K: int, counts: torch.Tensor, offsets: torch.Tensor,
                   sorted_idx: torch.Tensor, ws: torch.Tensor | None = None,
                   stream=None, d: int = 1, dtype=torch.float32,
                   deterministic: bool = False) -> None:
    dev = _device(labels, "labels")
    if labels.dim() != 2:
        raise ValueError("labels must be (B, N)")
    B, N = labels.shape
    _want(labels, "labels", torch.int32, (B, N), dev)
    _want(counts, "counts", torch.int32, (B, K), dev)
    _want(offsets, "offsets", torch.int32, (B, K + 1), dev)
    _want(sorted_idx, "sorted_idx", torch.int32, (B, N), dev)
    _want_ws(ws, dev)
    _need_gpu(dev)
    p = problem(B, N, K, d, dtype, deterministic)
    ws = workspace(p, dev) if ws is None else ws
    _check(lib.fk_sort_labels(ctypes.byref(p), _ptr(labels), _ptr(counts), _ptr(offsets),
                              _ptr(sorted_idx), _ptr(ws), ws.numel(), _stream(stream)),
           "fk_sort_labels")


def _update_args(X, labels, C_prev, C_next, C_next_lowp, counts, deterministic):
    dev = _device(X, "X")
    if not isinstance(C_prev, torch.Tensor) or C_prev.dim() != 3:
        raise ValueError("C_prev must be a (B, K, d) tensor")
    p = _problem_from(X, C_prev.shape[1], deterministic)
    B, N, K, d = p.B, p.N, p.K, p.d
    _want(X, "X", X.dtype, (B, N, d), dev)
    _want(labels, "labels", torch.int32, (B, N), dev)
    _want(C_prev, "C_prev", torch.float32, (B, K, d), dev)
    _want(C_next, "C_next", torch.float32, (B, K, d), dev)
    _want(C_next_lowp, "C_next_lowp", X.dtype, (B, K, d), dev, optional=True)
    _want(counts, "counts", torch.int32, (B, K), dev)
    return p, dev


def fk_update(X: torch.Tensor, labels: torch.Tensor, C_prev: torch.Tensor, C_next: torch.Tensor,
              C_next_lowp: torch.Tensor | None, counts: torch.Tensor,
              ws: torch.Tensor | None = None, stream=None, deterministic: bool = False) -> None:
    p, dev = _update_args(X, labels, C_prev, C_next, C_next_lowp, counts, deterministic)
    _want_ws(ws, dev)
    _need_gpu(dev)
    ws = workspace(p, dev) if ws is None else ws
    _check(lib.fk_update(ctypes.byref(p), _ptr(X), _ptr(labels), _ptr(C_prev), _ptr(C_next),
                         _ptr(C_next_lowp), _ptr(counts), _ptr(ws), ws.numel(),
                         _stream(stream)), "fk_update")


def fk_update_bias(X: torch.Tensor, labels: torch.Tensor, C_prev: torch.Tensor,
                   C_next: torch.Tensor, C_next_lowp: torch.Tensor | None, counts: torch.Tensor,
                   bias_next: torch.Tensor, ws: torch.Tensor | None = None, stream=None,
                   deterministic: bool = False) -> None:
    """fk_update that also writes the next assignment's centroid bias."""
    p, dev = _update_args(X, labels, C_prev, C_next, C_next_lowp, counts, deterministic)
    _want(bias_next, "bias_next", torch.float32, (p.B, p.K), dev)
    _want_ws(ws, dev)
    _need_gpu(dev)
    ws = workspace(p, dev) if ws is None else ws
    _check(lib.fk_update_bias(ctypes.byref(p), _ptr(X), _ptr(labels), _ptr(C_prev), _ptr(C_next),
                              _ptr(C_next_lowp), _ptr(counts), _ptr(bias_next), _ptr(ws),
                              ws.numel(), _stream(stream)), "fk_update_bias")


def fk_update_bias_noalloc(X: torch.Tensor, labels: torch.Tensor, C_prev: torch.Tensor,
                           C_next: torch.Tensor, C_next_lowp: torch.Tensor | None,
                           counts: torch.Tensor, bias_next: torch.Tensor, stream=None,
                           deterministic: bool = False) -> None:
    """fk_update_bias on the library's static per-device scratch: no
    workspace, nothing allocated.  Calls that overlap on one GPU race."""
    p, dev = _update_args(X, labels, C_prev, C_next, C_next_lowp, counts, deterministic)
    _want(bias_next, "bias_next", torch.float32, (p.B, p.K), dev)
    _need_gpu(dev)
    _check(lib.fk_update_bias_noalloc(ctypes.byref(p), _ptr(X), _ptr(labels), _ptr(C_prev),
                                      _ptr(C_next), _ptr(C_next_lowp), _ptr(counts),
                                      _ptr(bias_next), _stream(stream)),
           "fk_update_bias_noalloc")


def _lloyd_args(X, C, labels, counts, deterministic, x_device=True):
    if not isinstance(C, torch.Tensor) or C.dim() != 3:
        raise ValueError("C must be a (B, K, d) tensor")
    dev = _device(C, "C")
    p = _problem_from(X, C.shape[1], deterministic)
    B, N, K, d = p.B, p.N, p.K, p.d
    _want(X, "X", X.dtype, (B, N, d), dev if x_device else torch.device("cpu"))
    _want(C, "C", torch.float32, (B, K, d), dev)
    _want(labels, "labels", torch.int32, (B, N), dev)
    _want(counts, "counts", torch.int32, (B, K), dev)
    return p, dev


def fk_lloyd(X: torch.Tensor, C: torch.Tensor, labels: torch.Tensor, counts: torch.Tensor,
             max_iters: int, tol: float = 0.0, want_n_iter: bool = False,
             ws: torch.Tensor | None = None, stream=None, deterministic: bool = False):
    """Runs Lloyd iterations in place on the fp32 centroids C.  Returns the
    number of iterations run when want_n_iter (one sync per iteration)."""
    p, dev = _lloyd_args(X, C, labels, counts, deterministic)
    _want_ws(ws, dev)
    _need_gpu(dev)
    ws = workspace(p, dev) if ws is None else ws
    n = ctypes.c_int(0)
    _check(lib.fk_lloyd(ctypes.byref(p), _ptr(X), _ptr(C), _ptr(labels), _ptr(counts),
                        int(max_iters), float(tol), ctypes.byref(n) if want_n_iter else None,
                        _ptr(ws), ws.numel(), _stream(stream)), "fk_lloyd")
    return n.value if want_n_iter else None


def fk_lloyd_streamed(X_host: torch.Tensor, C: torch.Tensor, labels: torch.Tensor,
                      counts: torch.Tensor, max_iters: int, chunk_points: int,
                      ws: torch.Tensor | None = None, compute_stream=None, copy_stream=None,
                      deterministic: bool = False) -> None:
    """Lloyd iterations on a pinned host tensor X_host (B, N, d), streamed to
    the GPU in chunks of chunk_points points; C, labels, counts on the GPU."""
    p, dev = _lloyd_args(X_host, C, labels, counts, deterministic, x_device=False)
    if not X_host.is_pinned():
        raise ValueError("X_host must be a pinned CPU tensor (pin_memory=True)")
    _want_ws(ws, dev)
    _need_gpu(dev)
    ws = workspace(p, dev, chunk_points) if ws is None else ws
    cs = _stream(compute_stream)
    xs = _stream(copy_stream) if copy_stream is not None else cs
    _check(lib.fk_lloyd_streamed(ctypes.byref(p), _ptr(X_host), int(chunk_points), _ptr(C),
                                 _ptr(labels), _ptr(counts), int(max_iters), _ptr(ws), ws.numel(),
                                 cs, xs), "fk_lloyd_streamed")


def fk_error_count(p: Problem, ws: torch.Tensor, stream=None) -> int:
    _want_ws(ws, _device(ws, "ws"))
    _need_gpu(ws.device)
    n = ctypes.c_int64(0)
    _check(lib.fk_error_count(ctypes.byref(p), _ptr(ws), ws.numel(), ctypes.byref(n),
                              _stream(stream)), "fk_error_count")
    return n.value


# ---- baselines (include/fk_baseline.h): the unfused forms, for comparison --

def fk_baseline_scores(X: torch.Tensor, C: torch.Tensor, bias: torch.Tensor,
                       D: torch.Tensor, stream=None) -> None:
    """D (B, N, K) fp32 = X . C^T + bias, written to memory in full."""
    dev = _device(X, "X")
    if not isinstance(C, torch.Tensor) or C.dim() != 3:
        raise ValueError("C must be a (B, K, d) tensor")
    p = _problem_from(X, C.shape[1])
    _want(C, "C", X.dtype, (p.B, p.K, p.d), dev)
    _want(bias, "bias", torch.float32, (p.B, p.K), dev)
    _want(D, "D", torch.float32, (p.B, p.N, p.K), dev)
    _need_gpu(dev)
    _check(lib.fk_baseline_scores(ctypes.byref(p), _ptr(X), _ptr(C), _ptr(bias), _ptr(D),
                                  _stream(stream)), "fk_baseline_scores")


def fk_baseline_argmin(D: torch.Tensor, labels: torch.Tensor, stream=None) -> None:
    dev = _device(D, "D")
    if D.dim() != 3:
        raise ValueError("D must be (B, N, K)")
    B, N, K = D.shape
    _want(D, "D", torch.float32, (B, N, K), dev)
    _want(labels, "labels", torch.int32, (B, N), dev)
    _need_gpu(dev)
    p = problem(B, N, K, 1, torch.float32)
    _check(lib.fk_baseline_argmin(ctypes.byref(p), _ptr(D), _ptr(labels), _stream(stream)),
           "fk_baseline_argmin")


def fk_baseline_update_scatter(X: torch.Tensor, labels: torch.Tensor, C_prev: torch.Tensor,
                               C_next: torch.Tensor, C_next_lowp: torch.Tensor | None,
                               counts: torch.Tensor, sums: torch.Tensor, stream=None) -> None:
    p, dev = _update_args(X, labels, C_prev, C_next, C_next_lowp, counts, False)
    _want(sums, "sums", torch.float32, (p.B, p.K, p.d), dev)
    _need_gpu(dev)
    _check(lib.fk_baseline_update_scatter(ctypes.byref(p), _ptr(X), _ptr(labels), _ptr(C_prev),
                                          _ptr(C_next), _ptr(C_next_lowp), _ptr(counts),
                                          _ptr(sums), _stream(stream)),
           "fk_baseline_update_scatter")


def fk_assign_variant(X: torch.Tensor, C: torch.Tensor, bias: torch.Tensor, labels: torch.Tensor,
                      point_blocks: int, waves: int, grid_wgs: int = 0, stream=None) -> None:
    """The fp16 fused assign with an explicit kernel shape (include/fk_tune.h)."""
    p, dev = _assign_args(X, C, labels, None)
    _want(bias, "bias", torch.float32, (p.B, p.K), dev)
    _need_gpu(dev)
    _check(lib.fk_assign_variant(ctypes.byref(p), _ptr(X), _ptr(C), _ptr(bias), _ptr(labels),
                                 int(point_blocks), int(waves), int(grid_wgs), _stream(stream)),
           "fk_assign_variant")


from .api import KMeans, batch_kmeans_euclid, initial_centroids  # noqa: E402  (uses the above)
