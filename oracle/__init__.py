"""fp64 CPU oracle for one exact Lloyd k-means iteration (batched).

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  The GPU library and
its Python binding never import it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over points); this
module only marshals numpy arrays.  What each function computes, and which
passage of the pages it follows, is stated in ``oracle.c``.

Conventions (readings where the pages are silent):
  * labels are 0-based int32; the lowest index wins an exact tie;
  * an empty cluster keeps its previous centroid;
  * counts are exact integers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}

_default = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile oracle.c with gcc into a shared library (in-tree by default)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_abi_version.restype = I
    lib.oracle_max_threads.restype = I
    lib.oracle_decode.argtypes = [I, P, I64, P]
    lib.oracle_encode_f16_rne.argtypes = [P, I64, P]
    lib.oracle_encode_bf16_rne.argtypes = [P, I64, P]
    lib.oracle_assign.argtypes = [I, I, I64, I64, I64, I64, P, P, P, I64, P, P, P, I]
    lib.oracle_update.argtypes = [I, I, I64, I64, I64, I64, P, P, P, P, P, I]
    lib.oracle_update.restype = I64
    lib.oracle_lloyd.argtypes = [I, I64, I64, I64, I64, P, P, I64, P, P, P, I]
    lib.oracle_pair_dist.argtypes = [I, I, I64, I64, I64, I64, P, P, P, P, I64, P]
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_name(a: np.ndarray, name: str | None) -> str:
    """Stored dtype of an array.  16-bit floats travel as uint16 bit patterns,
    so their format ('f16' or 'bf16') must be named explicitly."""
    if name is not None:
        return name
    if a.dtype == np.float32:
        return "f32"
    if a.dtype == np.float64:
        return "f64"
    if a.dtype == np.float16:
        return "f16"
    raise ValueError(f"name the 16-bit format of a {a.dtype} array ('f16' or 'bf16')")


def _as_storage(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return a


class Oracle:
    """The oracle library loaded from one shared object (the in-tree build by
    default; tests also load deliberately broken builds to check the pins)."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = _LIB_PATH
            if not os.path.exists(path):
                build()
        self.path = path
        self.lib = _bind(ctypes.CDLL(path))

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def decode(self, a: np.ndarray, fmt: str | None = None) -> np.ndarray:
        """Exact fp64 value of every stored element (the oracle's own decoder)."""
        fmt = _dtype_name(a, fmt)
        s = _as_storage(a)
        out = np.empty(s.shape, dtype=np.float64)
        self.lib.oracle_decode(DTYPE_CODE[fmt], _ptr(s), s.size, _ptr(out))
        return out

    def encode_rne(self, a: np.ndarray, fmt: str) -> np.ndarray:
        """fp32 -> fp16/bf16 bit patterns (uint16), round to nearest, ties to even."""
        src = np.ascontiguousarray(a, dtype=np.float32)
        out = np.empty(src.shape, dtype=np.uint16)
        fn = {"f16": self.lib.oracle_encode_f16_rne, "bf16": self.lib.oracle_encode_bf16_rne}[fmt]
        fn(_ptr(src), src.size, _ptr(out))
        return out

    def assign(self, X: np.ndarray, C: np.ndarray, fmt_x: str | None = None, fmt_c: str | None = None,
               rows: np.ndarray | None = None, nthreads: int = 0):
        """Nearest centroid per point, lowest index on exact ties.

        X: (B, N, d) stored dtype; C: (B, K, d) stored dtype (or fp64).
        rows: optional flattened point ids (b*N + i) to evaluate one by one.
        Returns (labels int32, d1 fp64, d2 fp64): d1 = nearest squared distance,
        d2 = second nearest over the other centroids (d2 == d1 on an exact tie).
        """
        B, N, d = X.shape
        Bc, K, dc = C.shape
        assert (Bc, dc) == (B, d)
        fx, fc = _dtype_name(X, fmt_x), _dtype_name(C, fmt_c)
        Xs, Cs = _as_storage(X), _as_storage(C)
        if rows is None:
            shape = (B, N)
            n = B * N
            rows_arr = None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            assert rows_arr.min(initial=0) >= 0 and rows_arr.max(initial=0) < B * N
            shape = rows_arr.shape
            n = rows_arr.size
        labels = np.empty(shape, dtype=np.int32)
        d1 = np.empty(shape, dtype=np.float64)
        d2 = np.empty(shape, dtype=np.float64)
        self.lib.oracle_assign(DTYPE_CODE[fx], DTYPE_CODE[fc], B, N, K, d, _ptr(Xs), _ptr(Cs),
                              _ptr(rows_arr), n, _ptr(labels), _ptr(d1), _ptr(d2), nthreads)
        return labels, d1, d2

    def pair_dist(self, X: np.ndarray, C: np.ndarray, points: np.ndarray, cents: np.ndarray,
                  fmt_x: str | None = None, fmt_c: str | None = None) -> np.ndarray:
        """fp64 squared distance of each (flattened point id, centroid index) pair."""
        B, N, d = X.shape
        _, K, _ = C.shape
        fx, fc = _dtype_name(X, fmt_x), _dtype_name(C, fmt_c)
        Xs, Cs = _as_storage(X), _as_storage(C)
        pts = np.ascontiguousarray(points, dtype=np.int64).reshape(-1)
        cen = np.ascontiguousarray(cents, dtype=np.int32).reshape(-1)
        assert pts.size == cen.size
        assert pts.size == 0 or (pts.min() >= 0 and pts.max() < B * N)
        assert cen.size == 0 or (cen.min() >= 0 and cen.max() < K)
        out = np.empty(pts.size, dtype=np.float64)
        self.lib.oracle_pair_dist(DTYPE_CODE[fx], DTYPE_CODE[fc], B, N, K, d, _ptr(Xs), _ptr(Cs),
                                  _ptr(pts), _ptr(cen), pts.size, _ptr(out))
        return out

    def update(self, X: np.ndarray, labels: np.ndarray, C_prev: np.ndarray, fmt_x: str | None = None,
               fmt_c: str | None = None, nthreads: int = 0):
        """Counts and per-cluster means from a given label vector.

        X: (B, N, d) stored dtype; labels: (B, N) int32; C_prev: (B, K, d) (fp32
        or fp64), the centroids an empty cluster keeps.
        Returns (counts int64 (B, K), C_next fp64 (B, K, d), n_bad_labels).
        """
        B, N, d = X.shape
        Bc, K, dc = C_prev.shape
        assert (Bc, dc) == (B, d) and labels.shape == (B, N)
        fx, fc = _dtype_name(X, fmt_x), _dtype_name(C_prev, fmt_c)
        Xs, Cs = _as_storage(X), _as_storage(C_prev)
        lab = np.ascontiguousarray(labels, dtype=np.int32)
        counts = np.empty((B, K), dtype=np.int64)
        C_next = np.empty((B, K, d), dtype=np.float64)
        bad = self.lib.oracle_update(DTYPE_CODE[fx], DTYPE_CODE[fc], B, N, K, d, _ptr(Xs), _ptr(lab),
                                    _ptr(Cs), _ptr(counts), _ptr(C_next), nthreads)
        return counts, C_next, int(bad)

    def lloyd(self, X: np.ndarray, C0: np.ndarray, T: int, fmt_x: str | None = None, nthreads: int = 0):
        """Free-running fp64 Lloyd: T x (assign, update) with fp64 centroids.

        Returns (C_T fp64, labels of the last assign, counts of the last assign,
        objective per iteration fp64 (T,)).
        """
        B, N, d = X.shape
        _, K, _ = C0.shape
        fx = _dtype_name(X, fmt_x)
        Xs = _as_storage(X)
        C = np.ascontiguousarray(C0, dtype=np.float64).copy()
        labels = np.empty((B, N), dtype=np.int32)
        counts = np.empty((B, K), dtype=np.int64)
        obj = np.empty((T,), dtype=np.float64)
        self.lib.oracle_lloyd(DTYPE_CODE[fx], B, N, K, d, _ptr(Xs), _ptr(C), T, _ptr(labels),
                             _ptr(counts), _ptr(obj), nthreads)
        return C, labels, counts, obj


def argsort_valid(labels: np.ndarray, sorted_idx: np.ndarray, K: int) -> bool:
    """True iff sorted_idx (B, N) is, per problem, a permutation of 0..N-1 that
    lists points in nondecreasing label order (any order within a label is a
    correct argsort; only the grouping is unique)."""
    B, N = labels.shape
    if sorted_idx.shape != (B, N):
        return False
    for b in range(B):
        s = sorted_idx[b].astype(np.int64)
        if s.min(initial=0) < 0 or s.max(initial=0) >= N:
            return False
        if np.bincount(s, minlength=N).max(initial=1) != 1:
            return False
        lab = labels[b][s]
        if np.any(lab[1:] < lab[:-1]):
            return False
    return True


def default() -> Oracle:
    """The in-tree oracle (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def max_threads() -> int:
    return default().max_threads()


def decode(*a, **k):
    return default().decode(*a, **k)


def encode_rne(*a, **k):
    return default().encode_rne(*a, **k)


def assign(*a, **k):
    return default().assign(*a, **k)


def update(*a, **k):
    return default().update(*a, **k)


def pair_dist(*a, **k):
    return default().pair_dist(*a, **k)


def lloyd(*a, **k):
    return default().lloyd(*a, **k)
