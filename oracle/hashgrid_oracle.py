"""Python handle on the CPU oracle (``hashgrid_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package's smoke check
and by the CPU-baseline leg of the benchmark, never by the product path.  It
shares no code with the HIP library; inputs come from the shared seeded
generator module, which holds none of the method's arithmetic.

Every function takes and returns numpy arrays; results are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hashgrid_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_handle = None


class OracleGrid(ctypes.Structure):
    _fields_ = [
        ("n_dims", ctypes.c_int32),
        ("n_levels", ctypes.c_int32),
        ("n_features", ctypes.c_int32),
        ("log2_table_size", ctypes.c_int32),
        ("base_resolution", ctypes.c_int32),
        ("finest_resolution", ctypes.c_int32),
        ("table_is_half", ctypes.c_int32),
    ]


def build() -> str:
    """Compile the oracle with the host C compiler (plain C11, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _lib():
    global _handle
    with _lock:
        if _handle is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            G = ctypes.POINTER(OracleGrid)
            lib.oracle_resolutions.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
            lib.oracle_corners.argtypes = [G, P, ctypes.c_int64, P, P]
            lib.oracle_forward.argtypes = [G, P, ctypes.c_int64, P, P]
            lib.oracle_backward.argtypes = [G, P, ctypes.c_int64, P, ctypes.c_int64, P]
            lib.oracle_input_grad.argtypes = [G, P, ctypes.c_int64, P, P, ctypes.c_int64, P]
            lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_half_to_double.restype = ctypes.c_double
            lib.oracle_set_threads.argtypes = [ctypes.c_int]
            lib.oracle_get_threads.restype = ctypes.c_int
            _handle = lib
    return _handle


def set_threads(n: int) -> None:
    _lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_lib().oracle_get_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def grid(n_levels, n_features, log2_table_size, base_resolution, finest_resolution,
         table_dtype="f32", n_dims=3) -> OracleGrid:
    return OracleGrid(n_dims, n_levels, n_features, log2_table_size, base_resolution,
                      finest_resolution, 1 if table_dtype == "f16" else 0)


def grid_of(w) -> OracleGrid:
    """Grid of a workload from the shared input module."""
    return grid(w.n_levels, w.n_features, w.log2_table_size, w.base_resolution,
                w.finest_resolution, w.table_dtype, n_dims=getattr(w, "n_dims", 3))


def resolutions(n_levels: int, base_resolution: int, finest_resolution: int) -> np.ndarray:
    out = np.zeros(n_levels, dtype=np.int32)
    rc = _lib().oracle_resolutions(n_levels, base_resolution, finest_resolution, _ptr(out))
    if rc:
        raise ValueError("invalid resolution parameters")
    return out


def half_to_double(bits: int) -> float:
    return float(_lib().oracle_half_to_double(int(bits)))


def _points(g: OracleGrid, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] != g.n_dims:
        raise ValueError(f"points must be [n, {g.n_dims}] float32")
    return x


def _table(g: OracleGrid, table: np.ndarray) -> np.ndarray:
    want = np.float16 if g.table_is_half else np.float32
    t = np.ascontiguousarray(table, dtype=want)
    if t.shape != (g.n_levels, 1 << g.log2_table_size, g.n_features):
        raise ValueError(f"table shape {t.shape} does not match the grid")
    return t


def corners(g: OracleGrid, x: np.ndarray):
    """(idx uint32 [n, L, 2^D], w float64 [n, L, 2^D])."""
    x = _points(g, x)
    n = x.shape[0]
    K = 1 << g.n_dims
    idx = np.zeros((n, g.n_levels, K), dtype=np.uint32)
    w = np.zeros((n, g.n_levels, K), dtype=np.float64)
    if _lib().oracle_corners(ctypes.byref(g), _ptr(x), n, _ptr(idx), _ptr(w)):
        raise ValueError("invalid grid")
    return idx, w


def forward(g: OracleGrid, x: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Encoded features, float64 [n, L*F]."""
    x = _points(g, x)
    t = _table(g, table)
    out = np.zeros((x.shape[0], g.n_levels * g.n_features), dtype=np.float64)
    if _lib().oracle_forward(ctypes.byref(g), _ptr(x), x.shape[0], _ptr(t), _ptr(out)):
        raise ValueError("invalid grid")
    return out


def backward(g: OracleGrid, x: np.ndarray, dout: np.ndarray, grad: np.ndarray | None = None) -> np.ndarray:
    """Table gradient, float64 [L, T, F]; added into ``grad`` when given."""
    x = _points(g, x)
    dout = np.ascontiguousarray(dout, dtype=np.float32)
    if dout.ndim != 2 or dout.shape[0] != x.shape[0] or dout.shape[1] < g.n_levels * g.n_features:
        raise ValueError("dout must be [n, >= L*F] float32")
    shape = (g.n_levels, 1 << g.log2_table_size, g.n_features)
    if grad is None:
        grad = np.zeros(shape, dtype=np.float64)
    elif grad.shape != shape or grad.dtype != np.float64 or not grad.flags.c_contiguous:
        raise ValueError("grad must be a contiguous float64 [L, T, F] array")
    if _lib().oracle_backward(ctypes.byref(g), _ptr(x), x.shape[0], _ptr(dout), dout.shape[1], _ptr(grad)):
        raise ValueError("invalid grid")
    return grad


def input_grad(g: OracleGrid, x: np.ndarray, table: np.ndarray, dout: np.ndarray) -> np.ndarray:
    """dL/dx [n, D] float64 of upstream dL/dout [n, >= L*F] (oracle_input_grad)."""
    x = _points(g, x)
    t = _table(g, table)
    dout = np.ascontiguousarray(dout, dtype=np.float32)
    n = x.shape[0]
    if dout.ndim != 2 or dout.shape[0] != n or dout.shape[1] < g.n_levels * g.n_features:
        raise ValueError("dout must be [n, >= L*F]")
    dx = np.zeros((n, g.n_dims), dtype=np.float64)
    if _lib().oracle_input_grad(ctypes.byref(g), _ptr(x), n, _ptr(t), _ptr(dout), dout.shape[1], _ptr(dx)):
        raise ValueError("bad grid")
    return dx
