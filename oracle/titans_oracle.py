"""ctypes wrapper of the fp64 oracle (titans_oracle.c).

TEST INFRASTRUCTURE ONLY.  Argument marshalling and the gcc build step live
here; every step of the method is in the C file, which follows the update,
forgetting and retrieval rules of "Titans: Learning to Memorize at Test
Time" (mer.dev notes, sections 3.1 and 3.2) token by token in float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "titans_oracle.c")
_LIB = os.path.join(_HERE, "libtitans_oracle.so")
_lib = None

_dptr = ctypes.POINTER(ctypes.c_double)


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (strict IEEE fp64: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.tmo_param_count.restype = ctypes.c_int64
        lib.tmo_param_count.argtypes = [ctypes.c_int] * 3
        lib.tmo_memory_apply.restype = ctypes.c_int
        lib.tmo_memory_apply.argtypes = [ctypes.c_int] * 3 + [_dptr] * 3
        lib.tmo_memory_grad.restype = ctypes.c_int
        lib.tmo_memory_grad.argtypes = [ctypes.c_int] * 3 + [_dptr] * 5
        lib.tmo_forward.restype = ctypes.c_int
        lib.tmo_forward.argtypes = [ctypes.c_int] * 7 + [_dptr] * 12 + [ctypes.c_int]
        lib.tmo_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.cast(None, _dptr)
    return a.ctypes.data_as(_dptr)


def max_threads() -> int:
    return int(_load().tmo_max_threads())


def param_count(d: int, hidden: int, n_layers: int) -> int:
    p = int(_load().tmo_param_count(d, hidden, n_layers))
    if p < 0:
        raise ValueError("bad memory shape")
    return p


def memory_apply(W: np.ndarray, x: np.ndarray, d: int, hidden: int, n_layers: int) -> np.ndarray:
    """M_W(x) for one vector."""
    W, x = _c(W), _c(x)
    y = np.empty(d)
    rc = _load().tmo_memory_apply(d, hidden, n_layers, _p(W), _p(x), _p(y))
    if rc:
        raise RuntimeError(f"tmo_memory_apply failed ({rc})")
    return y


def memory_grad(W: np.ndarray, k: np.ndarray, v: np.ndarray, d: int, hidden: int,
                n_layers: int) -> Tuple[np.ndarray, float]:
    """(grad of 0.5||M_W(k) - v||^2 w.r.t. W, that loss)."""
    W, k, v = _c(W), _c(k), _c(v)
    g = np.empty_like(W)
    loss = np.zeros(1)
    rc = _load().tmo_memory_grad(d, hidden, n_layers, _p(W), _p(k), _p(v), _p(g), _p(loss))
    if rc:
        raise RuntimeError(f"tmo_memory_grad failed ({rc})")
    return g, float(loss[0])


def forward(k, v, q, alpha, eta, theta, W_in, S_in, *, d: int, hidden: int, n_layers: int,
            chunk: int, read_mode: int = 0, threads: int = 0, want_w_norm: bool = False,
            chunk_gates: bool = False):
    """Chunked memory over independent streams (leading axis of every array).

    k, v, q: [S, N, d]; alpha, eta, theta: [S, N]; W_in, S_in: [S, P].
    Returns (y [S,N,d], W_out [S,P], S_out [S,P]) and, if asked, the
    per-chunk ||W||_F trajectory [S, ceil(N/chunk)].

    chunk_gates: alpha, eta, theta are [S, ceil(N/chunk)], one value per
    chunk shared by all its tokens ("Parameters as the Function of Chunks",
    mer.dev notes section 3.2); the token loop then runs with each token
    taking its chunk's values.
    """
    k, v, q = _c(k), _c(v), _c(q)
    if chunk_gates:
        N = k.shape[1]
        alpha, eta, theta = (np.repeat(np.asarray(g, np.float64), chunk, axis=1)[:, :N]
                             for g in (alpha, eta, theta))
    alpha, eta, theta = _c(alpha), _c(eta), _c(theta)
    W_in, S_in = _c(W_in), _c(S_in)
    S, N = alpha.shape
    P = param_count(d, hidden, n_layers)
    if k.shape != (S, N, d) or v.shape != (S, N, d) or q.shape != (S, N, d):
        raise ValueError("k, v, q must be [S, N, d]")
    if W_in.shape != (S, P) or S_in.shape != (S, P):
        raise ValueError("W_in, S_in must be [S, P]")
    y = np.empty((S, N, d))
    W_out = np.empty((S, P))
    S_out = np.empty((S, P))
    n_chunks = (N + chunk - 1) // chunk if chunk > 0 else 0
    wn = np.empty((S, n_chunks)) if want_w_norm else None
    rc = _load().tmo_forward(S, N, d, hidden, n_layers, chunk, read_mode,
                             _p(k), _p(v), _p(q), _p(alpha), _p(eta), _p(theta),
                             _p(W_in), _p(S_in), _p(y), _p(W_out), _p(S_out), _p(wn),
                             int(threads))
    if rc:
        raise RuntimeError(f"tmo_forward failed ({rc})")
    if want_w_norm:
        return y, W_out, S_out, wn
    return y, W_out, S_out
