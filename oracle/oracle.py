"""Oracle for SparseConv2D -- TEST INFRASTRUCTURE ONLY.

ctypes wrapper over ``oracle.c`` (plain CPU loops, float64).  Only the test
suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this module.  It imports nothing from the HIP library package and
the library never imports it.

Every function takes numpy arrays, converts floating inputs to float64
(exactly: bf16 and fp32 values are representable in float64) and returns
float64 results.  See ``oracle.c`` for the definitions and the passages of
"SV-TAD: Native Sparse Convolutions for Efficient Temporal Action Detection"
(paper notes page: Overall Architecture, Key Designs 1 to 3) that each one
follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

STATUS_OK = 0
STATUS_BAD_ARGS = 1
STATUS_COORD_RANGE = 5
STATUS_DUPLICATE = 6


def compile_source(src: str, out: str) -> str:
    """gcc -O3 -fopenmp: one C file to one shared library (with libm)."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O3", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                           src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


class Oracle:
    """One loaded build of oracle.c (the default build, or -- in the pin
    tests only -- a deliberately mutated copy)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.orc_threads.argtypes = [ctypes.c_int]
        lib.orc_threads.restype = ctypes.c_int
        lib.orc_build_index.argtypes = [P, P, i32, i32, i32, i64, i32, P, P]
        lib.orc_build_index.restype = ctypes.c_int
        lib.orc_fwd.argtypes = [P, P, P, P, P, i64, i32, i32, i32]
        lib.orc_fwd_rows.argtypes = [P, P, P, P, P, i64, P, i32, i32, i32]
        lib.orc_bwd_dx.argtypes = [P, P, P, P, i64, i32, i32, i32]
        lib.orc_bwd_dx_rows.argtypes = [P, P, P, P, i64, P, i32, i32, i32]
        lib.orc_bwd_dx_scatter.argtypes = [P, P, P, P, i64, i32, i32, i32]
        lib.orc_bwd_dw.argtypes = [P, P, P, P, i64, i32, i32, i32]
        lib.orc_bwd_dw_rows.argtypes = [P, P, P, P, i64, P, i64, i32, i32, i32]
        lib.orc_bwd_db.argtypes = [P, P, i64, i32]
        lib.orc_xattn_fwd.argtypes = [P, P, P, P, i64, i64, i32, ctypes.c_double]
        lib.orc_xattn_bwd.argtypes = [P, P, P, P, P, i64, i64, i32, ctypes.c_double]
        lib.orc_adapter_fwd.argtypes = [P, P, i64, i32, i32, i32, P, P, P, P, P, P, P, P, P]
        lib.orc_adapter_bwd.argtypes = [P, P, i64, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P, P]
        for f in ("orc_fwd", "orc_fwd_rows", "orc_bwd_dx", "orc_bwd_dx_rows",
                  "orc_bwd_dx_scatter", "orc_bwd_dw", "orc_bwd_dw_rows", "orc_bwd_db",
                  "orc_xattn_fwd", "orc_xattn_bwd", "orc_adapter_fwd", "orc_adapter_bwd"):
            getattr(lib, f).restype = None
        self.lib = lib
        self.path = path

    def threads(self, want: int = 0) -> int:
        """Set (want > 0) and return the OpenMP thread count the oracle uses."""
        return int(self.lib.orc_threads(int(want)))

    def build_index(self, coords, frame_offsets, T, H, W, want_map=False, K=3):
        """Returns (status, N [n,K*K] int32, M [T,H,W] int32 or None)."""
        coords = _i32(coords)
        offs = _i32(frame_offsets)
        n = coords.shape[0]
        N = np.full((n, K * K), -7, dtype=np.int32)
        M = np.full((T, H, W), -7, dtype=np.int32) if want_map else None
        st = self.lib.orc_build_index(_p(coords), _p(offs), int(T), int(H), int(W), int(n), int(K),
                                      _p(N), _p(M))
        return int(st), N, M

    def fwd(self, X, N, Wt, b=None):
        X, N, Wt = _f64(X), _i32(N), _f64(Wt)
        n, Ci = X.shape
        Co = Wt.shape[2]
        bb = None if b is None else _f64(b)
        Y = np.empty((n, Co), dtype=np.float64)
        self.lib.orc_fwd(_p(X), _p(N), _p(Wt), _p(bb), _p(Y), n, Ci, Co, _taps(N, Wt))
        return Y

    def fwd_rows(self, X, N, Wt, b, rows):
        X, N, Wt, rows = _f64(X), _i32(N), _f64(Wt), _i64(rows)
        Ci, Co = Wt.shape[1], Wt.shape[2]
        bb = None if b is None else _f64(b)
        out = np.empty((rows.shape[0], Co), dtype=np.float64)
        self.lib.orc_fwd_rows(_p(X), _p(N), _p(Wt), _p(bb), _p(rows), rows.shape[0], _p(out),
                              Ci, Co, _taps(N, Wt))
        return out

    def bwd_dx(self, dY, N, Wt):
        dY, N, Wt = _f64(dY), _i32(N), _f64(Wt)
        n = dY.shape[0]
        Ci, Co = Wt.shape[1], Wt.shape[2]
        dX = np.empty((n, Ci), dtype=np.float64)
        self.lib.orc_bwd_dx(_p(dY), _p(N), _p(Wt), _p(dX), n, Ci, Co, _taps(N, Wt))
        return dX

    def bwd_dx_rows(self, dY, N, Wt, rows):
        dY, N, Wt, rows = _f64(dY), _i32(N), _f64(Wt), _i64(rows)
        Ci, Co = Wt.shape[1], Wt.shape[2]
        out = np.empty((rows.shape[0], Ci), dtype=np.float64)
        self.lib.orc_bwd_dx_rows(_p(dY), _p(N), _p(Wt), _p(rows), rows.shape[0], _p(out), Ci, Co,
                                 _taps(N, Wt))
        return out

    def bwd_dx_scatter(self, dY, N, Wt):
        dY, N, Wt = _f64(dY), _i32(N), _f64(Wt)
        n = dY.shape[0]
        Ci, Co = Wt.shape[1], Wt.shape[2]
        dX = np.empty((n, Ci), dtype=np.float64)
        self.lib.orc_bwd_dx_scatter(_p(dY), _p(N), _p(Wt), _p(dX), n, Ci, Co, _taps(N, Wt))
        return dX

    def bwd_dw(self, X, N, dY):
        X, N, dY = _f64(X), _i32(N), _f64(dY)
        n, Ci = X.shape
        Co = dY.shape[1]
        taps = N.shape[1]
        dW = np.empty((taps, Ci, Co), dtype=np.float64)
        self.lib.orc_bwd_dw(_p(X), _p(N), _p(dY), _p(dW), n, Ci, Co, taps)
        return dW

    def bwd_dw_rows(self, X, N, dY, rows):
        """rows: flat (j * Ci + i) indices; returns [len(rows), Co]."""
        X, N, dY, rows = _f64(X), _i32(N), _f64(dY), _i64(rows)
        n, Ci = X.shape
        Co = dY.shape[1]
        out = np.empty((rows.shape[0], Co), dtype=np.float64)
        self.lib.orc_bwd_dw_rows(_p(X), _p(N), _p(dY), _p(rows), rows.shape[0], _p(out), n, Ci,
                                 Co, N.shape[1])
        return out

    def bwd_db(self, dY):
        dY = _f64(dY)
        n, Co = dY.shape
        db = np.empty((Co,), dtype=np.float64)
        self.lib.orc_bwd_db(_p(dY), _p(db), n, Co)
        return db

    def xattn_fwd(self, Q, X, scale=None):
        """Cross-attention of the queries Q [m,d] over X [n,d] (keys = values).
        Returns (O [m,d], lse [m]).  scale defaults to 1/sqrt(d)."""
        Q, X = _f64(Q), _f64(X)
        m, d = Q.shape
        n = X.shape[0]
        sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
        O = np.empty((m, d), dtype=np.float64)
        lse = np.empty((m,), dtype=np.float64)
        self.lib.orc_xattn_fwd(_p(Q), _p(X.reshape(n, d) if n else np.zeros((1, d))), _p(O), _p(lse),
                               m, n, d, sc)
        return O, lse

    def xattn_bwd(self, Q, X, dO, scale=None):
        """Gradients (dQ [m,d], dX [n,d]) of <O, dO> for O = xattn_fwd(Q, X)."""
        Q, X, dO = _f64(Q), _f64(X), _f64(dO)
        m, d = Q.shape
        n = X.shape[0]
        sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
        dQ = np.empty((m, d), dtype=np.float64)
        dX = np.empty((max(n, 1), d), dtype=np.float64)
        Xp = X.reshape(n, d) if n else np.zeros((1, d))
        self.lib.orc_xattn_bwd(_p(Q), _p(Xp), _p(dO), _p(dQ), _p(dX), m, n, d, sc)
        return dQ, dX[:n]

    def adapter_fwd(self, X, N, Wd, bd, Wc, bc, Wu, bu):
        """Bottleneck adapter: returns (Y [n,C], H1 [n,r], H2 [n,r]) for
        H1 = X Wd + bd, H2 = conv_K(H1; N, Wc) + bc, Y = X + H2 Wu + bu.
        Wd [C,r], Wc [K*K,r,r], Wu [r,C]; biases may be None."""
        X, N, Wd, Wc, Wu = _f64(X), _i32(N), _f64(Wd), _f64(Wc), _f64(Wu)
        n, C = X.shape
        r = Wd.shape[1]
        assert Wd.shape == (C, r) and Wc.shape == (N.shape[1], r, r) and Wu.shape == (r, C)
        bd, bc, bu = (None if v is None else _f64(v) for v in (bd, bc, bu))
        H1 = np.empty((n, r), dtype=np.float64)
        H2 = np.empty((n, r), dtype=np.float64)
        Y = np.empty((n, C), dtype=np.float64)
        self.lib.orc_adapter_fwd(_p(X), _p(N), n, N.shape[1], C, r, _p(Wd), _p(bd), _p(Wc), _p(bc), _p(Wu),
                                 _p(bu), _p(H1), _p(H2), _p(Y))
        return Y, H1, H2

    def adapter_bwd(self, X, N, Wd, bd, Wc, bc, Wu, dY):
        """Gradients of <Y, dY> for Y = adapter_fwd(...): a dict with dX,
        dWd, dbd, dWc, dbc, dWu, dbu."""
        X, N, Wd, Wc, Wu, dY = _f64(X), _i32(N), _f64(Wd), _f64(Wc), _f64(Wu), _f64(dY)
        n, C = X.shape
        r = Wd.shape[1]
        taps = N.shape[1]
        assert Wd.shape == (C, r) and Wc.shape == (taps, r, r) and Wu.shape == (r, C) and dY.shape == (n, C)
        bd, bc = (None if v is None else _f64(v) for v in (bd, bc))
        g = {"dX": np.empty((n, C)), "dWd": np.empty((C, r)), "dbd": np.empty(r), "dWc": np.empty((taps, r, r)),
             "dbc": np.empty(r), "dWu": np.empty((r, C)), "dbu": np.empty(C)}
        self.lib.orc_adapter_bwd(_p(X), _p(N), n, taps, C, r, _p(Wd), _p(bd), _p(Wc), _p(bc), _p(Wu), _p(dY),
                                 *(_p(g[k]) for k in ("dX", "dWd", "dbd", "dWc", "dbc", "dWu", "dbu")))
        return g


def _taps(N, Wt):
    """Number of taps of a call: the columns of N, which must match the
    weights' first dimension."""
    assert N.ndim == 2 and Wt.shape[0] == N.shape[1], (N.shape, Wt.shape)
    return int(N.shape[1])


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _p(a):
    return None if a is None else a.ctypes.data


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c as committed."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _default = Oracle(_LIB)
    return _default


def threads(want: int = 0) -> int:
    return default().threads(want)


def build_index(coords, frame_offsets, T, H, W, want_map=False, K=3):
    return default().build_index(coords, frame_offsets, T, H, W, want_map, K)


def fwd(X, N, Wt, b=None):
    return default().fwd(X, N, Wt, b)


def fwd_rows(X, N, Wt, b, rows):
    return default().fwd_rows(X, N, Wt, b, rows)


def bwd_dx(dY, N, Wt):
    return default().bwd_dx(dY, N, Wt)


def bwd_dx_rows(dY, N, Wt, rows):
    return default().bwd_dx_rows(dY, N, Wt, rows)


def bwd_dx_scatter(dY, N, Wt):
    return default().bwd_dx_scatter(dY, N, Wt)


def bwd_dw(X, N, dY):
    return default().bwd_dw(X, N, dY)


def bwd_dw_rows(X, N, dY, rows):
    return default().bwd_dw_rows(X, N, dY, rows)


def bwd_db(dY):
    return default().bwd_db(dY)


def adapter_fwd(X, N, Wd, bd, Wc, bc, Wu, bu):
    return default().adapter_fwd(X, N, Wd, bd, Wc, bc, Wu, bu)


def adapter_bwd(X, N, Wd, bd, Wc, bc, Wu, dY):
    return default().adapter_bwd(X, N, Wd, bd, Wc, bc, Wu, dY)


def xattn_fwd(Q, X, scale=None):
    return default().xattn_fwd(Q, X, scale)


def xattn_bwd(Q, X, dO, scale=None):
    return default().xattn_bwd(Q, X, dO, scale)
