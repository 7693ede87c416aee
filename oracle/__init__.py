"""Python handle on the CPU oracle (``serac_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The matching
library never does; it shares no code with the oracle.

``build()`` compiles ``serac_oracle.c`` with gcc (-O2, OpenMP, no fast-math,
no FMA contraction) into ``liboracle.so`` beside it; the functions below load
that library and marshal NumPy arrays.  Every function follows the plain
definition spelled out in the C file's header (the SERAC README, sections
"What changed" and "Exactness").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "serac_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build(src: str = SRC, out: str = LIB, extra: tuple = ()) -> str:
    """Compile the oracle (always); returns the library path."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path: str = LIB) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    i32p = ctypes.POINTER(ctypes.c_int32)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    i32 = ctypes.c_int32
    lib.oracle_top2.argtypes = [u8p, i32, u8p, i32, i32p, i32p, ctypes.c_int]
    lib.oracle_rows.argtypes = [u8p, i32, u8p, i32, i32p, i32, i32p, ctypes.c_int]
    lib.oracle_cols.argtypes = [u8p, i32, u8p, i32, i32p, i32, i32p, ctypes.c_int]
    lib.oracle_angle.argtypes = [i32]
    lib.oracle_angle.restype = ctypes.c_double
    lib.oracle_accept.argtypes = [i32, i32, i32, i32, i32, ctypes.c_double,
                                  ctypes.c_double, i32]
    lib.oracle_match_pair.argtypes = [u8p, i32, u8p, i32, ctypes.c_double,
                                      ctypes.c_double, i32, u32p, i32p,
                                      ctypes.c_int]
    lib.oracle_match_pair_sym.argtypes = [u8p, i32, u8p, i32, ctypes.c_double,
                                          ctypes.c_double, u32p, i32p, ctypes.c_int]
    lib.oracle_max_threads.argtypes = []
    for f in (lib.oracle_top2, lib.oracle_rows, lib.oracle_cols,
              lib.oracle_accept, lib.oracle_match_pair, lib.oracle_match_pair_sym,
              lib.oracle_max_threads):
        f.restype = ctypes.c_int
    return lib


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = load()
    return _lib


def _u8(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint8)
    if x.ndim != 2 or x.shape[1] != 128:
        raise ValueError("descriptors must be [n, 128] uint8")
    return x


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(ctypes.POINTER(t))


def max_threads() -> int:
    return lib().oracle_max_threads()


def top2(A, B, nthreads: int = 0, L=None):
    """(row_top2 int32 [nA, 3] = best, idx, second; col_best int32 [nB, 2])."""
    L = L or lib()
    A, B = _u8(A), _u8(B)
    row = np.zeros((A.shape[0], 3), dtype=np.int32)
    col = np.zeros((B.shape[0], 2), dtype=np.int32)
    rc = L.oracle_top2(_p(A, ctypes.c_uint8), A.shape[0], _p(B, ctypes.c_uint8),
                       B.shape[0], _p(row, ctypes.c_int32),
                       _p(col, ctypes.c_int32), nthreads)
    if rc:
        raise RuntimeError("oracle_top2 failed")
    return row, col


def rows(A, B, idx, nthreads: int = 0, L=None):
    """Row top-2 for the rows listed in idx (int32 [len(idx), 3])."""
    L = L or lib()
    A, B = _u8(A), _u8(B)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    out = np.zeros((len(idx), 3), dtype=np.int32)
    rc = L.oracle_rows(_p(A, ctypes.c_uint8), A.shape[0], _p(B, ctypes.c_uint8),
                       B.shape[0], _p(idx, ctypes.c_int32), len(idx),
                       _p(out, ctypes.c_int32), nthreads)
    if rc:
        raise RuntimeError("oracle_rows failed")
    return out


def cols(A, B, idx, nthreads: int = 0, L=None):
    """Column best for the columns listed in idx (int32 [len(idx), 2])."""
    L = L or lib()
    A, B = _u8(A), _u8(B)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    out = np.zeros((len(idx), 2), dtype=np.int32)
    rc = L.oracle_cols(_p(A, ctypes.c_uint8), A.shape[0], _p(B, ctypes.c_uint8),
                       B.shape[0], _p(idx, ctypes.c_int32), len(idx),
                       _p(out, ctypes.c_int32), nthreads)
    if rc:
        raise RuntimeError("oracle_cols failed")
    return out


def angle(s: int, L=None) -> float:
    return (L or lib()).oracle_angle(int(s))


def accept(i, best, idx, second, colidx_of_best, max_ratio=0.8,
           max_distance=float("inf"), cross_check=True, L=None) -> bool:
    return bool((L or lib()).oracle_accept(int(i), int(best), int(idx),
                                          int(second), int(colidx_of_best),
                                          float(max_ratio), float(max_distance),
                                          int(bool(cross_check))))


def cap(X, max_features: int = 0) -> np.ndarray:
    """The match cap: only the first max_features descriptors of an image
    take part (0: no cap).  The SERAC README ("Memory") describes lowering
    COLMAP's cap as clamping the lower-scale features away, i.e. features
    are kept in their stored order, largest scale first, up to the cap."""
    if max_features < 0:
        raise ValueError("max_features must be >= 0")
    return X[:max_features] if max_features else X


def match_pair(A, B, max_ratio=0.8, max_distance=float("inf"),
               cross_check=True, nthreads: int = 0, L=None, symmetric=False,
               max_features: int = 0) -> np.ndarray:
    """Accepted correspondences, uint32 [count, 2] = (row of A, row of B).

    symmetric: the column side passes the same gates (serac_oracle.c,
    "symmetric"); it implies the cross-check.  max_features: the match cap
    (see cap())."""
    L = L or lib()
    A, B = _u8(cap(A, max_features)), _u8(cap(B, max_features))
    out = np.zeros((max(A.shape[0], 1), 2), dtype=np.uint32)
    cnt = ctypes.c_int32(0)
    if symmetric:
        rc = L.oracle_match_pair_sym(_p(A, ctypes.c_uint8), A.shape[0],
                                     _p(B, ctypes.c_uint8), B.shape[0],
                                     float(max_ratio), float(max_distance),
                                     _p(out, ctypes.c_uint32), ctypes.byref(cnt), nthreads)
    else:
        rc = L.oracle_match_pair(_p(A, ctypes.c_uint8), A.shape[0],
                                 _p(B, ctypes.c_uint8), B.shape[0],
                                 float(max_ratio), float(max_distance),
                                 int(bool(cross_check)), _p(out, ctypes.c_uint32),
                                 ctypes.byref(cnt), nthreads)
    if rc:
        raise RuntimeError("oracle_match_pair failed")
    return out[:cnt.value].copy()


def match_rows(A, B, sample, max_ratio=0.8, max_distance=float("inf"),
               cross_check=True, nthreads: int = 0, L=None) -> dict:
    """The accept decision for a sample of rows, computed one by one.

    For each sampled row: its full row top-2, then (if cross-checking) the
    best row of its best column.  Returns {row: idx or -1 (rejected)}.
    """
    L = L or lib()
    sample = np.ascontiguousarray(sample, dtype=np.int32)
    r3 = rows(A, B, sample, nthreads, L)
    need = np.unique(r3[:, 1][r3[:, 1] >= 0]).astype(np.int32)
    cb = cols(A, B, need, nthreads, L) if (cross_check and len(need)) else \
        np.zeros((0, 2), dtype=np.int32)
    cidx = {int(j): int(c[1]) for j, c in zip(need, cb)}
    out = {}
    for i, (best, idx, second) in zip(sample, r3):
        ok = accept(i, best, idx, second, cidx.get(int(idx), -1), max_ratio,
                    max_distance, cross_check, L)
        out[int(i)] = int(idx) if ok else -1
    return out
