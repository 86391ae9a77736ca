"""ctypes binding of the plain fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg
may use it; the GPU library never does.  Inputs are the raw bfloat16 bit patterns (uint16
numpy arrays) produced by ``workloads``; results are float64 arrays of the exact-product,
fp64-summed values, with separate rounding helpers to float32 and bfloat16.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

B_KN, B_NK = 0, 1
EPI_NONE, EPI_BIAS, EPI_SILU, EPI_BIAS_SILU = 0, 1, 2, 3
_STATUS = {0: "ok", 1: "bad argument", 2: "bad group offsets", 3: "bad user index", 4: "out of memory"}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle: {_STATUS.get(code, code)}")
        self.code = code


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no HIP involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        p, i64, i32, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        L.oracle_gemm.argtypes = [i64, i64, i64, p, i64, p, i64, i, p, i, p, i64, p]
        L.oracle_grouped_gemm.argtypes = [i32, i64, i64, i64, p, p, i, p, p, i, p, i64, p]
        L.oracle_broadcast_gemm.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, i, p, i, p, i64, p]
        L.oracle_grouped_wgrad.argtypes = [i32, i64, i64, i64, p, p, p, p, i64, p]
        L.oracle_ikbo_attention.argtypes = [i64, i64, i64, i64, i64, ctypes.c_double, p, p, p, p, p, i64, p]
        for f in (L.oracle_gemm, L.oracle_grouped_gemm, L.oracle_broadcast_gemm, L.oracle_grouped_wgrad,
                  L.oracle_ikbo_attention):
            f.restype = ctypes.c_int
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_round_bf16.argtypes = [ctypes.c_double]
        L.oracle_round_bf16.restype = ctypes.c_uint16
        L.oracle_round_bf16_array.argtypes = [p, i64, p]
        L.oracle_round_f32_array.argtypes = [p, i64, p]
        L.oracle_set_threads.argtypes = [i]
        L.oracle_max_threads.restype = i
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _rows(rows, n_all):
    if rows is None:
        return None, n_all
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, len(r)


def _check(code: int):
    if code != 0:
        raise OracleError(code)


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def silu(v: float) -> float:
    return float(lib().oracle_silu(float(v)))


def round_bf16(v) -> np.ndarray:
    """Nearest bfloat16 (ties to even) of each double, rounded in one step; uint16 bits."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_round_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def round_f32(v) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.float32)
    lib().oracle_round_f32_array(_ptr(v), v.size, _ptr(out))
    return out


def gemm(A, B, b_layout: int, bias=None, epi: int = EPI_NONE, rows=None) -> np.ndarray:
    """v[t, j] = epi(sum_k A[r, k] B(k, j) + bias[j]) for r = rows[t] (all rows by default)."""
    A, B = _u16(A), _u16(B)
    M, K = A.shape
    N = B.shape[1] if b_layout == B_KN else B.shape[0]
    assert (B.shape[0] if b_layout == B_KN else B.shape[1]) == K
    ldb = B.shape[1]
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    r, n = _rows(rows, M)
    out = np.empty((n, N), dtype=np.float64)
    _check(lib().oracle_gemm(M, N, K, _ptr(A), K, _ptr(B), ldb, b_layout, _ptr(bias), epi,
                             _ptr(r), n, _ptr(out)))
    return out


def grouped_gemm(X, W, w_layout: int, offsets, bias=None, epi: int = EPI_NONE,
                 rows=None) -> np.ndarray:
    """Group g (rows offsets[g] .. offsets[g+1]-1) multiplies W[g]; returns float64 rows."""
    X, W = _u16(X), _u16(W)
    M_total, K = X.shape
    G = W.shape[0]
    N = W.shape[2] if w_layout == B_KN else W.shape[1]
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int32))
    assert off.shape == (G + 1,)
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    r, n = _rows(rows, M_total)
    out = np.empty((n, N), dtype=np.float64)
    _check(lib().oracle_grouped_gemm(G, M_total, N, K, _ptr(X), _ptr(W), w_layout, _ptr(off),
                                     _ptr(bias), epi, _ptr(r), n, _ptr(out)))
    return out


def broadcast_gemm(Xu, Xc, idx, W, w_layout: int, bias=None, epi: int = EPI_NONE,
                   rows=None) -> np.ndarray:
    """Y[r] = epi([Xu[idx[r]] | Xc[r]] . W + bias), the broadcast materialised row by row."""
    Xu, Xc, W = _u16(Xu), _u16(Xc), _u16(W)
    U, Ku = Xu.shape
    Mc, Kc = Xc.shape
    N = W.shape[1] if w_layout == B_KN else W.shape[0]
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    assert idx.shape == (Mc,)
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    r, n = _rows(rows, Mc)
    out = np.empty((n, N), dtype=np.float64)
    _check(lib().oracle_broadcast_gemm(U, Mc, Ku, Kc, N, _ptr(Xu), _ptr(Xc), _ptr(idx), _ptr(W),
                                       w_layout, _ptr(bias), epi, _ptr(r), n, _ptr(out)))
    return out


def grouped_wgrad(X, dY, offsets, rows=None) -> np.ndarray:
    """Weight gradient of the grouped GEMM: dW[g] = X_g^T . dY_g over group g's rows
    (offsets[g] .. offsets[g+1]-1), zero for an empty group.  Returns float64 rows of dW
    flattened to (G * K, N); `rows` selects flat row indices g * K + i."""
    X, dY = _u16(X), _u16(dY)
    M_total, K = X.shape
    assert dY.shape[0] == M_total
    N = dY.shape[1]
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int32))
    G = off.shape[0] - 1
    r, n = _rows(rows, G * K)
    out = np.empty((n, N), dtype=np.float64)
    _check(lib().oracle_grouped_wgrad(G, M_total, K, N, _ptr(X), _ptr(dY), _ptr(off), _ptr(r), n,
                                      _ptr(out)))
    return out


def ikbo_attention(Q, K, V, offsets, scale: float, rows=None) -> np.ndarray:
    """Attention of every candidate's query over its user's keys and values: Q [Mc, H, D],
    K and V [U, L, H, D] (uint16 bfloat16 bits), offsets [U + 1] (candidates contiguous by user).
    Returns float64 [nrows, H, D] for the selected candidate rows (all by default)."""
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    Mc, H, D = Q.shape
    U, L = K.shape[0], K.shape[1]
    assert K.shape == (U, L, H, D) and V.shape == K.shape
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int32))
    assert off.shape == (U + 1,)
    r, n = _rows(rows, Mc)
    out = np.empty((n, H, D), dtype=np.float64)
    _check(lib().oracle_ikbo_attention(U, Mc, H, D, L, float(scale), _ptr(off), _ptr(Q), _ptr(K), _ptr(V),
                                       _ptr(r), n, _ptr(out)))
    return out


def problem_list(problems: Sequence, epi: int, rows_per_problem=None):
    """One plain gemm per problem (every B_p stored K x N); returns a list of float64 arrays."""
    outs = []
    for i, p in enumerate(problems):
        rows = None if rows_per_problem is None else rows_per_problem[i]
        outs.append(gemm(p.A, p.B, B_KN, p.bias, epi, rows))
    return outs
