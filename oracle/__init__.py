"""CPU oracle for the Stream-K GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``work_centric_decomposition_amd``) and never imports it.

Contents (each function cites the passage it follows):

* :func:`gemm` -- C = alpha*A*B + beta*C_in by the sequential cache-blocked
  six-loop GEMM (Stream-K page, section 3.1, Algorithm 1), fp64 accumulate,
  exact decode of the inputs, one round-to-nearest-even to the output type,
  and the componentwise bound D = |alpha||A||B| + |beta||C_in|.
* :func:`gemm_entries` -- the same definition for selected (i, j) only.
* :func:`sk_plan` / :func:`sk_execute` -- the page's decompositions
  (Algorithms 2, 4, 5 and the two hybrids of section 5.2) as per-CTA segment
  lists, and their simulated execution with host partials/flags.
* :func:`abft_check` -- one ABFT verification domain (fault-tolerant GEMM
  page, Fig. 3 and the threadblock-level scheme of Figs. 5-7).
* :func:`freivalds` -- randomised product check (textbook identity).
* :func:`quantization_efficiency` -- processor utilisation of a schedule
  (Stream-K page, section 1, Figs. 1-2).

Function with no independent pin: none (every function is pinned by a test
in ``tests/test_oracle_*.py``; the grid-size model is not part of the oracle).
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libskoracle.so")

# dtype and layout codes (numerically equal to the public ABI's values)
F32, F16, BF16 = 0, 1, 2
A_ROW_B_ROW, A_ROW_B_COL, A_COL_B_ROW, A_COL_B_COL = 0, 1, 2, 3
# decomposition modes
DP, FIXED, SK, HYBRID1, HYBRID2, DP_PERSISTENT = 0, 1, 2, 3, 4, 5

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        i64, f64, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        L.or_gemm.argtypes = [i64, i64, i64, f64, vp, i64, vp, i64, f64, vp, i64, ci, ci,
                              i64, i64, i64, vp, vp, vp, ci]
        L.or_gemm.restype = ci
        L.or_gemm_entries.argtypes = [i64, i64, i64, f64, vp, i64, vp, i64, f64, vp, i64, ci, ci,
                                      i64, vp, vp, vp, vp, ci]
        L.or_gemm_entries.restype = ci
        L.or_sk_plan.argtypes = [i64, i64, i64, i64, i64, i64, ci, i64, vp, i64, vp]
        L.or_sk_plan.restype = i64
        L.or_sk_execute.argtypes = [i64, i64, i64, f64, vp, i64, vp, i64, f64, vp, i64, ci, ci,
                                    i64, i64, i64, ci, i64, ctypes.c_uint64, ci, vp, vp]
        L.or_sk_execute.restype = ci
        L.or_abft_check.argtypes = [i64, i64, i64, vp, vp, vp, f64, vp, vp, vp]
        L.or_abft_check.restype = ci
        L.or_freivalds.argtypes = [i64, i64, i64, f64, vp, i64, vp, i64, f64, vp, i64, vp, i64,
                                   ci, ci, i64, vp, vp, ci]
        L.or_freivalds.restype = ci
        L.or_decode_f16.argtypes = [ctypes.c_uint16]
        L.or_decode_f16.restype = f64
        L.or_decode_bf16.argtypes = [ctypes.c_uint16]
        L.or_decode_bf16.restype = f64
        L.or_round_f16.argtypes = [f64]
        L.or_round_f16.restype = ctypes.c_uint16
        L.or_round_bf16.argtypes = [f64]
        L.or_round_bf16.restype = ctypes.c_uint16
        L.or_num_threads.argtypes = []
        L.or_num_threads.restype = ci
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _storage(x: np.ndarray, dtype: int) -> np.ndarray:
    """The raw storage array the oracle reads: float32 or 16-bit patterns."""
    if dtype == F32:
        assert x.dtype == np.float32
    else:
        assert x.dtype in (np.uint16, np.float16), x.dtype
    return np.ascontiguousarray(x)


def num_threads() -> int:
    return int(lib().or_num_threads())


def decode_f16(bits: int) -> float:
    return float(lib().or_decode_f16(bits))


def decode_bf16(bits: int) -> float:
    return float(lib().or_decode_bf16(bits))


def round_f16(x: float) -> int:
    return int(lib().or_round_f16(x))


def round_bf16(x: float) -> int:
    return int(lib().or_round_bf16(x))


def gemm(m, n, k, alpha, A, lda, B, ldb, beta, Cin, ldc, dtype, layout,
         blk=(64, 64, 64), nthreads=0, want_round=True):
    """Algorithm 1 (Stream-K page, section 3.1) in fp64.

    A, B, Cin are flat storage arrays (float32, or uint16 bit patterns for
    fp16/bf16) addressed with the given leading dimensions and layout.
    Returns (out64 [m, n] float64, bound [m, n] float64, rounded [m, n] in the
    storage type or None).
    """
    A = _storage(A, dtype)
    B = _storage(B, dtype)
    Cin = None if Cin is None else _storage(Cin, dtype)
    out64 = np.empty((m, n), np.float64)
    bound = np.empty((m, n), np.float64)
    rnd = None
    if want_round:
        rnd = np.empty((m, n), np.float32 if dtype == F32 else np.uint16)
    rc = lib().or_gemm(m, n, k, alpha, _ptr(A), lda, _ptr(B), ldb, beta, _ptr(Cin), ldc,
                       dtype, layout, blk[0], blk[1], blk[2], _ptr(out64), _ptr(bound),
                       _ptr(rnd), nthreads)
    if rc != 0:
        raise RuntimeError(f"or_gemm failed ({rc})")
    return out64, bound, rnd


def gemm_entries(m, n, k, alpha, A, lda, B, ldb, beta, Cin, ldc, dtype, layout, rows, cols,
                 nthreads=0):
    """Selected entries of the same definition (plain dot products, k ascending)."""
    A = _storage(A, dtype)
    B = _storage(B, dtype)
    Cin = None if Cin is None else _storage(Cin, dtype)
    rows = np.ascontiguousarray(rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    out = np.empty(rows.shape[0], np.float64)
    bound = np.empty(rows.shape[0], np.float64)
    rc = lib().or_gemm_entries(m, n, k, alpha, _ptr(A), lda, _ptr(B), ldb, beta, _ptr(Cin),
                               ldc, dtype, layout, rows.shape[0], _ptr(rows), _ptr(cols),
                               _ptr(out), _ptr(bound), nthreads)
    if rc != 0:
        raise RuntimeError(f"or_gemm_entries failed ({rc})")
    return out, bound


PLAN_FIELDS = ("cta", "tile", "lb", "le", "started", "ended", "last_peer")


def sk_plan(m, n, k, bm, bn, bk, mode, param):
    """Per-CTA segment lists of a decomposition (Stream-K page, Algorithms 2,
    4, 5 and section 5.2).  Returns (records [N, 7] int64, n_cta)."""
    t = -(-m // bm) * -(-n // bn)
    cap = 8 * (t + 4) + 4 * (max(param, t) + 4) * 2 + 16
    while True:
        rec = np.empty((cap, 7), np.int64)
        ncta = ctypes.c_int64(0)
        c = lib().or_sk_plan(m, n, k, bm, bn, bk, mode, param, _ptr(rec), cap,
                             ctypes.byref(ncta))
        if c == -3:
            cap *= 4
            continue
        if c == -2:
            raise ValueError("decomposition not defined for this shape")
        if c < 0:
            raise RuntimeError(f"or_sk_plan failed ({c})")
        return rec[:c].copy(), int(ncta.value)


def sk_execute(m, n, k, alpha, A, lda, B, ldb, beta, Cin, ldc, dtype, layout, bm, bn, bk,
               mode, param, seed=0, policy=0):
    """Simulated execution of a decomposition with host partials and flags.

    Returns (out64 [m, n], n_yields)."""
    A = _storage(A, dtype)
    B = _storage(B, dtype)
    Cin = None if Cin is None else _storage(Cin, dtype)
    out = np.full((m, n), np.nan, np.float64)
    ny = ctypes.c_int64(0)
    rc = lib().or_sk_execute(m, n, k, alpha, _ptr(A), lda, _ptr(B), ldb, beta, _ptr(Cin), ldc,
                             dtype, layout, bm, bn, bk, mode, param, seed, policy, _ptr(out),
                             ctypes.byref(ny))
    if rc == -4:
        raise RuntimeError("simulated schedule deadlocked")
    if rc != 0:
        raise RuntimeError(f"or_sk_execute failed ({rc})")
    return out, int(ny.value)


def abft_check(A_blk: np.ndarray, B_blk: np.ndarray, C_blk: np.ndarray, c_tau: float = 1.0):
    """One ABFT verification domain.  C_blk (float32) is corrected in place.

    Returns (status, (i, j, delta) or None): status 0 clean, 1 corrected,
    2 mismatch not locatable to one element."""
    A_blk = np.ascontiguousarray(A_blk, np.float64)
    B_blk = np.ascontiguousarray(B_blk, np.float64)
    assert C_blk.dtype == np.float32 and C_blk.flags["C_CONTIGUOUS"]
    rows, kk = A_blk.shape
    kk2, cols = B_blk.shape
    assert kk == kk2 and C_blk.shape == (rows, cols)
    fi, fj, fd = ctypes.c_int64(-1), ctypes.c_int64(-1), ctypes.c_double(0)
    st = lib().or_abft_check(rows, cols, kk, _ptr(A_blk), _ptr(B_blk), _ptr(C_blk), c_tau,
                             ctypes.byref(fi), ctypes.byref(fj), ctypes.byref(fd))
    if st < 0:
        raise RuntimeError("or_abft_check failed")
    return st, ((fi.value, fj.value, fd.value) if st == 1 else None)


def freivalds(m, n, k, alpha, A, lda, B, ldb, beta, Cin, ldc, Cout, ldo, dtype, layout,
              X: np.ndarray, nthreads=0) -> float:
    """Largest normalised residual of C_out x against alpha A (B x) + beta C_in x
    over the rows of X (each a length-n vector)."""
    A = _storage(A, dtype)
    B = _storage(B, dtype)
    Cin = None if Cin is None else _storage(Cin, dtype)
    Cout = _storage(Cout, dtype)
    X = np.ascontiguousarray(X, np.float64)
    assert X.shape[1] == n
    w = ctypes.c_double(0)
    rc = lib().or_freivalds(m, n, k, alpha, _ptr(A), lda, _ptr(B), ldb, beta, _ptr(Cin), ldc,
                            _ptr(Cout), ldo, dtype, layout, X.shape[0], _ptr(X),
                            ctypes.byref(w), nthreads)
    if rc != 0:
        raise RuntimeError("or_freivalds failed")
    return float(w.value)


def quantization_efficiency(cta_work: Sequence[float], p: int) -> float:
    """Processor utilisation of a grid of CTAs on p SMs (Stream-K page,
    section 1, Figs. 1-2): CTAs are dispatched in order to whichever SM is
    free first; utilisation = total work / (p * makespan)."""
    free_at = [0.0] * p
    for w in cta_work:
        s = min(range(p), key=lambda i: free_at[i])
        free_at[s] += w
    makespan = max(free_at)
    total = float(sum(cta_work))
    return total / (p * makespan) if makespan > 0 else 1.0


def plan_cta_work(records: np.ndarray, n_cta: int):
    """MAC iterations per CTA from plan records."""
    work = [0] * n_cta
    for r in records:
        work[int(r[0])] += int(r[3] - r[2])
    return work
