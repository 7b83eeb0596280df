"""Helpers for the GPU parity tests: seeded inputs, upload through torch, one
call through the C ABI, and the comparison with the oracle.

Error metric: max over elements of |C_gpu - C_ref| / D, where C_ref is the
oracle's unrounded fp64 value and D = |alpha| |A||B| + |beta| |C_in| is the
componentwise bound (elements with D == 0 must match exactly).  The one
rounding of the result to the output format is allowed its absolute floor:
below the smallest normal number the format's spacing is fixed (fp16:
2^-24), so a correctly rounded subnormal result may be off by half of it
whatever its size; that much is taken off |C_gpu - C_ref| first.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sk_synth as S
import work_centric_decomposition_amd as sk

TOL = {sk.F32: 1e-5, sk.F16: 5e-3, sk.BF16: 5e-3}
TORCH_DT = {sk.F32: torch.float32, sk.F16: torch.float16, sk.BF16: torch.bfloat16}


def orders(layout):
    a = "row" if layout in (sk.A_ROW_B_ROW, sk.A_ROW_B_COL) else "col"
    b = "row" if layout in (sk.A_ROW_B_ROW, sk.A_COL_B_ROW) else "col"
    return a, b


def to_dev(arr: np.ndarray, dtype: int) -> torch.Tensor:
    if dtype == sk.F32:
        return torch.from_numpy(np.ascontiguousarray(arr)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
    return t.view(TORCH_DT[dtype]).cuda()


def from_dev(t: torch.Tensor, dtype: int) -> np.ndarray:
    if dtype == sk.F32:
        return t.cpu().numpy()
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def decode(arr: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == sk.F32:
        return arr.astype(np.float64)
    if dtype == sk.F16:
        return arr.view(np.float16).astype(np.float64)
    return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Case:
    """Seeded inputs of one GEMM, on the host (storage arrays) and device."""

    def __init__(self, m, n, k, dtype, layout, seed, dist="uniform", scale=1.0, pad=0,
                 with_c=True):
        self.m, self.n, self.k, self.dtype, self.layout = m, n, k, dtype, layout
        ao, bo = orders(layout)
        self.lda = max(1, (k if ao == "row" else m) + pad)
        self.ldb = max(1, (n if bo == "row" else k) + pad)
        self.ldc = max(1, n + pad)
        self.A = S.matrix(seed, S.STREAM_A, m, k, dtype, dist, ao, self.lda, scale)
        self.B = S.matrix(seed, S.STREAM_B, k, n, dtype, dist, bo, self.ldb, scale)
        if with_c:
            self.Cin = S.matrix(seed, S.STREAM_C, m, n, dtype, dist, "row", self.ldc, scale)
        else:  # beta = 0 cases: C_in is never read, a zero buffer is enough
            size = (m - 1) * self.ldc + n if m > 0 and n > 0 else 0
            self.Cin = np.zeros(size, np.float32 if dtype == sk.F32 else np.uint16)
        # device buffers sized to the storage (at least one element)
        self.dA = to_dev(self.A if self.A.size else np.zeros(1, self.A.dtype), dtype)
        self.dB = to_dev(self.B if self.B.size else np.zeros(1, self.B.dtype), dtype)
        self.dC = to_dev(self.Cin if self.Cin.size else np.zeros(1, self.Cin.dtype), dtype)

    def reset_c(self):
        self.dC.copy_(to_dev(self.Cin if self.Cin.size else np.zeros(1, self.Cin.dtype),
                             self.dtype))

    def desc(self, alpha=1.0, beta=0.0):
        return sk.make_desc(self.m, self.n, self.k, alpha, self.dA, self.lda, self.dB, self.ldb, beta,
                            self.dC, self.ldc, self.dtype, self.layout)

    def run(self, alpha=1.0, beta=0.0, opts=None, report=None):
        d = self.desc(alpha, beta)
        if opts is None and report is None:
            sk.gemm(self.m, self.n, self.k, alpha, self.dA, self.lda, self.dB, self.ldb, beta,
                    self.dC, self.ldc, self.dtype, self.layout)
        else:
            sk.gemm_ex(d, opts, report)
        torch.cuda.synchronize()
        return self.result()

    def result(self) -> np.ndarray:
        """C as an (m, n) storage array."""
        flat = from_dev(self.dC, self.dtype)
        if self.m == 0 or self.n == 0:
            return flat[:0].reshape(self.m, self.n)
        view = np.lib.stride_tricks.as_strided(flat, shape=(self.m, self.n),
                                               strides=(self.ldc * flat.itemsize, flat.itemsize))
        return view.copy()

    def reference(self, alpha=1.0, beta=0.0):
        out64, bound, _ = oracle.gemm(self.m, self.n, self.k, alpha, self.A, self.lda, self.B,
                                      self.ldb, beta, self.Cin, self.ldc, self.dtype, self.layout,
                                      want_round=False)
        return out64, bound

    def reference_entries(self, rows, cols, alpha=1.0, beta=0.0):
        return oracle.gemm_entries(self.m, self.n, self.k, alpha, self.A, self.lda, self.B,
                                   self.ldb, beta, self.Cin, self.ldc, self.dtype, self.layout,
                                   rows, cols)

    def freivalds(self, C_out: np.ndarray, alpha=1.0, beta=0.0, seed=99, nvec=2) -> float:
        X = np.stack([S.signs(seed, v, self.n) for v in range(nvec)])
        return oracle.freivalds(self.m, self.n, self.k, alpha, self.A, self.lda, self.B, self.ldb,
                                beta, self.Cin, self.ldc, np.ascontiguousarray(C_out), self.n,
                                self.dtype, self.layout, X)


# half the spacing of each output format's subnormal numbers
SUBNORMAL_HALF_ULP = {sk.F32: 2.0 ** -150, sk.F16: 2.0 ** -25, sk.BF16: 2.0 ** -134}


def rel_err(got: np.ndarray, dtype: int, ref64: np.ndarray, bound: np.ndarray) -> float:
    g = decode(got, dtype)
    diff = np.maximum(np.abs(g - ref64) - SUBNORMAL_HALF_ULP[dtype], 0.0)
    zero = bound == 0
    if np.any(zero & (diff != 0)) or np.any(~np.isfinite(g)):
        return float("inf")
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(zero, 0.0, diff / np.where(zero, 1.0, bound))
    return float(r.max()) if r.size else 0.0


def sample_indices(m, n, count, seed):
    u = S.u64(seed, 555, 0, 2 * count)
    rows = (u[:count] % np.uint64(m)).astype(np.int64)
    cols = (u[count:] % np.uint64(n)).astype(np.int64)
    # always include the corners and the last tile's edge
    rows = np.concatenate([rows, [0, 0, m - 1, m - 1]])
    cols = np.concatenate([cols, [0, n - 1, 0, n - 1]])
    return rows, cols


# ------------------------------------------------- per-tile sampling
#
# Freivalds' check (C x against A (B x) for random sign vectors x) cannot
# gate fp16/bf16 results element by element: its bound normalises each row
# by sum_j D_ij |x_j| over all n columns, so an error as large as D_ij in
# every element of one 256-wide tile moves the ratio by about sqrt(256)/n
# (2e-3 at n = 8192), under the 5e-3 tolerance.  The parity tests therefore
# compare sampled entries with the oracle entry by entry, sampled so that
# every output tile is seen, and keep Freivalds only as a supplement.

def split_tiles(plan) -> np.ndarray:
    """Linear indices (in the plan's tile size) of the tiles whose k range
    is split over more than one workgroup under `plan`."""
    out = set()
    for wg in range(plan.grid):
        for (tile, _b, _e, started, ended, _lp) in sk.plan_segments(plan, wg):
            if not (started and ended):
                out.add(int(tile))
    return np.array(sorted(out), dtype=np.int64)


def tile_sample_indices(m, n, seed, tile=128, extra=2, split=None, split_tm=256, split_tn=256,
                        tiles_n=None):
    """Entries of an m x n output such that every `tile` x `tile` output
    tile (128 refines both fp16/bf16 instances' tiles and the fp32 tile) is
    checked at its first and its last row (each at a seeded column of the
    tile), its first and last column (each at a seeded row), and at `extra`
    seeded entries.  Every tile listed in `split` (linear indices of
    split_tm x split_tn tiles, row-major over tiles_n tile columns: the
    tiles a schedule splits over workgroups) is also checked at a seeded
    permutation that meets each of its rows and each of its columns once.
    Returns (rows, cols) without duplicates."""
    if m == 0 or n == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    tm, tn = -(-m // tile), -(-n // tile)
    ti = np.repeat(np.arange(tm, dtype=np.int64), tn)
    tj = np.tile(np.arange(tn, dtype=np.int64), tm)
    r0, c0 = ti * tile, tj * tile
    h = np.minimum(m - r0, tile)
    w = np.minimum(n - c0, tile)
    T = tm * tn
    u = S.u64(seed, 556, 0, (4 + 2 * extra) * T).reshape(4 + 2 * extra, T)
    rnd_r = lambda q: r0 + (u[q] % h.astype(np.uint64)).astype(np.int64)  # noqa: E731
    rnd_c = lambda q: c0 + (u[q] % w.astype(np.uint64)).astype(np.int64)  # noqa: E731
    rows = [r0, r0 + h - 1, rnd_r(0), rnd_r(1)]
    cols = [rnd_c(2), rnd_c(3), c0, c0 + w - 1]
    for e in range(extra):
        rows.append(rnd_r(4 + 2 * e))
        cols.append(rnd_c(5 + 2 * e))
    if split is not None and len(split):
        tiles_n = tiles_n or -(-n // split_tn)
        for idx, t in enumerate(np.asarray(split, np.int64)):
            a, b = int(t) // tiles_n, int(t) % tiles_n
            sr0, sc0 = a * split_tm, b * split_tn
            sh, sw = min(m - sr0, split_tm), min(n - sc0, split_tn)
            L = max(sh, sw)
            perm = np.argsort(S.u64(seed, 557 + idx, 0, L), kind="stable")
            i = np.arange(L, dtype=np.int64)
            rows.append(sr0 + i % sh)
            cols.append(sc0 + perm % sw)
    rows, cols = np.concatenate(rows), np.concatenate(cols)
    lin = np.unique(rows * n + cols)
    return lin // n, lin % n


def sampled_err(got: np.ndarray, dtype: int, rows, cols, ref64, bound) -> float:
    """The parity metric over the sampled entries."""
    return rel_err(got[rows, cols], dtype, ref64, bound)
