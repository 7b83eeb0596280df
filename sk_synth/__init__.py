"""Seeded synthetic inputs for the GEMM tests and benchmark.

This module only draws numbers; it contains none of the GEMM arithmetic and
is the one piece of code that both the CPU oracle's callers and the GPU
path's callers use.

Generator: a counter-based SplitMix64 (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014): the 64-bit output
for (seed, stream, index) is mix(key(seed, stream) + (index + 1) * GAMMA),
where mix is the SplitMix64 finaliser and GAMMA = 0x9E3779B97F4A7C15.  The
element index of a matrix entry is its logical row-major index i * cols + j,
so the same logical matrix comes out for every storage order and leading
dimension.

Distributions:
* ``uniform``: 2 * (top 24 bits * 2^-24) - 1, i.e. multiples of 2^-23 in
  [-1, 1) (exact in fp32; rounded to nearest-even for fp16/bf16).
* ``normal``: Box-Muller in fp64 from two 53-bit uniforms taken from streams
  2s and 2s+1 ... of the same counter, times ``scale``.
* ``int``: integers uniform in [-r, r] (exact in every type for r <= 256).

Storage: float32 arrays for fp32, uint16 bit patterns for fp16/bf16.  Cells
of the storage that are not part of the logical matrix (leading-dimension
padding) hold a NaN pattern, so any read of them poisons the result.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32, F16, BF16 = 0, 1, 2
GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

# Seeds of the five workload families (SGEMM correctness case, SGEMM square
# sweep, HGEMM 8192^3, Stream-K shape sweep, ABFT case).
SEED_SGEMM_SMALL = 1001
SEED_SGEMM_SQUARE = 1002
SEED_HGEMM_LARGE = 1003
SEED_SWEEP = 1004
SEED_ABFT = 1005

# stream ids of the operands
STREAM_A, STREAM_B, STREAM_C = 0, 1, 2


def _mix(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        k = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) * GAMMA + np.uint64(stream & 0xFFFFFFFF)
        return _mix(np.array([k], np.uint64))[0]


def u64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Raw 64-bit draws for indices [start, start + count)."""
    key = _key(seed, stream)
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + idx * GAMMA)


def _uniform_pm1(seed, stream, start, count) -> np.ndarray:
    u = u64(seed, stream, start, count) >> np.uint64(40)  # top 24 bits
    return u.astype(np.float64) * (2.0 ** -23) - 1.0


def _normal(seed, stream, start, count) -> np.ndarray:
    a = (u64(seed, 2 * stream + 1000, start, count) >> np.uint64(11)).astype(np.float64)
    b = (u64(seed, 2 * stream + 1001, start, count) >> np.uint64(11)).astype(np.float64)
    u1 = (a + 1.0) * (2.0 ** -53)  # (0, 1]
    u2 = b * (2.0 ** -53)  # [0, 1)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def _ints(seed, stream, start, count, r) -> np.ndarray:
    u = u64(seed, stream, start, count)
    return (u % np.uint64(2 * r + 1)).astype(np.int64).astype(np.float64) - r


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (nearest-even) -> bf16 bits (nearest-even)."""
    f = np.ascontiguousarray(x, np.float32).view(np.uint32)
    nan = (f & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (f >> np.uint32(16)) & np.uint32(1)
    r = ((f + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    r[nan] = np.uint16(0x7FC0)
    return r


def encode(x: np.ndarray, dtype: int) -> np.ndarray:
    """fp64 values -> storage array of the type (nearest-even)."""
    if dtype == F32:
        return x.astype(np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    return to_bf16_bits(x)


def nan_fill(dtype: int):
    return np.float32(np.nan) if dtype == F32 else np.uint16(0x7E00 if dtype == F16 else 0x7FC0)


def values(seed: int, stream: int, start: int, count: int, dist: str = "uniform",
           scale: float = 1.0, int_range: int = 4) -> np.ndarray:
    if dist == "uniform":
        v = _uniform_pm1(seed, stream, start, count)
    elif dist == "normal":
        v = _normal(seed, stream, start, count)
    elif dist == "int":
        v = _ints(seed, stream, start, count, int_range)
    else:
        raise ValueError(dist)
    return v * scale if scale != 1.0 else v


def matrix(seed: int, stream: int, rows: int, cols: int, dtype: int, dist: str = "uniform",
           order: str = "row", ld: int | None = None, scale: float = 1.0,
           int_range: int = 4) -> np.ndarray:
    """Flat storage array of a rows x cols matrix.

    order "row": element (i, j) at i*ld + j (ld >= cols);
    order "col": element (i, j) at j*ld + i (ld >= rows).
    """
    contig = cols if order == "row" else rows
    outer = rows if order == "row" else cols
    ld = contig if ld is None else ld
    assert ld >= max(contig, 1)
    stype = np.float32 if dtype == F32 else np.uint16
    size = (outer - 1) * ld + contig if outer > 0 and contig > 0 else 0
    out = np.full(max(size, 0), nan_fill(dtype), dtype=stype)
    if size == 0:
        return out
    view = np.lib.stride_tricks.as_strided(out, shape=(outer, contig),
                                           strides=(ld * out.itemsize, out.itemsize))
    total = rows * cols

    def fill(start):
        cnt = min(_CHUNK, total - start)
        enc = encode(values(seed, stream, start, cnt, dist, scale, int_range), dtype)
        li = np.arange(start, start + cnt, dtype=np.int64)
        i, j = li // cols, li % cols
        if order == "row":
            view[i, j] = enc
        else:
            view[j, i] = enc

    starts = range(0, total, _CHUNK)
    if len(starts) == 1:
        fill(0)
    else:
        # chunks are independent (counter-based draws into disjoint cells);
        # numpy releases the interpreter lock in this arithmetic
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(fill, starts))
    return out


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def signs(seed: int, stream: int, n: int) -> np.ndarray:
    """+-1 vector (fp64) for randomised product checks."""
    u = u64(seed, stream, 0, n)
    return np.where((u >> np.uint64(63)) == np.uint64(1), 1.0, -1.0)


def sweep_shapes(count: int = 2000, seed: int = SEED_SWEEP, tile_m: int = 256,
                 tile_n: int = 256, p: int = 256):
    """Shape list of the Stream-K sweep: m, n, k log-uniform on [128, 16384]
    rounded to multiples of 16 (3/4 of the list), skinny shapes with
    m in [128, 256] and k in [8192, 16384] (1/8), and shapes whose tile count
    is 256*j + r with small r, just above a multiple of the CU count (1/8)."""
    n_skinny = count // 8
    n_adv = count // 8
    n_rand = count - n_skinny - n_adv
    raw = u64(seed, 77, 0, 64 * count)
    pos = [0]

    def unif():
        v = float(raw[pos[0]] >> np.uint64(11)) * (2.0 ** -53)
        pos[0] += 1
        return v

    def logu(lo, hi):
        x = math.exp(math.log(lo) + unif() * (math.log(hi) - math.log(lo)))
        return int(min(hi, max(lo, 16 * round(x / 16))))

    shapes = []
    for _ in range(n_rand):
        shapes.append(("random", logu(128, 16384), logu(128, 16384), logu(128, 16384)))
    for _ in range(n_skinny):
        shapes.append(("skinny", logu(128, 256), logu(128, 16384), logu(8192, 16384)))
    max_tiles = 16384 // min(tile_m, tile_n)
    while len(shapes) < count:
        j = 1 + int(unif() * 8)
        r = 1 + int(unif() * 8)
        t = p * j + r
        # factor t as tiles_m * tiles_n with both within the [128, 16384] range
        facs = [d for d in range(1, int(math.isqrt(t)) + 1)
                if t % d == 0 and t // d <= max_tiles]
        if not facs:
            continue
        tm = max(facs)
        tn = t // tm
        if unif() < 0.5:
            tm, tn = tn, tm
        dm = 16 * int(unif() * (tile_m // 16))
        dn = 16 * int(unif() * (tile_n // 16))
        m = max(16, tm * tile_m - dm)
        n = max(16, tn * tile_n - dn)
        shapes.append(("adversarial", m, n, logu(128, 16384)))
    return shapes
