"""Pins of the oracle's GEMM (CPU only).

The oracle is the GEMM definition C = alpha*A*B + beta*C_in (Stream-K page,
section 3 background) computed by the six-loop blocked structure of the same
page's Algorithm 1.  None of these checks re-types that formula: they compare
it with exact rational arithmetic on tiny inputs, with closed forms, with the
IEEE formats' definitions (via numpy's own conversions), and with identities.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import sk_synth as S

LAYOUTS = [oracle.A_ROW_B_ROW, oracle.A_ROW_B_COL, oracle.A_COL_B_ROW, oracle.A_COL_B_COL]
DTYPES = [oracle.F32, oracle.F16, oracle.BF16]


def _orders(layout):
    a = "row" if layout in (oracle.A_ROW_B_ROW, oracle.A_ROW_B_COL) else "col"
    b = "row" if layout in (oracle.A_ROW_B_ROW, oracle.A_COL_B_ROW) else "col"
    return a, b


def _inputs(seed, m, n, k, dtype, layout, dist="uniform", pad=0, scale=1.0):
    ao, bo = _orders(layout)
    lda = (k if ao == "row" else m) + pad
    ldb = (n if bo == "row" else k) + pad
    ldc = n + pad
    A = S.matrix(seed, 0, m, k, dtype, dist, ao, lda, scale)
    B = S.matrix(seed, 1, k, n, dtype, dist, bo, ldb, scale)
    C = S.matrix(seed, 2, m, n, dtype, dist, "row", ldc, scale)
    return A, lda, B, ldb, C, ldc


def _dec(arr, dtype):
    if dtype == oracle.F32:
        return arr.astype(np.float64)
    if dtype == oracle.F16:
        return arr.view(np.float16).astype(np.float64)
    return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _logical(arr, rows, cols, order, ld, dtype):
    v = _dec(arr, dtype)
    out = np.empty((rows, cols))
    for i in range(rows):
        for j in range(cols):
            out[i, j] = v[i * ld + j] if order == "row" else v[j * ld + i]
    return out


# ---------------------------------------------------------------- formats

def test_f16_decode_matches_ieee_for_all_patterns():
    """Every binary16 pattern decodes to numpy's (exact) half -> double value."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    L = oracle.lib()
    got = np.array([L.or_decode_f16(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0xC000, -2.0), (0x7BFF, 65504.0), (0x0400, 2.0 ** -14),
    (0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24), (0x3555, 0.333251953125),
])
def test_f16_known_values(bits, value):
    assert oracle.decode_f16(bits) == value


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0x4049, 3.140625), (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126),
    (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127), (0xBF00, -0.5),
])
def test_bf16_known_values(bits, value):
    assert oracle.decode_bf16(bits) == value


def test_f16_rounding_matches_numpy_including_ties():
    rng = np.random.default_rng(5)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(-30, 17, 3000)))
    # exact midpoints between neighbouring halves (ties go to the even one)
    h = np.arange(0, 0x7BFF, 97, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    xs += list((lo + hi) / 2) + list(-(lo + hi) / 2)
    xs += [65519.99, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26, 0.0, -0.0]
    for x in xs:
        want = np.float64(x).astype(np.float16).view(np.uint16)
        assert oracle.round_f16(float(x)) == int(want), x


def _bf16_nearest_brute(x):
    """Nearest finite bf16 by search over all patterns of the same sign."""
    pats = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (pats << 16).view(np.float32).astype(np.float64)
    a = abs(x)
    d = np.abs(vals - a)
    best = d.min()
    cand = pats[d == best]
    pick = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
    top = (2 - 2.0 ** -8) * 2.0 ** 127  # halfway to the next binade -> inf
    if a >= top:
        pick = 0x7F80
    return int(pick) | (0x8000 if x < 0 else 0)


def test_bf16_rounding_brute_force():
    rng = np.random.default_rng(11)
    xs = list(rng.standard_normal(150) * np.exp2(rng.integers(-140, 128, 150)))
    # ties: midpoints of adjacent patterns
    for p in (0x3F80, 0x3F81, 0x0001, 0x0002, 0x7F7E, 0x1234):
        a = float(np.array([p << 16], np.uint32).view(np.float32)[0])
        b = float(np.array([(p + 1) << 16], np.uint32).view(np.float32)[0])
        xs.append((a + b) / 2)
    for x in xs:
        assert oracle.round_bf16(float(x)) == _bf16_nearest_brute(float(x)), x


# --------------------------------------------------- six-loop GEMM core

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_gemm_exact_rational_tiny(layout, dtype):
    """out64 agrees with the exact rational product to fp64 round-off."""
    rng = np.random.default_rng(100 + 10 * layout + dtype)
    for trial in range(6):
        m, n, k = (int(x) for x in rng.integers(1, 9, 3))
        pad = int(rng.integers(0, 3))
        alpha, beta = [(1.0, 0.0), (0.75, -1.25), (-2.0, 0.5)][trial % 3]
        A, lda, B, ldb, C, ldc = _inputs(200 + trial, m, n, k, dtype, layout, pad=pad)
        out64, bound, rnd = oracle.gemm(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, dtype,
                                        layout, blk=(3, 2, 2))
        ao, bo = _orders(layout)
        Al = _logical(A, m, k, ao, lda, dtype)
        Bl = _logical(B, k, n, bo, ldb, dtype)
        Cl = _logical(C, m, n, "row", ldc, dtype)
        for i in range(m):
            for j in range(n):
                exact = Fraction(alpha) * sum(Fraction(Al[i, l]) * Fraction(Bl[l, j])
                                              for l in range(k))
                if beta != 0.0:
                    exact += Fraction(beta) * Fraction(Cl[i, j])
                absb = abs(alpha) * sum(abs(Al[i, l] * Bl[l, j]) for l in range(k)) + \
                    abs(beta) * abs(Cl[i, j])
                assert abs(Fraction(out64[i, j]) - exact) <= Fraction((k + 2) * 2.0 ** -52 * absb)
                assert bound[i, j] == pytest.approx(absb, rel=1e-14, abs=0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_gemm_bruteforce_all_tiny_shapes_integer_exact(dtype):
    """Brute force over every m, n, k in [1, 6]: with small-integer inputs the
    product is exact, so out64 equals a plain triple loop bit for bit."""
    for m in range(1, 7):
        for n in range(1, 7):
            for k in range(1, 7):
                layout = (m + n + k) % 4
                A, lda, B, ldb, C, ldc = _inputs(7 * m + 11 * n + 13 * k, m, n, k, dtype, layout,
                                                 dist="int")
                out64, _, _ = oracle.gemm(m, n, k, 1.0, A, lda, B, ldb, 2.0, C, ldc, dtype,
                                          layout, blk=(2, 4, 3), want_round=False)
                ao, bo = _orders(layout)
                Al = _logical(A, m, k, ao, lda, dtype)
                Bl = _logical(B, k, n, bo, ldb, dtype)
                Cl = _logical(C, m, n, "row", ldc, dtype)
                want = np.zeros((m, n))
                for i in range(m):
                    for j in range(n):
                        s = 0.0
                        for l in range(k):
                            s += Al[i, l] * Bl[l, j]
                        want[i, j] = s + 2.0 * Cl[i, j]
                assert np.array_equal(out64, want)


def test_gemm_blocking_does_not_change_bits():
    """Algorithm 1 keeps k ascending per element, so any blocking gives the
    same fp64 bits."""
    m, n, k = 37, 29, 53
    A, lda, B, ldb, C, ldc = _inputs(3, m, n, k, oracle.F32, oracle.A_ROW_B_ROW)
    outs = [oracle.gemm(m, n, k, 1.0, A, lda, B, ldb, 1.0, C, ldc, oracle.F32, 0, blk=b)[0]
            for b in [(1, 1, 1), (8, 16, 4), (64, 64, 64), (5, 7, 53)]]
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint64), outs[0].view(np.uint64))


def test_gemm_identity_and_permutations_exact():
    m = k = 24
    n = 17
    rng = np.random.default_rng(0)
    Bv = S.matrix(9, 1, k, n, S.F32)  # row-major k x n
    I = np.eye(m, k, dtype=np.float32).ravel()
    out, _, rnd = oracle.gemm(m, n, k, 1.0, I, k, Bv, n, 0.0, None, n, oracle.F32, 0)
    assert np.array_equal(rnd.ravel(), Bv)
    perm = rng.permutation(m)
    P = np.zeros((m, k), np.float32)
    P[np.arange(m), perm] = 1.0
    out, _, rnd = oracle.gemm(m, n, k, 1.0, P.ravel(), k, Bv, n, 0.0, None, n, oracle.F32, 0)
    assert np.array_equal(rnd, Bv.reshape(k, n)[perm])
    # A * Q permutes columns of A
    Av = S.matrix(9, 0, m, k, S.F32)
    q = rng.permutation(k)
    Q = np.zeros((k, k), np.float32)
    Q[q, np.arange(k)] = 1.0
    out, _, rnd = oracle.gemm(m, k, k, 1.0, Av, k, Q.ravel(), k, 0.0, None, k, oracle.F32, 0)
    assert np.array_equal(rnd, Av.reshape(m, k)[:, q])


@pytest.mark.parametrize("dtype", DTYPES)
def test_gemm_all_ones_equals_k(dtype):
    m, n, k = 33, 20, 77
    one = {oracle.F32: np.float32(1.0), oracle.F16: np.uint16(0x3C00), oracle.BF16: np.uint16(0x3F80)}[dtype]
    A = np.full(m * k, one)
    B = np.full(k * n, one)
    out, bound, rnd = oracle.gemm(m, n, k, 1.0, A, k, B, n, 0.0, None, n, dtype, 0, blk=(8, 8, 8))
    assert (out == k).all() and (bound == k).all()


def test_gemm_rank_one_closed_form():
    """A = x y^T, B = y' z^T  =>  C = (y . y') x z^T, exact for integers."""
    m, n, k = 19, 23, 31
    r = np.random.default_rng(4)
    x, y, yp, z = (r.integers(-5, 6, s).astype(np.float64) for s in (m, k, k, n))
    A = np.outer(x, y).astype(np.float32).ravel()
    B = np.outer(yp, z).astype(np.float32).ravel()
    out, _, _ = oracle.gemm(m, n, k, 1.0, A, k, B, n, 0.0, None, n, oracle.F32, 0)
    assert np.array_equal(out, float(y @ yp) * np.outer(x, z))


def test_gemm_alpha_beta_semantics():
    m, n, k = 9, 11, 5
    A = np.zeros(m * k, np.float32)
    B = S.matrix(1, 1, k, n, S.F32)
    C = S.matrix(1, 2, m, n, S.F32)
    out, bound, _ = oracle.gemm(m, n, k, 3.0, A, k, B, n, -0.5, C, n, oracle.F32, 0)
    assert np.array_equal(out, -0.5 * C.reshape(m, n).astype(np.float64))
    assert np.array_equal(bound, 0.5 * np.abs(C.reshape(m, n).astype(np.float64)))
    # beta == 0: C_in is not read (NaN in C does not propagate)
    Cn = np.full(m * n, np.nan, np.float32)
    A1 = S.matrix(1, 0, m, k, S.F32)
    out, _, _ = oracle.gemm(m, n, k, 1.0, A1, k, B, n, 0.0, Cn, n, oracle.F32, 0)
    assert np.isfinite(out).all()


def test_gemm_bound_equals_value_for_nonnegative_inputs():
    m, n, k = 14, 15, 40
    A = np.abs(S.matrix(2, 0, m, k, S.F32))
    B = np.abs(S.matrix(2, 1, k, n, S.F32))
    out, bound, _ = oracle.gemm(m, n, k, 1.0, A, k, B, n, 0.0, None, n, oracle.F32, 0)
    assert np.array_equal(out, bound)
    out2, bound2, _ = oracle.gemm(m, n, k, -1.0, A, k, B, n, 0.0, None, n, oracle.F32, 0)
    assert np.array_equal(out2, -bound) and np.array_equal(bound2, bound)


@pytest.mark.parametrize("dtype", DTYPES)
def test_rounded_output_is_rne_of_out64(dtype):
    m, n, k = 21, 13, 70
    A, lda, B, ldb, C, ldc = _inputs(8, m, n, k, dtype, oracle.A_ROW_B_COL, dist="normal",
                                     scale=0.3)
    out, _, rnd = oracle.gemm(m, n, k, 1.0, A, lda, B, ldb, 1.0, C, ldc, dtype,
                              oracle.A_ROW_B_COL)
    if dtype == oracle.F32:
        assert np.array_equal(rnd, out.astype(np.float32))
    elif dtype == oracle.F16:
        assert np.array_equal(rnd, out.astype(np.float16).view(np.uint16))
    else:
        for v, r in zip(out.ravel()[:200], rnd.ravel()[:200]):
            assert int(r) == _bf16_nearest_brute(float(v))


def test_entries_match_full_oracle():
    m, n, k = 50, 45, 300
    A, lda, B, ldb, C, ldc = _inputs(12, m, n, k, oracle.BF16, oracle.A_COL_B_COL, pad=3)
    out, bound, _ = oracle.gemm(m, n, k, 0.5, A, lda, B, ldb, 2.0, C, ldc, oracle.BF16,
                                oracle.A_COL_B_COL)
    rows = np.arange(0, m, 3)
    cols = (rows * 7) % n
    e, eb = oracle.gemm_entries(m, n, k, 0.5, A, lda, B, ldb, 2.0, C, ldc, oracle.BF16,
                                oracle.A_COL_B_COL, rows, cols)
    assert np.array_equal(e, out[rows, cols]) and np.array_equal(eb, bound[rows, cols])


def test_padding_is_never_read():
    """Leading-dimension padding holds NaN; a finite result proves the oracle
    reads only the logical matrix."""
    m, n, k = 17, 19, 23
    for layout in LAYOUTS:
        A, lda, B, ldb, C, ldc = _inputs(21, m, n, k, oracle.F16, layout, pad=5)
        out, bound, _ = oracle.gemm(m, n, k, 1.0, A, lda, B, ldb, 1.0, C, ldc, oracle.F16, layout)
        assert np.isfinite(out).all() and np.isfinite(bound).all()


# ------------------------------------------------------------- Freivalds

def test_freivalds_accepts_oracle_result_and_catches_a_planted_error():
    m, n, k = 64, 48, 96
    A, lda, B, ldb, C, ldc = _inputs(31, m, n, k, oracle.F32, oracle.A_ROW_B_ROW)
    out, bound, rnd = oracle.gemm(m, n, k, 1.0, A, lda, B, ldb, 1.0, C, ldc, oracle.F32, 0)
    X = np.stack([S.signs(5, 0, n), S.signs(5, 1, n)])
    w = oracle.freivalds(m, n, k, 1.0, A, lda, B, ldb, 1.0, C, ldc, rnd, n, oracle.F32, 0, X)
    assert w < 1e-6
    bad = rnd.copy()
    bad[7, 9] += 0.01 * bound[7, 9]
    w2 = oracle.freivalds(m, n, k, 1.0, A, lda, B, ldb, 1.0, C, ldc, bad, n, oracle.F32, 0, X)
    assert w2 > 1e-4
