"""Pins of the oracle's ABFT verification domain (CPU only).

Fault-tolerant GEMM page: the checksum relations e^T(AB) = (e^T A)B and
(AB)e = A(Be) (thread-level scheme, Fig. 3; threadblock-level, Figs. 5-7);
a fault is located at the intersection of the mismatching row and column
and corrected from the checksum.
"""
import numpy as np
import pytest

import oracle
import sk_synth as S


def _block(seed, rows, cols, kk, dist="int"):
    A = S.matrix(seed, 0, rows, kk, S.F32, dist).reshape(rows, kk).astype(np.float64)
    B = S.matrix(seed, 1, kk, cols, S.F32, dist).reshape(kk, cols).astype(np.float64)
    C, _, _ = oracle.gemm(rows, cols, kk, 1.0, A.astype(np.float32).ravel(), kk,
                          B.astype(np.float32).ravel(), cols, 0.0, None, cols, oracle.F32, 0,
                          want_round=False)
    return A, B, C


def test_checksum_identities_exact_on_integers():
    A, B, C = _block(1, 24, 20, 30)
    e_m, e_n = np.ones(24), np.ones(20)
    assert np.array_equal(e_m @ C, (e_m @ A) @ B)
    assert np.array_equal(C @ e_n, A @ (B @ e_n))


def test_clean_block_reports_nothing():
    for seed in range(20):
        A, B, C = _block(seed, 32, 32, 64, dist="uniform")
        c32 = C.astype(np.float32)
        st, _ = oracle.abft_check(A, B, c32)
        assert st == 0


def test_every_position_of_a_tiny_block_is_located_and_corrected():
    """Brute force: a 1e3 additive fault at each position of an 8 x 6 block."""
    A, B, C = _block(3, 8, 6, 12)
    for i in range(8):
        for j in range(6):
            c = C.astype(np.float32).copy()
            c[i, j] += np.float32(1e3)
            st, info = oracle.abft_check(A, B, c)
            assert st == 1 and info[:2] == (i, j)
            assert info[2] == pytest.approx(1e3)
            assert np.array_equal(c, C.astype(np.float32))  # exact on integers


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan, 3.0e38])
def test_nonfinite_and_huge_faults_are_corrected(bad):
    A, B, C = _block(4, 16, 16, 40, dist="uniform")
    c = C.astype(np.float32)
    want = c.copy()
    c[5, 11] = np.float32(bad)
    st, info = oracle.abft_check(A, B, c)
    assert st == 1 and info[:2] == (5, 11)
    assert abs(float(c[5, 11]) - float(want[5, 11])) <= 1e-5 * float(np.abs(A[5]) @ np.abs(B[:, 11]))


def test_bit_flips_of_high_bits_are_located():
    A, B, C = _block(6, 16, 16, 64, dist="uniform")
    c0 = C.astype(np.float32)
    for bit in (30, 29, 28, 27, 26, 31):
        c = c0.copy()
        u = c.view(np.uint32)
        u[3, 7] ^= np.uint32(1 << bit)
        st, info = oracle.abft_check(A, B, c)
        assert st == 1 and info[:2] == (3, 7), bit


def test_two_faults_in_one_domain_are_not_guessed():
    A, B, C = _block(7, 10, 10, 20)
    c = C.astype(np.float32)
    c[1, 2] += 500.0
    c[4, 8] -= 700.0
    st, _ = oracle.abft_check(A, B, c)
    assert st == 2
