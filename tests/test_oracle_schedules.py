"""Pins of the oracle's decompositions and their simulated execution (CPU).

Worked values come from the Stream-K page (tests/golden/stream_k_worked_examples.json
cites each); invariants are the ones the page states in section 4 and 5.2.
"""
import json
import os

import numpy as np
import pytest

import oracle
import sk_synth as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "stream_k_worked_examples.json")))


def _segs_by_cta(rec, n_cta):
    out = [[] for _ in range(n_cta)]
    for r in rec:
        out[int(r[0])].append(tuple(int(v) for v in r[1:]))
    return out


def test_section4_example_72_iterations_per_cta():
    g = GOLD["section4_basic_stream_k_example"]
    rec, ncta = oracle.sk_plan(g["m"], g["n"], g["k"], g["blk_m"], g["blk_n"], g["blk_k"],
                               oracle.SK, g["g"])
    work = oracle.plan_cta_work(rec, ncta)
    assert ncta == g["g"] and work == [g["iters_per_cta"]] * g["g"]
    assert g["iters_per_cta"] * g["blk_k"] == g["cta_volume_k"]
    ipt = g["k"] // g["blk_k"]
    assert ipt == g["single_iteration_vs_tile_ratio"]
    # the worked schedule: CTA0 tiles 0, 1 and the head of tile 2, ...
    segs = _segs_by_cta(rec, ncta)
    assert [s[0] for s in segs[0]] == [0, 1, 2]
    assert segs[0][2][1:3] == (0, 8) and segs[1][0][:3] == (2, 8, 32)


def test_fig1_fig2_utilisation():
    g = GOLD["fig1_fig2_384x384x128_on_4_sms"]
    p = g["p"]
    # (a) DP with 128x128x128 CTAs
    rec, n = oracle.sk_plan(384, 384, 128, 128, 128, 128, oracle.DP, 0)
    assert n == g["dp_128x128x128_ctas"]
    assert oracle.quantization_efficiency(oracle.plan_cta_work(rec, n), p) == \
        pytest.approx(g["dp_128x128x128_utilisation"])
    # (b) DP with 128x64x128 CTAs
    rec, n = oracle.sk_plan(384, 384, 128, 128, 64, 128, oracle.DP, 0)
    assert n == g["dp_128x64x128_ctas"]
    w = [x * 0.5 for x in oracle.plan_cta_work(rec, n)]  # half-size tiles
    assert oracle.quantization_efficiency(w, p) == pytest.approx(g["dp_128x64x128_utilisation"])
    # Fig. 2a fixed split s=2, 128x128x64 CTAs (BLK_K = 64: one iteration per split)
    rec, n = oracle.sk_plan(384, 384, 128, 128, 128, 64, oracle.FIXED, 2)
    assert n == g["fixed_split_s2_ctas"]
    assert set(oracle.plan_cta_work(rec, n)) == {1}
    assert oracle.quantization_efficiency(oracle.plan_cta_work(rec, n), p) == \
        pytest.approx(g["fixed_split_s2_utilisation"])
    # Fig. 2b basic Stream-K, g = 4
    rec, n = oracle.sk_plan(384, 384, 128, 128, 128, 4, oracle.SK, 4)
    assert oracle.quantization_efficiency(oracle.plan_cta_work(rec, n), p) == \
        pytest.approx(g["stream_k_g4_utilisation"])


def test_fig3a_start_offsets():
    g = GOLD["section5_2_fig3a_skew"]
    rec, n = oracle.sk_plan(g["m"], g["n"], g["k"], g["blk_m"], g["blk_n"], g["blk_k"],
                            oracle.SK, g["g"])
    segs = _segs_by_cta(rec, n)
    starts = [segs[x][0][1] * g["blk_k"] for x in range(n)]
    assert starts == g["start_k_offsets"]


@pytest.mark.parametrize("shape", [(384, 384, 128, 128, 128, 4), (300, 520, 200, 64, 128, 16),
                                   (1000, 64, 999, 128, 64, 32)])
def test_sk_with_g_equal_t_is_data_parallel(shape):
    m, n, k, bm, bn, bk = shape
    t = -(-m // bm) * -(-n // bn)
    sk, ns = oracle.sk_plan(m, n, k, bm, bn, bk, oracle.SK, t)
    dp, nd = oracle.sk_plan(m, n, k, bm, bn, bk, oracle.DP, 0)
    assert ns == nd and np.array_equal(sk, dp)


@pytest.mark.parametrize("s", [2, 4, 8])
def test_sk_with_g_multiple_of_t_is_fixed_split(s):
    m, n, k, bm, bn, bk = 384, 256, 256, 128, 128, 8  # ipt = 32, divisible by s
    t = 6
    sk, ns = oracle.sk_plan(m, n, k, bm, bn, bk, oracle.SK, s * t)
    fx, nf = oracle.sk_plan(m, n, k, bm, bn, bk, oracle.FIXED, s)
    assert ns == nf
    a = sorted(tuple(r[1:6]) for r in sk)
    b = sorted(tuple(r[1:6]) for r in fx)
    assert a == b


def _check_plan_invariants(rec, n_cta, t, ipt):
    segs = _segs_by_cta(rec, n_cta)
    cover = {}
    for x, ss in enumerate(segs):
        for idx, (tile, lb, le, st, en, lp) in enumerate(ss):
            if not st:
                assert idx == 0  # only a CTA's first segment can be a partial
            assert st == (lb == 0) and en == (le == ipt)
            cover.setdefault(tile, []).append((lb, le, x))
    assert sorted(cover) == list(range(t))
    for tile, parts in cover.items():
        parts.sort()
        assert parts[0][0] == 0 and parts[-1][1] == ipt
        for a, b in zip(parts, parts[1:]):
            assert a[1] == b[0]  # contiguous, no overlap
    return segs, cover


@pytest.mark.parametrize("t_tiles,p", [(576 // 1, 256), (300, 256), (257, 256), (20, 8), (13, 4)])
def test_two_tile_hybrid_invariants(t_tiles, p):
    """Section 5.2: each Stream-K CTA gets more than one and less than two
    tiles of iterations, and every owner receives from exactly one peer."""
    bm = bn = 16
    m, n = bm * t_tiles, bn
    k, bk = 640, 64  # ipt = 10
    ipt = 10
    rec, nc = oracle.sk_plan(m, n, k, bm, bn, bk, oracle.HYBRID2, p)
    segs, cover = _check_plan_invariants(rec, nc, t_tiles, ipt)
    r = t_tiles % p
    sk_tiles = r + p
    sk_work = [sum(le - lb for (tile, lb, le, *_ ) in ss if tile < sk_tiles) for ss in segs]
    assert all(ipt <= w_ < 2 * ipt for w_ in sk_work[:-1])
    for tile, parts in cover.items():
        assert len(parts) <= 2
    for r_ in rec:
        if r_[6] >= 0:
            assert r_[6] == r_[0] + 1  # exactly one peer, the next CTA


def test_one_tile_hybrid_and_basic_sk_invariants():
    for (m, n, k, bm, bn, bk, mode, prm) in [(16 * 13, 16, 640, 16, 16, 64, oracle.HYBRID1, 4),
                                             (16 * 9, 16, 640, 16, 16, 64, oracle.SK, 7),
                                             (128, 128, 384 * 4, 128, 128, 4, oracle.SK, 4),
                                             (16 * 3, 16, 640, 16, 16, 64, oracle.SK, 50)]:
        rec, nc = oracle.sk_plan(m, n, k, bm, bn, bk, mode, prm)
        t = -(-m // bm) * -(-n // bn)
        _check_plan_invariants(rec, nc, t, -(-k // bk))
        # one partial slot per CTA is enough
        for x in range(nc):
            assert sum(1 for r in rec if r[0] == x and r[4] == 0) <= 1


def test_fig9_single_tile_strong_scaling():
    """Fig. 9: 128x128x384 on four SMs; data-parallel runs the whole k range
    in one CTA, Stream-K splits it over all four."""
    rec, n = oracle.sk_plan(128, 128, 384, 128, 128, 4, oracle.DP, 0)
    assert n == 1 and oracle.plan_cta_work(rec, n) == [96]
    rec, n = oracle.sk_plan(128, 128, 384, 128, 128, 4, oracle.SK, 4)
    assert oracle.plan_cta_work(rec, n) == [24] * 4
    owner = [r for r in rec if r[4] == 1]
    assert len(owner) == 1 and owner[0][6] == 3  # CTA 0 sums the partials of CTAs 1..3


# ------------------------------------------------------ simulated execution

def _int_problem(seed, m, n, k, layout=oracle.A_ROW_B_ROW, dtype=oracle.F32):
    ao = "row" if layout in (0, 1) else "col"
    bo = "row" if layout in (0, 2) else "col"
    A = S.matrix(seed, 0, m, k, dtype, "int", ao)
    B = S.matrix(seed, 1, k, n, dtype, "int", bo)
    C = S.matrix(seed, 2, m, n, dtype, "int", "row")
    lda = k if ao == "row" else m
    ldb = n if bo == "row" else k
    return A, lda, B, ldb, C, n


def test_stream_k_execution_bit_exact_for_every_grid_size():
    """Integer inputs make every partial sum exact, so each decomposition must
    reproduce the six-loop result bit for bit, for every g in [1, 2*total]."""
    m, n, k, bm, bn, bk = 40, 24, 36, 16, 8, 4  # t = 9, ipt = 9, total = 81
    A, lda, B, ldb, C, ldc = _int_problem(1, m, n, k)
    ref, _, _ = oracle.gemm(m, n, k, 1.0, A, lda, B, ldb, -1.0, C, ldc, oracle.F32, 0,
                            want_round=False)
    total = 81
    for g in range(1, 2 * total + 1):
        out, _ = oracle.sk_execute(m, n, k, 1.0, A, lda, B, ldb, -1.0, C, ldc, oracle.F32, 0,
                                   bm, bn, bk, oracle.SK, g, seed=g, policy=g % 3)
        assert np.array_equal(out, ref), g


@pytest.mark.parametrize("mode,param", [(oracle.DP, 0), (oracle.FIXED, 3), (oracle.HYBRID1, 4),
                                        (oracle.HYBRID2, 4), (oracle.DP_PERSISTENT, 3)])
def test_other_decompositions_bit_exact(mode, param):
    m, n, k, bm, bn, bk = 16 * 7, 8 * 3, 50, 16, 8, 4  # t = 21, ipt = 13
    for layout in range(4):
        A, lda, B, ldb, C, ldc = _int_problem(2 + layout, m, n, k, layout, oracle.BF16)
        ref, _, _ = oracle.gemm(m, n, k, 2.0, A, lda, B, ldb, 1.0, C, ldc, oracle.BF16, layout,
                                want_round=False)
        for seed in range(3):
            out, _ = oracle.sk_execute(m, n, k, 2.0, A, lda, B, ldb, 1.0, C, ldc, oracle.BF16,
                                       layout, bm, bn, bk, mode, param, seed=seed, policy=seed)
            assert np.array_equal(out, ref)


def test_adversarial_interleavings_yield_and_still_agree():
    """Lowest-id-first makes every owner reach its wait before its peer has
    produced, so waits must yield; results still agree."""
    m, n, k = 64, 64, 256
    A, lda, B, ldb, C, ldc = _int_problem(9, m, n, k)
    ref, _, _ = oracle.gemm(m, n, k, 1.0, A, lda, B, ldb, 0.0, None, ldc, oracle.F32, 0,
                            want_round=False)
    out, ny = oracle.sk_execute(m, n, k, 1.0, A, lda, B, ldb, 0.0, None, ldc, oracle.F32, 0,
                                32, 32, 8, oracle.SK, 11, seed=0, policy=1)
    assert ny > 0 and np.array_equal(out, ref)


def test_real_valued_execution_within_rounding():
    m, n, k = 70, 50, 300
    A = S.matrix(4, 0, m, k, S.F32)
    B = S.matrix(4, 1, k, n, S.F32)
    ref, bound, _ = oracle.gemm(m, n, k, 1.0, A, k, B, n, 0.0, None, n, oracle.F32, 0,
                                want_round=False)
    out, _ = oracle.sk_execute(m, n, k, 1.0, A, k, B, n, 0.0, None, n, oracle.F32, 0,
                               32, 32, 16, oracle.SK, 17, seed=3)
    assert np.max(np.abs(out - ref) / bound) < 1e-13
