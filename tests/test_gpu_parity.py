"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Tolerances (max |C - C_ref| / (|alpha||A||B| + |beta||C_in|)): 1e-5 for
fp32, 5e-3 for fp16/bf16 inputs with fp32 accumulation.  Schedule
equivalences are bitwise.
"""
import functools

import numpy as np
import pytest

import oracle
import sk_synth as S
import work_centric_decomposition_amd as sk

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gemm_check import (TOL, Case, decode, from_dev, rel_err, sampled_err,  # noqa: E402
                        split_tiles, tile_sample_indices, to_dev)

DTYPES = [sk.F32, sk.F16, sk.BF16]
LAYOUTS = [sk.A_ROW_B_ROW, sk.A_ROW_B_COL, sk.A_COL_B_ROW, sk.A_COL_B_COL]


@pytest.fixture(autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    assert sk.device_status() == sk.OK


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------ the SGEMM correctness case

@pytest.mark.parametrize("forced", [0, 4])
def test_sgemm_384_uniform_auto_and_forced_grid4(forced):
    """384x384x128 fp32, row-major A and B, U[-1,1], alpha=1 beta=0; AUTO and a
    forced Stream-K grid of 4 workgroups (partial-tile fixup)."""
    _say("case sgemm 384^2x128 forced", forced)
    c = Case(384, 384, 128, sk.F32, sk.A_ROW_B_ROW, S.SEED_SGEMM_SMALL)
    opts = sk.make_options(forced_grid=forced) if forced else None
    got = c.run(1.0, 0.0, opts)
    ref, bound = c.reference()
    assert rel_err(got, sk.F32, ref, bound) <= TOL[sk.F32]


# ------------------------------------- ragged shapes, all types and layouts

TILES = [sk.TILE_AUTO, sk.TILE_LARGE, sk.TILE_SMALL]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("tile", TILES)
def test_ragged_shapes_all_layouts(dtype, layout, tile):
    # (520, 264, 320): interior tiles with vector-aligned rows and alpha, beta
    # not 1, 0 (the epilogue's straight-line path) next to edge tiles
    for (m, n, k, pad, alpha, beta) in [(300, 520, 200, 0, 1.0, 0.0), (513, 257, 1000, 8, 0.5, -1.5),
                                        (17, 33, 48, 0, 1.0, 1.0), (1, 1, 8, 0, 2.0, 0.0),
                                        (520, 264, 320, 0, 0.75, 1.25)]:
        _say("case ragged", dtype, layout, tile, m, n, k, pad)
        c = Case(m, n, k, dtype, layout, 7 + m + layout, pad=pad)
        got = c.run(alpha, beta, sk.make_options(tile=tile))
        ref, bound = c.reference(alpha, beta)
        assert rel_err(got, dtype, ref, bound) <= TOL[dtype], (m, n, k)


@pytest.mark.parametrize("dtype", DTYPES)
def test_k_not_multiple_of_vector_width_and_odd_ld(dtype):
    for (m, n, k, pad) in [(129, 130, 131, 1), (64, 300, 77, 3), (260, 70, 5, 0)]:
        _say("case odd", dtype, m, n, k, pad)
        c = Case(m, n, k, dtype, sk.A_ROW_B_COL, 40 + k, pad=pad)
        got = c.run(1.0, 0.5)
        ref, bound = c.reference(1.0, 0.5)
        assert rel_err(got, dtype, ref, bound) <= TOL[dtype], (m, n, k)


@pytest.mark.parametrize("dtype", DTYPES)
def test_repacked_operands_buffers_grow_and_shrink_between_calls(dtype):
    """Operands the kernels cannot read in place are repacked into copies the
    stream's workspace keeps from call to call: small, larger (the copies
    grow), smaller again (the larger copies are reused), in the layouts that
    repack one or both operands (fp16/bf16: any mn-contiguous operand; fp32:
    a leading dimension that is not a multiple of four), each against the
    oracle; the tile edges of the 64 x 64 transposes are exercised by ragged
    m, n and k, and the source is read 16, 8, 4 or 2 bytes at a time as its
    rows' alignment allows."""
    if dtype == sk.F32:
        runs = [(130, 70, 77, sk.A_ROW_B_ROW, 1), (1000, 1500, 700, sk.A_COL_B_ROW, 3),
                (300, 130, 65, sk.A_COL_B_COL, 1), (131, 66, 94, sk.A_COL_B_ROW, 1)]
    else:
        runs = [(130, 70, 77, sk.A_ROW_B_ROW, 0), (1000, 1500, 700, sk.A_COL_B_ROW, 0),
                (300, 130, 65, sk.A_COL_B_COL, 5), (257, 513, 129, sk.A_ROW_B_ROW, 3),
                # source rows 8-byte aligned (A: k = 300, B: n = 1004) and
                # 4-byte aligned (A: m = 258, B: k = 138), not 16
                (200, 1004, 300, sk.A_ROW_B_ROW, 0), (258, 130, 138, sk.A_COL_B_COL, 0)]
    for (m, n, k, layout, pad) in runs:
        _say("case repack", dtype, m, n, k, layout, pad)
        c = Case(m, n, k, dtype, layout, 60 + m + layout, pad=pad)
        plan = sk.plan_query(c.desc(1.0, 0.5))
        assert plan.packs != 0, (m, n, k, layout, pad)
        got = c.run(1.0, 0.5)
        ref, bound = c.reference(1.0, 0.5)
        assert rel_err(got, dtype, ref, bound) <= TOL[dtype], (m, n, k, layout)


# ------------------- m-contiguous A, n-contiguous B read in place (fp16/bf16)

# m, n, k, pad, alpha, beta: m and n multiples of 8 but of neither tile size
# (ragged last tiles), or not multiples of 8 (those operands repacked), k
# below one iteration and below one 16-byte chunk (down to a single k-row),
# several iterations with a tail of k-rows, padded leading dimensions, alpha
# and beta applied
MN_CASES = [(296, 520, 200, 0, 1.0, 0.0), (513, 264, 1000, 8, 0.5, -1.5), (64, 2048, 64, 0, 1.0, 1.0),
            (256, 256, 5, 0, 1.0, 0.0), (264, 136, 4100, 16, 1.0, 0.0), (1000, 1000, 1000, 0, 0.75, 1.25),
            (96, 136, 1, 0, 1.0, 0.5)]


def _expected_packs(c):
    """Repack bits the planner must choose for a Case on the 256 or 128
    instance: an operand is read in place when its leading dimension is a
    multiple of 8 elements and, k-contiguous, k is a multiple of 8, or,
    mn-contiguous, its m (A) or n (B) is."""
    a_row = c.layout in (sk.A_ROW_B_ROW, sk.A_ROW_B_COL)
    b_col = c.layout in (sk.A_ROW_B_COL, sk.A_COL_B_COL)
    a_ok = c.lda % 8 == 0 and (c.k if a_row else c.m) % 8 == 0
    b_ok = c.ldb % 8 == 0 and (c.k if b_col else c.n) % 8 == 0
    return (0 if a_ok else 1) | (0 if b_ok else 2)


@pytest.mark.parametrize("dtype", [sk.F16, sk.BF16])
@pytest.mark.parametrize("tile", [sk.TILE_LARGE, sk.TILE_SMALL])
@pytest.mark.parametrize("sched", ["auto", "dp", "forced7"])
def test_mn_contiguous_operands_read_in_place_against_oracle(dtype, tile, sched):
    """Column-major (m-contiguous) A and row-major (n-contiguous) B read in
    place by the 256 and 128 instances (transposing LDS reads) against the
    full oracle output, in the three storage orders with such an operand."""
    kw = {"auto": {}, "dp": {"schedule": sk.SCHED_DP}, "forced7": {"forced_grid": 7}}[sched]
    for (m, n, k, pad, alpha, beta) in MN_CASES:
        for layout in (sk.A_ROW_B_ROW, sk.A_COL_B_ROW, sk.A_COL_B_COL):
            _say("case mn-contiguous", dtype, tile, sched, m, n, k, layout, pad)
            c = Case(m, n, k, dtype, layout, 70 + m + k + layout, pad=pad)
            opts = sk.make_options(tile=tile, **kw)
            p = sk.plan_query(c.desc(alpha, beta), opts)
            assert p.packs == _expected_packs(c), (p.packs, m, n, k, layout, pad)
            got = c.run(alpha, beta, opts)
            ref, bound = c.reference(alpha, beta)
            assert rel_err(got, dtype, ref, bound) <= TOL[dtype], (m, n, k, layout)


def _storage(arr, rows, cols, ld):
    """(rows x cols) view of a row-major storage array with leading dim ld."""
    return np.lib.stride_tricks.as_strided(arr, shape=(rows, cols), strides=(ld * arr.itemsize, arr.itemsize))


@pytest.mark.parametrize("dtype", [sk.F16, sk.BF16])
@pytest.mark.parametrize("tile", [sk.TILE_LARGE, sk.TILE_SMALL])
@pytest.mark.parametrize("layout", [sk.A_ROW_B_ROW, sk.A_COL_B_ROW, sk.A_COL_B_COL])
def test_mn_contiguous_bitwise_equal_to_k_contiguous(dtype, tile, layout):
    """The same operands stored mn-contiguous (read in place, transposed in
    LDS) and k-contiguous feed the MFMAs the same fragments in the same
    order: the outputs are bit for bit equal, on random inputs, under
    data-parallel and split schedules and with beta != 0."""
    for (m, n, k, pad) in [(296, 520, 200, 0), (1000, 1000, 1000, 0), (264, 136, 4104, 16)]:
        _say("case operand order bitwise", dtype, tile, layout, m, n, k, pad)
        c = Case(m, n, k, dtype, layout, 90 + m + layout, pad=pad)
        a_row = layout == sk.A_ROW_B_ROW
        b_col = layout == sk.A_COL_B_COL
        # the same logical A (m x k) and B (k x n), both stored k-contiguous
        Ak = _storage(c.A, m, k, c.lda) if a_row else _storage(c.A, k, m, c.lda).T
        Bk = _storage(c.B, n, k, c.ldb) if b_col else _storage(c.B, k, n, c.ldb).T
        dA2 = to_dev(np.ascontiguousarray(Ak).reshape(-1), dtype)
        dB2 = to_dev(np.ascontiguousarray(Bk).reshape(-1), dtype)
        for kw in ({"schedule": sk.SCHED_DP}, {"forced_grid": 7}, {"forced_grid": 255}):
            o = sk.make_options(tile=tile, **kw)
            d1 = c.desc(1.0, 0.5)
            d2 = sk.make_desc(m, n, k, 1.0, dA2, k, dB2, k, 0.5, c.dC, c.ldc, dtype, sk.A_ROW_B_COL)
            p1, p2 = sk.plan_query(d1, o), sk.plan_query(d2, o)
            assert p1.packs == 0 and p2.packs == 0, (p1.packs, p2.packs)
            assert (p1.grid, p1.schedule, p1.tile_m) == (p2.grid, p2.schedule, p2.tile_m)
            c.reset_c()
            got1 = c.run(1.0, 0.5, o)
            c.reset_c()
            sk.gemm_ex(d2, o)
            torch.cuda.synchronize()
            got2 = c.result()
            assert np.array_equal(got1.view(np.uint8), got2.view(np.uint8)), (m, n, k, kw)


@pytest.mark.parametrize("layout", [sk.A_ROW_B_ROW, sk.A_COL_B_ROW])
def test_mn_contiguous_offsets_at_the_31_bit_limit(layout):
    """mn-contiguous operands whose k-rows span almost 2^31 bytes, the most
    the in-place read takes (2 (k + 64) ld + 1024 below 2^31 - 1): the
    buffer offsets of the last k-rows sit just under 2^31.  The leading
    dimension is padded far beyond m and n, the padding holds NaN (never
    read: chunks at or past m or n are fetched out of range), and every
    128 x 128 output tile and split tile is checked against the oracle on
    the compact matrices.  A leading dimension 8 elements longer crosses the
    limit and the operand is repacked instead."""
    dtype, m, n, k, ld = sk.F16, 1024, 1024, 65464, 16384
    assert 2 * (k + 64) * ld + 1024 < 2 ** 31 - 1 < 2 * (k + 64) * (ld + 8) + 1024
    a_col = layout == sk.A_COL_B_ROW
    _say("case 31-bit offsets", layout, m, n, k, ld)
    A = S.matrix(41, S.STREAM_A, m, k, dtype, "normal", "col" if a_col else "row", None, 1 / np.sqrt(k))
    B = S.matrix(41, S.STREAM_B, k, n, dtype, "normal", "row")

    def padded(host, outer, contig):
        t = torch.full(((outer - 1) * ld + contig,), float("nan"), dtype=torch.float16, device="cuda")
        t.as_strided((outer, contig), (ld, 1)).copy_(to_dev(host, dtype).view(outer, contig))
        return t

    dA, lda = (padded(A, k, m), ld) if a_col else (to_dev(A, dtype), k)
    dB, ldb = padded(B, k, n), ld
    dC = torch.zeros(m * n, dtype=torch.float16, device="cuda")
    d = sk.make_desc(m, n, k, 1.0, dA, lda, dB, ldb, 0.0, dC, n, dtype, layout)
    p = sk.plan_query(d)
    assert p.packs == 0
    sk.gemm_ex(d, None)
    torch.cuda.synchronize()
    got = from_dev(dC, dtype).reshape(m, n)
    rows, cols = tile_sample_indices(m, n, 31, split=split_tiles(p), split_tm=p.tile_m, split_tn=p.tile_n,
                                     tiles_n=p.tiles_n)
    ref, bound = oracle.gemm_entries(m, n, k, 1.0, A, m if a_col else k, B, n, 0.0, None, n, dtype, layout,
                                     rows, cols)
    assert sampled_err(got, dtype, rows, cols, ref, bound) <= TOL[dtype]
    d8 = sk.make_desc(m, n, k, 1.0, dA, lda, dB, ld + 8, 0.0, dC, n, dtype, layout)
    assert sk.plan_query(d8).packs & 2


# storage order of the first and second operands of C^T = B^T A^T
_SWAPPED = {sk.A_ROW_B_ROW: sk.A_COL_B_COL, sk.A_ROW_B_COL: sk.A_ROW_B_COL,
            sk.A_COL_B_ROW: sk.A_COL_B_ROW, sk.A_COL_B_COL: sk.A_ROW_B_ROW}


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_column_major_c_by_transposition(dtype, layout):
    """A column-major C computed as the row-major C^T = B^T A^T, as the
    header describes (m and n swapped, B first, each storage order flipped),
    against the oracle's C, with beta != 0 reading the column-major C_in."""
    for (m, n, k) in [(300, 520, 200), (520, 264, 1000)]:
        _say("case column-major C", dtype, layout, m, n, k)
        c = Case(m, n, k, dtype, layout, 500 + m + layout)
        cin = _storage(c.Cin, m, n, c.ldc)
        dCt = to_dev(np.ascontiguousarray(cin.T).reshape(-1), dtype)  # element (i, j) at j * m + i
        rc = sk.gemm(n, m, k, 0.75, c.dB, c.ldb, c.dA, c.lda, 1.25, dCt, m, dtype, _SWAPPED[layout])
        assert rc == sk.OK
        torch.cuda.synchronize()
        got = from_dev(dCt, dtype).reshape(n, m).T
        ref, bound = c.reference(0.75, 1.25)
        assert rel_err(np.ascontiguousarray(got), dtype, ref, bound) <= TOL[dtype], (m, n, k)


# ------------------------------------------------ the narrow-m instance

# m, n, k, layout, pad, alpha, beta: every row-block count (BM = 64, 128,
# 192, 256 and the edges of each), ragged n and k (k below one iteration,
# not a multiple of the 16-byte chunk, several iterations with a tail),
# operands read in place and repacked (layouts with a non-k-contiguous
# operand), alpha and beta applied
NARROW_CASES = [(1, 300, 200, sk.A_ROW_B_COL, 0, 1.0, 0.0), (17, 513, 1000, sk.A_ROW_B_COL, 8, 0.5, -1.5),
                (64, 256, 64, sk.A_ROW_B_COL, 0, 1.0, 1.0), (65, 700, 4100, sk.A_ROW_B_ROW, 0, 1.0, 0.0),
                (100, 1000, 777, sk.A_COL_B_COL, 3, 2.0, 0.0), (128, 520, 136, sk.A_ROW_B_COL, 0, 1.0, 0.0),
                (144, 2000, 3000, sk.A_ROW_B_COL, 0, 1.0, 0.0), (192, 257, 5000, sk.A_COL_B_ROW, 0, 0.75, 1.25),
                (200, 3000, 1234, sk.A_ROW_B_COL, 0, 1.0, 0.0), (256, 512, 640, sk.A_ROW_B_COL, 0, 1.0, -1.0),
                (250, 1300, 17, sk.A_ROW_B_COL, 1, 1.0, 0.0)]


@pytest.mark.parametrize("dtype", [sk.F16, sk.BF16])
@pytest.mark.parametrize("sched", ["auto", "dp", "forced7", "forced255"])
def test_narrow_instance_against_oracle(dtype, sched):
    """The narrow-m tile (m <= 256) against the full oracle output on every
    case, under the XCD-aware split (AUTO), data-parallel, and basic
    Stream-K with 7 and 255 workgroups (owners adding several peers)."""
    kw = {"auto": {}, "dp": {"schedule": sk.SCHED_DP}, "forced7": {"forced_grid": 7},
          "forced255": {"forced_grid": 255}}[sched]
    for (m, n, k, layout, pad, alpha, beta) in NARROW_CASES:
        _say("case narrow", dtype, sched, m, n, k, layout, pad)
        c = Case(m, n, k, dtype, layout, 300 + m + k, pad=pad)
        opts = sk.make_options(tile=sk.TILE_NARROW, **kw)
        p = sk.plan_query(c.desc(alpha, beta), opts)
        want_bm = 64 if m <= 64 else 128 if m <= 128 else 192 if m <= 192 else 256
        assert (p.tile_m, p.tile_n, p.tiles_m) == (want_bm, 256, 1)
        got = c.run(alpha, beta, opts)
        ref, bound = c.reference(alpha, beta)
        assert rel_err(got, dtype, ref, bound) <= TOL[dtype], (m, n, k)


@pytest.mark.parametrize("dtype", [sk.F16, sk.BF16])
def test_narrow_stream_k_with_g_equal_t_is_bitwise_data_parallel(dtype):
    m, n, k = 176, 4000, 3000
    c = Case(m, n, k, dtype, sk.A_ROW_B_COL, 17)
    t = sk.plan_query(c.desc(1.0, 0.0), sk.make_options(tile=sk.TILE_NARROW)).tiles
    dp = c.run(1.0, 0.0, sk.make_options(schedule=sk.SCHED_DP, tile=sk.TILE_NARROW))
    c.reset_c()
    skg = c.run(1.0, 0.0, sk.make_options(forced_grid=t, tile=sk.TILE_NARROW))
    assert np.array_equal(dp.view(np.uint8), skg.view(np.uint8))


# ----------------------------------------------------------------- edges

@pytest.mark.parametrize("dtype", DTYPES)
def test_quick_returns(dtype):
    c = Case(40, 24, 16, dtype, sk.A_ROW_B_ROW, 3)
    before = c.result()
    sk.gemm(0, 24, 16, 1.0, c.dA, c.lda, c.dB, c.ldb, 1.0, c.dC, c.ldc, dtype, 0)
    torch.cuda.synchronize()
    assert np.array_equal(c.result().view(np.uint8), before.view(np.uint8))
    # k == 0: C = beta * C
    sk.gemm(40, 24, 0, 1.0, c.dA, c.lda, c.dB, c.ldb, -2.0, c.dC, c.ldc, dtype, 0)
    torch.cuda.synchronize()
    want = -2.0 * decode(before, dtype)  # exact: a power-of-two scale
    assert np.array_equal(decode(c.result(), dtype), want)
    # alpha == 0 and beta == 0 writes zeros without reading C (NaN in C)
    c.dC.fill_(float("nan"))
    sk.gemm(40, 24, 16, 0.0, c.dA, c.lda, c.dB, c.ldb, 0.0, c.dC, c.ldc, dtype, 0)
    torch.cuda.synchronize()
    assert np.all(decode(c.result(), dtype) == 0.0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_beta_zero_does_not_read_c(dtype):
    c = Case(300, 300, 64, dtype, sk.A_ROW_B_COL, 5)
    c.dC.fill_(float("nan"))
    got = c.run(1.0, 0.0)
    ref, bound = c.reference(1.0, 0.0)
    assert rel_err(got, dtype, ref, bound) <= TOL[dtype]


# ------------------------------------------------- schedule equivalences

@pytest.mark.parametrize("dtype,tile", [(sk.F32, sk.TILE_LARGE), (sk.F32, sk.TILE_SMALL),
                                        (sk.F16, sk.TILE_LARGE), (sk.F16, sk.TILE_SMALL)])
def test_stream_k_with_g_equal_t_is_bitwise_data_parallel(dtype, tile):
    m, n, k = (1024, 768, 2048) if dtype != sk.F32 else (640, 512, 1024)
    c = Case(m, n, k, dtype, sk.A_ROW_B_COL, 11)
    p = sk.plan_query(sk.make_desc(m, n, k, 1, c.dA, c.lda, c.dB, c.ldb, 0, c.dC, c.ldc, dtype,
                                   sk.A_ROW_B_COL), sk.make_options(tile=tile))
    t = p.tiles
    dp = c.run(1.0, 0.0, sk.make_options(schedule=sk.SCHED_DP, tile=tile))
    c.reset_c()
    skg = c.run(1.0, 0.0, sk.make_options(forced_grid=t, tile=tile))
    assert np.array_equal(dp.view(np.uint8), skg.view(np.uint8))


@pytest.mark.parametrize("dtype", DTYPES)
def test_every_grid_size_exact_on_integer_inputs(dtype):
    """Small integers make every partial sum exact in fp32, so every
    decomposition, and both tile instances of each type, give the same
    bits."""
    m, n, k = (700, 600, 1024) if dtype == sk.F32 else (600, 520, 2048)
    c = Case(m, n, k, dtype, sk.A_ROW_B_COL, 12, dist="int")
    ref = c.run(1.0, 0.0, sk.make_options(schedule=sk.SCHED_DP))
    for tile in [sk.TILE_LARGE, sk.TILE_SMALL]:
        for g in [1, 2, 3, 5, 7, 13, 31, 100, 255, 256, 300]:
            c.reset_c()
            got = c.run(1.0, 0.0, sk.make_options(forced_grid=g, tile=tile))
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), (tile, g)
        for sched in (sk.SCHED_DP, sk.SCHED_SK_HYBRID1, sk.SCHED_SK_HYBRID2, sk.SCHED_SK_BASIC,
                      sk.SCHED_XCD_ALIGNED, sk.SCHED_AUTO):
            c.reset_c()
            got = c.run(1.0, 0.0, sk.make_options(schedule=sched, tile=tile))
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), (tile, sched)
    # the fp32 sums are exact, so the one rounding to the output type must
    # give the oracle's rounded value bit for bit
    import oracle
    _, _, rnd = oracle.gemm(m, n, k, 1.0, c.A, c.lda, c.B, c.ldb, 0.0, None, c.ldc, dtype,
                            c.layout)
    assert np.array_equal(ref.view(np.uint8), rnd.view(np.uint8))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("beta", [1.0, -2.0])
def test_beta_nonzero_exact_on_integer_inputs(dtype, beta):
    """beta != 0 (for fp16/bf16 the kernel build that stages alpha*acc
    through LDS in fp32 and reads C in whole lines) on small integers: every
    decomposition on both tile instances gives the oracle's rounded result
    bit for bit (alpha*acc + beta*C is exact in fp32, then rounded once),
    owners adding split tiles' partials included.  The shape has full
    interior tiles and ragged edges on both instances."""
    m, n, k = (700, 600, 1024) if dtype == sk.F32 else (600, 520, 2048)
    c = Case(m, n, k, dtype, sk.A_ROW_B_COL, 17, dist="int")
    import oracle
    _, _, rnd = oracle.gemm(m, n, k, 1.0, c.A, c.lda, c.B, c.ldb, beta, c.Cin, c.ldc, dtype, c.layout)
    for tile in [sk.TILE_LARGE, sk.TILE_SMALL]:
        runs = [sk.make_options(schedule=sched, tile=tile)
                for sched in (sk.SCHED_DP, sk.SCHED_SK_BASIC, sk.SCHED_XCD_ALIGNED, sk.SCHED_AUTO)]
        runs += [sk.make_options(forced_grid=g, tile=tile) for g in (3, 31, 256)]
        for o in runs:
            c.reset_c()
            got = c.run(1.0, beta, o)
            assert np.array_equal(got.view(np.uint8), rnd.view(np.uint8)), (tile, o.schedule, o.forced_grid)


@pytest.mark.parametrize("dtype", DTYPES)
def test_forced_grids_against_oracle(dtype):
    m, n, k = 520, 600, 3000
    c = Case(m, n, k, dtype, sk.A_ROW_B_COL if dtype else sk.A_ROW_B_ROW, 13)
    ref, bound = c.reference(1.0, 1.0)
    for g in [1, 3, 7, 64, 200]:
        _say("case forced grid", dtype, g)
        c.reset_c()
        got = c.run(1.0, 1.0, sk.make_options(forced_grid=g))
        assert rel_err(got, dtype, ref, bound) <= TOL[dtype], g


def test_hybrid_schedule_hgemm_against_oracle():
    """17 x 16 = 272 tiles of 256 x 256: one full wave plus 16 tiles -> the
    two-tile Stream-K + DP hybrid."""
    m, n, k = 256 * 17, 256 * 16, 256
    c = Case(m, n, k, sk.F16, sk.A_ROW_B_COL, 14, dist="normal", scale=1 / 16)
    opts = sk.make_options(schedule=sk.SCHED_SK_HYBRID2)
    p = sk.plan_query(sk.make_desc(m, n, k, 1, c.dA, c.lda, c.dB, c.ldb, 0, c.dC, c.ldc, sk.F16,
                                   sk.A_ROW_B_COL), opts)
    assert p.schedule == sk.SCHED_SK_HYBRID2 and p.max_peers == 1
    got = c.run(1.0, 0.0, opts)
    ref, bound = c.reference()
    assert rel_err(got, sk.F16, ref, bound) <= TOL[sk.F16]
    again = c.run(1.0, 0.0, opts)
    assert np.array_equal(got.view(np.uint8), again.view(np.uint8))  # run-to-run bitwise


def test_auto_hybrid_on_a_long_k_shape_against_oracle():
    """272 tiles with k = 8192: AUTO keeps a Stream-K region of one wave plus
    the 16 leftover tiles, split in XCD lock-step quanta.  Every 128 x 128
    output tile is checked at its first and last rows and columns and two
    more entries, and every split tile at a permutation meeting each of its
    rows and columns (tile_sample_indices); Freivalds as a supplement."""
    m, n, k = 256 * 17, 256 * 16, 8192
    c = Case(m, n, k, sk.BF16, sk.A_ROW_B_COL, 16, dist="normal", scale=1 / np.sqrt(8192),
             with_c=False)
    p = sk.plan_query(sk.make_desc(m, n, k, 1, c.dA, c.lda, c.dB, c.ldb, 0, c.dC, c.ldc, sk.BF16,
                                   sk.A_ROW_B_COL))
    assert p.schedule == sk.SCHED_XCD_ALIGNED and p.sk_tiles == 272 and p.phase_div > 0
    split = split_tiles(p)
    assert len(split) > 0
    got = c.run(1.0, 0.0)
    rows, cols = tile_sample_indices(m, n, 16, split=split, split_tm=p.tile_m, split_tn=p.tile_n,
                                     tiles_n=p.tiles_n)
    ref, bound = c.reference_entries(rows, cols)
    assert sampled_err(got, sk.BF16, rows, cols, ref, bound) <= TOL[sk.BF16]
    assert c.freivalds(got) <= TOL[sk.BF16]


XCD_CASES = [
    # (m, n, k, dtype, layout): a wave or more of tiles (two-tile region plus
    # data-parallel tiles), ragged edges, and below one wave
    (256 * 17, 256 * 16, 256, sk.F16, sk.A_ROW_B_COL),
    (256 * 17 - 37, 256 * 16 - 5, 300, sk.BF16, sk.A_ROW_B_COL),
    (256 * 23, 256 * 24, 192, sk.F16, sk.A_ROW_B_COL),
    (1000, 1000, 5000, sk.F16, sk.A_ROW_B_COL),
    (3000, 2960, 200, sk.F32, sk.A_ROW_B_ROW),
    (128 * 47, 128 * 23, 96, sk.F32, sk.A_COL_B_COL),
    (600, 520, 3000, sk.F32, sk.A_COL_B_ROW),
]


@pytest.mark.parametrize("case", XCD_CASES)
@pytest.mark.parametrize("tile", [sk.TILE_LARGE, sk.TILE_SMALL])
def test_xcd_aligned_schedule_against_oracle(case, tile):
    m, n, k, dtype, layout = case
    _say("case xcd aligned", case, tile)
    c = Case(m, n, k, dtype, layout, 21, dist="normal", scale=1 / np.sqrt(k))
    opts = sk.make_options(schedule=sk.SCHED_XCD_ALIGNED, tile=tile)
    p = sk.plan_query(sk.make_desc(m, n, k, 1, c.dA, c.lda, c.dB, c.ldb, 0, c.dC, c.ldc, dtype,
                                   layout), opts)
    assert p.schedule == sk.SCHED_XCD_ALIGNED and p.sk_tiles > 0
    got = c.run(1.0, 1.0, opts)
    ref, bound = c.reference(1.0, 1.0)
    assert rel_err(got, dtype, ref, bound) <= TOL[dtype]
    c.reset_c()
    again = c.run(1.0, 1.0, opts)
    assert np.array_equal(got.view(np.uint8), again.view(np.uint8))  # run-to-run bitwise


def test_hybrid_schedule_sgemm_against_oracle():
    m, n, k = 128 * 23, 128 * 23, 128  # 529 tiles on 512 slots
    c = Case(m, n, k, sk.F32, sk.A_ROW_B_ROW, 15)
    got = c.run(1.0, 1.0, sk.make_options(schedule=sk.SCHED_SK_HYBRID2))
    ref, bound = c.reference(1.0, 1.0)
    assert rel_err(got, sk.F32, ref, bound) <= TOL[sk.F32]


# ------------------------------------------ full-size workloads (sampled)

@pytest.mark.parametrize("nsq", [1024, 2048, 3072, 4096, 5120, 6144])
def test_sgemm_square_sweep_sampled(nsq):
    """Square SGEMM, row-major, U[-1,1], C_in U[-1,1], alpha=1 beta=1.  Up to
    2n^3 = 2^36 every output element is compared with the oracle; above,
    every 128 x 128 tile at its first and last rows and columns and two more
    entries, plus every split tile of the plan at a permutation meeting each
    of its rows and columns; Freivalds as a supplement."""
    _say("case sgemm square", nsq)
    c = Case(nsq, nsq, nsq, sk.F32, sk.A_ROW_B_ROW, S.SEED_SGEMM_SQUARE)
    got = c.run(1.0, 1.0)
    if 2 * nsq ** 3 <= 2 ** 36:
        ref, bound = c.reference(1.0, 1.0)
        assert rel_err(got, sk.F32, ref, bound) <= TOL[sk.F32]
        return
    p = sk.plan_query(sk.make_desc(nsq, nsq, nsq, 1, c.dA, c.lda, c.dB, c.ldb, 1, c.dC, c.ldc, sk.F32,
                                   sk.A_ROW_B_ROW))
    rows, cols = tile_sample_indices(nsq, nsq, nsq, split=split_tiles(p), split_tm=p.tile_m,
                                     split_tn=p.tile_n, tiles_n=p.tiles_n)
    ref, bound = c.reference_entries(rows, cols, 1.0, 1.0)
    assert sampled_err(got, sk.F32, rows, cols, ref, bound) <= TOL[sk.F32]
    assert c.freivalds(got, 1.0, 1.0) <= TOL[sk.F32]


@pytest.mark.parametrize("dtype", [sk.F16, sk.BF16])
@pytest.mark.parametrize("layout", [sk.A_ROW_B_COL, sk.A_COL_B_ROW])
def test_hgemm_8192_sampled(dtype, layout):
    """8192^3, A row-major and B column-major (both k-contiguous), and A
    column-major and B row-major (both read in place mn-contiguous, through
    transposing LDS reads), entries N(0,1)/sqrt(k), alpha=1 beta=0, fp32
    accumulation.  Every 128 x 128 output tile (4096 of them) is checked at
    its first and last rows and columns and two more entries; Freivalds as a
    supplement."""
    _say("case hgemm 8192", dtype, layout)
    n = 8192
    c = Case(n, n, n, dtype, layout, S.SEED_HGEMM_LARGE, dist="normal",
             scale=1 / np.sqrt(n), with_c=False)
    got = c.run(1.0, 0.0)
    p = sk.plan_query(sk.make_desc(n, n, n, 1, c.dA, c.lda, c.dB, c.ldb, 0, c.dC, c.ldc, dtype, layout))
    assert p.packs == 0
    rows, cols = tile_sample_indices(n, n, 8192 + dtype, split=split_tiles(p), split_tm=p.tile_m,
                                     split_tn=p.tile_n, tiles_n=p.tiles_n)
    ref, bound = c.reference_entries(rows, cols)
    assert sampled_err(got, dtype, rows, cols, ref, bound) <= TOL[dtype]
    assert c.freivalds(got) <= TOL[dtype]


# ------------------------------------------------- Stream-K sweep shapes

# Strata of the 2000-shape fp16 sweep: (kind, AUTO's tile instance, whether
# AUTO keeps a Stream-K region) -> shapes taken.  These are all the kinds of
# plan AUTO resolves to on the sweep (planned for 256 slots, one MI355X).
SWEEP_STRATA = {
    ("random", 128, False): 9, ("random", 128, True): 9,
    ("random", 256, False): 6, ("random", 256, True): 6,
    ("skinny", 128, True): 8, ("skinny", 256, True): 2,
    ("adversarial", 128, False): 6, ("adversarial", 128, True): 4,
    ("adversarial", 256, False): 4, ("adversarial", 256, True): 6,
}
SWEEP_CASES = sum(SWEEP_STRATA.values())
FULL_ORACLE_FLOPS = 2 ** 36  # full output against the oracle up to this 2mnk


@functools.lru_cache(maxsize=1)
def _sweep_subset():
    """A seeded, stratified subset of the sweep: in each stratum, shapes
    drawn at random among those with at most 2.5e7 operand and output
    elements (6e7 in the strata with no such shape; the smallest ones when
    even that leaves too few), so the test's inputs fit in its time."""
    shapes = S.sweep_shapes(2000, S.SEED_SWEEP, 256, 256, 256)
    by = {}
    for kind, m, n, k in shapes:
        p = sk.plan_query(sk.make_desc(m, n, k, 1.0, 0, k, 0, k, 0.0, 0, n, sk.F16, sk.A_ROW_B_COL),
                          None, 256)
        by.setdefault((kind, p.tile_m, p.sk_tiles > 0), []).append((m * k + k * n + m * n, m, n, k))
    out = []
    for si, (key, want) in enumerate(SWEEP_STRATA.items()):
        cands = sorted(by.get(key, []))
        for cap in (2.5e7, 6e7):
            pool = [c for c in cands if c[0] <= cap]
            if len(pool) >= want:
                break
        if len(pool) < want:
            pool = cands[:want]
        order = np.argsort(S.u64(S.SEED_SWEEP, 900 + si, 0, len(pool)), kind="stable")
        out += [(key, pool[i][1], pool[i][2], pool[i][3]) for i in sorted(order[:want])]
    return out


PAGE_SCHEDULES = [sk.SCHED_SK_HYBRID2, sk.SCHED_SK_HYBRID1, sk.SCHED_SK_BASIC]


@pytest.mark.parametrize("idx", range(SWEEP_CASES))
def test_sweep_shapes_against_oracle(idx):
    """One shape of the stratified sweep subset, fp16, A row-major, B
    column-major, N(0,1)/sqrt(k), alpha=1 beta=0, run under AUTO, data-parallel
    on the large tile, AUTO with the small tile, and one of the page's
    schedules (two-tile hybrid, one-tile hybrid, basic Stream-K, in turn, on
    either instance).  With 2mnk <= 2^36 every output element of every run
    is compared with the oracle; above that, every 128 x 128 output tile is
    checked at its first and last rows and columns and two more entries, and
    every tile the run's plan splits over workgroups at a permutation that
    meets each of its rows and columns (tile_sample_indices); Freivalds'
    check runs beside it as a supplement only."""
    key, m, n, k = _sweep_subset()[idx]
    _say("case sweep", idx, key, m, n, k)
    c = Case(m, n, k, sk.F16, sk.A_ROW_B_COL, S.SEED_SWEEP + m + n + k, dist="normal",
             scale=1 / np.sqrt(k), with_c=False)
    runs = [sk.make_options(), sk.make_options(schedule=sk.SCHED_DP, tile=sk.TILE_LARGE),
            sk.make_options(tile=sk.TILE_SMALL),
            sk.make_options(schedule=PAGE_SCHEDULES[idx % 3],
                            tile=(sk.TILE_LARGE, sk.TILE_SMALL)[(idx // 3) % 2])]
    full = 2 * m * n * k <= FULL_ORACLE_FLOPS
    plans = []
    for o in runs:
        plans.append(sk.plan_query(sk.make_desc(m, n, k, 1.0, c.dA, c.lda, c.dB, c.ldb, 0.0, c.dC, c.ldc,
                                                sk.F16, sk.A_ROW_B_COL), o))
    assert (plans[0].tile_m, plans[0].sk_tiles > 0) == key[1:], (plans[0].tile_m, plans[0].sk_tiles)
    if full:
        ref, bound = c.reference()
    else:
        rr, cc = [], []
        for i, p in enumerate(plans):
            r, q = tile_sample_indices(m, n, m + 3 * n + i, split=split_tiles(p), split_tm=p.tile_m,
                                       split_tn=p.tile_n, tiles_n=p.tiles_n)
            rr.append(r)
            cc.append(q)
        lin = np.unique(np.concatenate(rr) * n + np.concatenate(cc))
        rows, cols = lin // n, lin % n
        ref, bound = c.reference_entries(rows, cols)
    for o, p in zip(runs, plans):
        got = c.run(1.0, 0.0, o)
        if full:
            err = rel_err(got, sk.F16, ref, bound)
        else:
            err = sampled_err(got, sk.F16, rows, cols, ref, bound)
            assert c.freivalds(got) <= TOL[sk.F16]
        assert err <= TOL[sk.F16], (key, m, n, k, p.schedule, p.tile_m, err)


# ------------------------------------------------ matrix-vector products

def _gemv_cases(dtype):
    """(m, n, k, layout, pad, alpha, beta): pad makes the matrix rows 16-byte
    aligned for a ragged k (and strides C for n == 1)."""
    vec = 4 if dtype == sk.F32 else 8
    out = []
    for k in (1, 5, 8, 64, 1000, 4097, 65539):
        pad = (-k) % vec
        for r in ((1, 7, 300, 4099) if k <= 4097 else (1, 7, 300)):
            out.append((1, r, k, sk.A_ROW_B_COL, pad, 1.0, 0.0))
            out.append((r, 1, k, sk.A_ROW_B_COL, pad + vec, 0.5, -1.5))
    for k in (8, 2048, 30000 - 30000 % vec):
        out.append((1, 513, k, sk.A_COL_B_COL, 0, 1.0, 1.0))
        out.append((513, 1, k, sk.A_ROW_B_ROW, 0, -2.0, 0.25))
    return out


@pytest.mark.parametrize("dtype", DTYPES)
def test_matrix_vector_split_against_oracle(dtype):
    """m == 1 and n == 1 products go to the even split of dot products (one
    chunk or many, k tails, strided C, alpha/beta, all operand orders the
    path takes) and match the oracle; repeated calls are bitwise equal."""
    for (m, n, k, layout, pad, alpha, beta) in _gemv_cases(dtype):
        _say("case gemv", dtype, m, n, k, layout, pad)
        c = Case(m, n, k, dtype, layout, 11 + m + 3 * n + k, pad=pad)
        d = sk.make_desc(m, n, k, alpha, c.dA, c.lda, c.dB, c.ldb, beta, c.dC, c.ldc, dtype, layout)
        assert sk.plan_query(d).schedule == sk.SCHED_GEMV_SPLIT, (m, n, k, layout)
        got = c.run(alpha, beta)
        ref, bound = c.reference(alpha, beta)
        assert rel_err(got, dtype, ref, bound) <= TOL[dtype], (m, n, k, layout)
        c.reset_c()
        again = c.run(alpha, beta, sk.make_options(schedule=sk.SCHED_GEMV_SPLIT))
        assert np.array_equal(got.view(np.uint8), again.view(np.uint8))


@pytest.mark.parametrize("dtype", DTYPES)
def test_matrix_vector_fallback_and_beta_zero(dtype):
    """Unaligned rows fall back to the tiled kernels (AUTO) or are refused
    (explicit split); beta == 0 never reads C."""
    c = Case(1, 300, 1001, dtype, sk.A_ROW_B_COL, 3, pad=2 if dtype == sk.F32 else 1)
    d = sk.make_desc(1, 300, 1001, 1.0, c.dA, c.lda, c.dB, c.ldb, 0.0, c.dC, c.ldc, dtype,
                     sk.A_ROW_B_COL)
    assert sk.plan_query(d).schedule != sk.SCHED_GEMV_SPLIT
    assert sk.gemm_ex(d, sk.make_options(schedule=sk.SCHED_GEMV_SPLIT), check=False) == \
        sk.ERR_UNSUPPORTED
    got = c.run(1.0, 0.0)
    ref, bound = c.reference(1.0, 0.0)
    assert rel_err(got, dtype, ref, bound) <= TOL[dtype]
    c = Case(5000, 1, 4096, dtype, sk.A_ROW_B_COL, 4)
    c.dC.fill_(float("nan"))
    got = c.run(1.0, 0.0)
    ref, bound = c.reference(1.0, 0.0)
    assert rel_err(got, dtype, ref, bound) <= TOL[dtype]


@pytest.mark.parametrize("dtype,m,n,k", [(sk.F32, 1, 1, 1 << 21), (sk.F32, 3, 1, 1 << 20),
                                         (sk.BF16, 1, 2, 1 << 21)])
def test_matrix_vector_long_dot_products(dtype, m, n, k):
    """Few, long dot products: hundreds of chunks per output, added by a
    workgroup per output; two calls agree bitwise."""
    _say("case gemv long", dtype, m, n, k)
    c = Case(m, n, k, dtype, sk.A_ROW_B_COL, 31 + m + n, with_c=False)
    d = sk.make_desc(m, n, k, 1.0, c.dA, c.lda, c.dB, c.ldb, 0.0, c.dC, c.ldc, dtype, sk.A_ROW_B_COL)
    assert sk.plan_query(d).sk_blocks >= 512
    got = c.run(1.0, 0.0)
    ref, bound = c.reference(1.0, 0.0)
    assert rel_err(got, dtype, ref, bound) <= TOL[dtype]
    again = c.run(1.0, 0.0)
    assert np.array_equal(got.view(np.uint8), again.view(np.uint8))


@pytest.mark.parametrize("dtype,m,n,k", [(sk.F32, 1, 16384, 4096), (sk.F16, 16384, 1, 4096),
                                         (sk.BF16, 1, 4096, 16384)])
def test_matrix_vector_large(dtype, m, n, k):
    """A 16384 x 4096 matrix against a vector (one chunk per dot product, or
    two when the rows are fewer and longer), against the oracle on every
    output."""
    _say("case gemv large", dtype, m, n, k)
    c = Case(m, n, k, dtype, sk.A_ROW_B_COL, 21 + m, with_c=False)
    got = c.run(1.0, 0.0)
    ref, bound = c.reference(1.0, 0.0)
    assert rel_err(got, dtype, ref, bound) <= TOL[dtype]


def _axpy_cases(dtype):
    """(m, n, k, layout, pad, alpha, beta) with the matrix operand contiguous
    along the output: pad aligns its rows to 16 bytes and also strides the
    vector (column-major A for m == 1, row-major B for n == 1) and C."""
    vec = 4 if dtype == sk.F32 else 8
    out = []
    for k in (1, 5, 64, 1000, 4097):
        for r in ((1, 7, 300, 4099, 20000) if k <= 1000 else (1, 7, 300, 4099)):
            pad = (-r) % vec
            out.append((1, r, k, sk.A_ROW_B_ROW, pad, 1.0, 0.0))
            out.append((r, 1, k, sk.A_COL_B_COL, pad + vec, 0.5, -1.5))
    for k in (8, 2048):
        out.append((1, 513, k, sk.A_COL_B_ROW, (-513) % vec, 1.0, 1.0))
        out.append((513, 1, k, sk.A_COL_B_ROW, (-513) % vec, -2.0, 0.25))
    return out


@pytest.mark.parametrize("dtype", DTYPES)
def test_matrix_vector_output_contiguous_against_oracle(dtype):
    """m == 1 with B row-major and n == 1 with A column-major take the axpy
    form (blocks of outputs over chunks of k rows; strided vectors and C,
    alpha/beta, ragged output lengths) and match the oracle; repeated calls
    are bitwise equal."""
    for (m, n, k, layout, pad, alpha, beta) in _axpy_cases(dtype):
        _say("case gemv axpy", dtype, m, n, k, layout, pad)
        c = Case(m, n, k, dtype, layout, 13 + m + 5 * n + k, pad=pad)
        d = sk.make_desc(m, n, k, alpha, c.dA, c.lda, c.dB, c.ldb, beta, c.dC, c.ldc, dtype, layout)
        p = sk.plan_query(d)
        # a single output may take either form
        assert p.schedule == sk.SCHED_GEMV_SPLIT and (p.tile_n > 0 or m == n == 1), (m, n, k, layout)
        got = c.run(alpha, beta)
        ref, bound = c.reference(alpha, beta)
        assert rel_err(got, dtype, ref, bound) <= TOL[dtype], (m, n, k, layout)
        c.reset_c()
        again = c.run(alpha, beta, sk.make_options(schedule=sk.SCHED_GEMV_SPLIT))
        assert np.array_equal(got.view(np.uint8), again.view(np.uint8))


@pytest.mark.parametrize("dtype,m,n,k,layout", [(sk.F16, 1, 16384, 4096, sk.A_ROW_B_ROW),
                                                (sk.F32, 8192, 1, 8192, sk.A_COL_B_COL),
                                                (sk.BF16, 1, 1, 1 << 20, sk.A_ROW_B_ROW)])
def test_matrix_vector_output_contiguous_large(dtype, m, n, k, layout):
    """Large axpy-form products (one output block over many row chunks, or
    many blocks) against the oracle on every output."""
    _say("case gemv axpy large", dtype, m, n, k, layout)
    c = Case(m, n, k, dtype, layout, 41 + m, with_c=False)
    got = c.run(1.0, 0.0)
    ref, bound = c.reference(1.0, 0.0)
    assert rel_err(got, dtype, ref, bound) <= TOL[dtype]


def _multi_cases(dtype):
    """(m, n, k, pad, alpha, beta): 2 .. 16 vectors (fp16/bf16: 8; m, or n
    with m > 16) against k-contiguous rows (A row-major, B column-major); pad
    aligns the rows for a ragged k and strides C."""
    vec = 4 if dtype == sk.F32 else 8
    out = []
    for k in (1, 5, 31, 64, 1000, 4097):
        pad = (-k) % vec
        for V in ((2, 5, 16) if dtype == sk.F32 else (2, 5, 8)):
            for R in ((7, 4099) if k <= 1000 else (300,)):
                out.append((V, R, k, pad, 1.0, 0.0))
                out.append((R + 16, V, k, pad + vec, 0.5, -1.5))
    return out


@pytest.mark.parametrize("dtype", DTYPES)
def test_matrix_vector_few_vectors_against_oracle(dtype):
    """A few vectors against k-contiguous rows take the multi form (MFMA
    over row blocks and k-chunks; k tails, rows and vectors past the end,
    strided C, alpha/beta) and match the oracle; repeated calls are bitwise
    equal."""
    for (m, n, k, pad, alpha, beta) in _multi_cases(dtype):
        _say("case gemv multi", dtype, m, n, k, pad)
        c = Case(m, n, k, dtype, sk.A_ROW_B_COL, 17 + m + 3 * n + k, pad=pad)
        d = sk.make_desc(m, n, k, alpha, c.dA, c.lda, c.dB, c.ldb, beta, c.dC, c.ldc, dtype, sk.A_ROW_B_COL)
        p = sk.plan_query(d)
        assert p.schedule == sk.SCHED_GEMV_SPLIT and p.tile_n == (64 if dtype == sk.F32 else 16), (m, n, k)
        got = c.run(alpha, beta)
        ref, bound = c.reference(alpha, beta)
        assert rel_err(got, dtype, ref, bound) <= TOL[dtype], (m, n, k)
        c.reset_c()
        again = c.run(alpha, beta, sk.make_options(schedule=sk.SCHED_GEMV_SPLIT))
        assert np.array_equal(got.view(np.uint8), again.view(np.uint8))


@pytest.mark.parametrize("dtype,m,n,k", [(sk.F16, 8, 16384, 4096), (sk.BF16, 16384, 4, 4096),
                                         (sk.F32, 16, 8192, 4096), (sk.F32, 3, 5, 1 << 20)])
def test_matrix_vector_few_vectors_large(dtype, m, n, k):
    """Large multi-form products against the oracle on every output."""
    _say("case gemv multi large", dtype, m, n, k)
    c = Case(m, n, k, dtype, sk.A_ROW_B_COL, 51 + m, with_c=False)
    got = c.run(1.0, 0.0)
    ref, bound = c.reference(1.0, 0.0)
    assert rel_err(got, dtype, ref, bound) <= TOL[dtype]
