"""C-ABI tests that need no GPU: exported symbols, the planner (against the
oracle's independent decompositions and the Stream-K page's rules) and the
argument checks that return before any HIP call."""
import ctypes

import numpy as np
import pytest

import oracle
import work_centric_decomposition_amd as sk


def test_every_declared_function_is_exported():
    names = sk.header_functions()
    assert {"sk_gemm", "sk_gemm_ex", "sk_plan_query", "sk_plan_segments", "sk_strerror",
            "sk_release_workspace", "sk_device_status"} <= set(names)
    lib = sk.library()
    for name in names:
        assert hasattr(lib, name), name


def _desc(m, n, k, dtype=sk.F16, layout=sk.A_ROW_B_COL):
    # aligned fake pointers: the planner only inspects their alignment
    return sk.make_desc(m, n, k, 1.0, 1 << 20, k if layout in (0, 1) else m, 1 << 21,
                        k if layout in (1, 3) else n, 0.0, 1 << 22, n, dtype, layout)


def _lib_plan_records(plan):
    rec = []
    for x in range(plan.grid):
        for s in sk.plan_segments(plan, x):
            rec.append((x,) + tuple(int(v) for v in s))
    return rec


def _oracle_records(m, n, k, bm, bn, bk, mode, param):
    rec, _ = oracle.sk_plan(m, n, k, bm, bn, bk, mode, param)
    return [tuple(int(v) for v in r) for r in rec]


SHAPES = [(384, 384, 128), (8192, 8192, 8192), (6144, 6144, 6144), (1000, 3000, 777),
          (128, 16384, 16384), (4096, 5120, 1024), (256 * 17, 256, 4096), (1, 1, 1),
          (3000, 200, 64)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [sk.F16, sk.F32])
@pytest.mark.parametrize("slots", [256, 512, 7])
def test_auto_plan_matches_oracle_decomposition(shape, dtype, slots):
    m, n, k = shape
    d = _desc(m, n, k, dtype)
    p = sk.plan_query(d, None, slots)
    t, ipt = p.tiles, p.iters_per_tile
    assert t == -(-m // p.tile_m) * -(-n // p.tile_n) and ipt == -(-k // p.tile_k)
    w, r = t // slots, t % slots
    assert (p.full_waves, p.tail_tiles) == (w, r)
    if r == 0:
        assert p.schedule == sk.SCHED_DP and p.sk_tiles == 0
        mode, param = oracle.DP_PERSISTENT, p.grid
    elif w >= 1 and p.schedule == sk.SCHED_SK_HYBRID2:
        assert p.grid == slots and p.sk_tiles == r + slots
        mode, param = oracle.HYBRID2, slots
    elif w >= 1:
        # the model judged the hybrid's fixup too costly for this k
        assert p.schedule == sk.SCHED_DP and p.sk_tiles == 0
        mode, param = oracle.DP_PERSISTENT, p.grid
    else:
        assert p.schedule in (sk.SCHED_SK_BASIC,) and t <= p.grid <= slots
        mode, param = oracle.SK, p.grid
    got = _lib_plan_records(p)
    want = _oracle_records(m, n, k, p.tile_m, p.tile_n, p.tile_k, mode, param)
    assert got == want


@pytest.mark.parametrize("shape", SHAPES[:6])
def test_forced_grid_and_explicit_schedules_match_oracle(shape):
    m, n, k = shape
    d = _desc(m, n, k, sk.F32, sk.A_ROW_B_ROW)
    for g in (1, 3, 4, 100, 256, 600):
        p = sk.plan_query(d, sk.make_options(forced_grid=g), 256)
        assert p.schedule == sk.SCHED_SK_BASIC and p.grid == g
        assert _lib_plan_records(p) == _oracle_records(m, n, k, p.tile_m, p.tile_n, p.tile_k,
                                                       oracle.SK, g)
    p = sk.plan_query(d, sk.make_options(schedule=sk.SCHED_SK_HYBRID1), 256)
    assert _lib_plan_records(p) == _oracle_records(m, n, k, p.tile_m, p.tile_n, p.tile_k,
                                                   oracle.HYBRID1, 256)
    p = sk.plan_query(d, sk.make_options(schedule=sk.SCHED_DP), 256)
    assert _lib_plan_records(p) == _oracle_records(m, n, k, p.tile_m, p.tile_n, p.tile_k,
                                                   oracle.DP_PERSISTENT, min(256, p.tiles))


def test_forced_grid_equal_tiles_is_data_parallel_plan():
    d = _desc(8192, 8192, 8192, sk.F16)
    p = sk.plan_query(d, sk.make_options(forced_grid=1024), 256)
    recs = _lib_plan_records(p)
    assert all(r[2] == 0 and r[3] == p.iters_per_tile and r[6] == -1 for r in recs)
    assert [r[1] for r in recs] == list(range(1024))


def test_page_example_plan_through_the_library():
    """Section 4 worked example scaled to this kernel's BLK_K: 384x384x128
    SGEMM on a grid of 4 gives equal shares and three fixups."""
    d = _desc(384, 384, 128, sk.F32, sk.A_ROW_B_ROW)
    p = sk.plan_query(d, sk.make_options(forced_grid=4), 512)
    assert p.tiles == 9 and p.iters_per_tile == 4 and p.total_iters == 36
    work = [sum(s[2] - s[1] for s in sk.plan_segments(p, x)) for x in range(4)]
    assert work == [9, 9, 9, 9]
    partials = sum(1 for x in range(4) for s in sk.plan_segments(p, x) if not s[3])
    assert partials == 3


def test_auto_takes_the_hybrid_only_when_k_pays_for_the_fixup():
    """t = 272 tiles on 256 slots: the hybrid saves 15/16 of a tile's
    iterations per workgroup, which beats one partial + one peer only when
    the tile has enough iterations."""
    short = sk.plan_query(_desc(256 * 17, 256 * 16, 256), None, 256)
    long_ = sk.plan_query(_desc(256 * 17, 256 * 16, 8192), None, 256)
    assert short.schedule == sk.SCHED_DP and long_.schedule == sk.SCHED_SK_HYBRID2


def test_two_tile_hybrid_owner_has_one_peer():
    for t_m, t_n in [(17, 17), (23, 12), (16, 17)]:
        d = _desc(256 * t_m, 256 * t_n, 4096, sk.F16)
        p = sk.plan_query(d, None, 256)
        assert p.schedule == sk.SCHED_SK_HYBRID2 and p.max_peers == 1


def test_grid_model_regimes():
    """Qualitative behaviour of the appendix A.1 model (Fig. 8): large-k
    short-wide shapes use every slot, a medium-k 64-tile shape stays at the
    tile count, a single tile with a huge k stops at a small grid."""
    model = (4.0, 2.0, 1.0, 2.0)
    # T(g) ~ c*I/g + d*g/t is minimised near sqrt(c*I*t/d); with t = 16 tiles
    # and I = 16 * 1024 iterations that lies beyond the 256 slots
    p = sk.plan_query(_desc(256, 256 * 16, 65536), sk.make_options(model=model), 256)
    assert p.grid == 256
    # 64 tiles of 4 iterations: splitting saves at most 2 iterations per
    # workgroup but costs b + d = 4
    p = sk.plan_query(_desc(256 * 8, 256 * 8, 256), sk.make_options(model=model), 256)
    assert p.grid == 64
    p = sk.plan_query(_desc(256, 256, 64 * 128), sk.make_options(model=model), 256)
    assert 1 < p.grid <= 16


def test_repack_flags():
    p = sk.plan_query(_desc(1000, 1000, 1000, sk.F16, sk.A_ROW_B_ROW), None, 256)
    assert p.packs == 2  # B is n-contiguous: repacked for the fp16 kernel
    p = sk.plan_query(_desc(1000, 1000, 1000, sk.F32, sk.A_COL_B_ROW), None, 256)
    assert p.packs == 0  # the fp32 kernel reads both orders directly
    p = sk.plan_query(_desc(1000, 1000, 1001, sk.F16, sk.A_ROW_B_COL), None, 256)
    assert p.packs == 3  # k not a multiple of 8


def test_invalid_arguments_are_rejected_before_any_gpu_call():
    assert sk.gemm(-1, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 16, 4, sk.F32, 0, stream=0,
                   check=False) == sk.ERR_INVALID_ARG
    assert sk.gemm(4, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 16, 4, 7, 0, stream=0,
                   check=False) == sk.ERR_INVALID_ARG
    assert sk.gemm(4, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 16, 4, sk.F32, 9, stream=0,
                   check=False) == sk.ERR_INVALID_ARG
    # m == 0 / n == 0: nothing to do, even with null pointers
    assert sk.gemm(0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, sk.F32, 0, stream=0,
                   check=False) == sk.OK
    d = sk.make_desc(8, 8, 8, 1.0, 16, 8, 16, 8, 0.0, 16, 8, sk.F16, 0)
    assert sk.gemm_ex(d, sk.make_options(abft=True), report=16, stream=0,
                      check=False) == sk.ERR_UNSUPPORTED
    d = sk.make_desc(8, 8, 8, 1.0, 16, 8, 16, 8, 0.0, 16, 8, sk.F32, 0)
    assert sk.gemm_ex(d, sk.make_options(abft=True), report=None, stream=0,
                      check=False) == sk.ERR_INVALID_ARG
    assert sk.gemm(8, 8, 8, 1.0, 16, 7, 16, 8, 0.0, 16, 8, sk.F32, 0, stream=0,
                   check=False) == sk.ERR_INVALID_ARG  # lda < k


def test_strerror_texts():
    assert sk.strerror(0) == "success"
    assert "time" in sk.strerror(sk.ERR_FIXUP_TIMEOUT)
    assert sk.version().startswith("sk_gemm")
    assert ctypes.sizeof(sk.AbftReport) == 16 + 64 * ctypes.sizeof(sk.AbftRecord)
