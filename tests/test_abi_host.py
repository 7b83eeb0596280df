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


def test_measurement_library_exports_what_its_header_declares():
    """libskmb.so (the machine-peak kernels bench.py reports against) loads
    without a GPU and exports every function include/sk_microbench.h
    declares; invalid sizes are refused before any launch."""
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(sk.HEADER_PATH), "sk_microbench.h")).read()
    names = re.findall(r"^int (skmb_\w+)\(", hdr, re.M)
    assert set(names) == {"skmb_mfma", "skmb_read", "skmb_lds"}
    mb = ctypes.CDLL(os.path.join(os.path.dirname(sk.LIB_PATH), "libskmb.so"))
    for name in names:
        assert hasattr(mb, name), name
    mb.skmb_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    mb.skmb_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert mb.skmb_mfma(3, 10, 1, 16, None) != 0  # unknown type
    assert mb.skmb_mfma(1, 0, 1, 16, None) != 0   # no rounds
    assert mb.skmb_read(16, 24, 1, 16, None) != 0  # not a multiple of 16 bytes
    mb.skmb_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert mb.skmb_lds(2, 10, 1, 16, None) != 0  # unknown mode
    assert mb.skmb_lds(0, 0, 1, 16, None) != 0   # no rounds


def test_calls_fail_loudly_without_the_library():
    """With libskgemm.so absent, importing the package still works (the build
    needs that) but the first call through the ABI raises ImportError: there
    is no fallback path.  Run in a fresh interpreter so that this process's
    loaded library is not reused."""
    import os
    import subprocess
    import sys
    code = ("import work_centric_decomposition_amd as sk\n"
            "sk.LIB_PATH = '/nonexistent/libskgemm.so'\n"
            "d = sk.make_desc(8, 8, 8, 1.0, 16, 8, 16, 8, 0.0, 16, 8, sk.F32, 0)\n"
            "try:\n"
            "    sk.plan_query(d, None, 256)\n"
            "except ImportError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('no error')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert "raised:" in out.stdout and "is not built" in out.stdout, out.stdout + out.stderr


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


def _check_schedule(p):
    """Invariants every schedule must keep: each (tile, k-iteration) is
    covered exactly once; the segment holding a tile's k = 0 iteration is its
    owner and, when it does not also hold the last iteration, adds the
    partials of exactly workgroups owner+1 .. last_peer, which cover the rest
    of the tile; a partial is always its workgroup's first segment (so an
    owner never waits on a peer that must first finish other work)."""
    t, ipt = p.tiles, p.iters_per_tile
    cover = {}
    for x in range(p.grid):
        segs = sk.plan_segments(p, x)
        for i, (tile, lb, le, st, en, lp) in enumerate(segs):
            assert 0 <= lb < le <= ipt
            assert st == (lb == 0) and en == (le == ipt)
            if not st:
                assert i == 0, (x, segs)
            cover.setdefault(tile, []).append((lb, le, x, st, en, lp))
    assert sorted(cover) == list(range(t))
    for tile, segs in cover.items():
        segs.sort()
        assert segs[0][0] == 0 and segs[-1][1] == ipt
        assert all(a[1] == b[0] for a, b in zip(segs, segs[1:])), (tile, segs)
        owner = segs[0]
        peers = sorted(s_[2] for s_ in segs[1:])
        if owner[4]:
            assert peers == [] and owner[5] == -1
        else:
            assert peers == list(range(owner[2] + 1, owner[5] + 1)), (tile, segs)


TILES = [sk.TILE_LARGE, sk.TILE_SMALL]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [sk.F16, sk.F32])
@pytest.mark.parametrize("slots", [256, 512, 8])
@pytest.mark.parametrize("tile", TILES)
def test_page_schedules_match_oracle_decomposition(shape, dtype, slots, tile):
    """The page's decompositions, chosen explicitly, against the oracle's own
    construction of Algorithms 2 and 5 and section 5.2's hybrids (both fp16
    tile instances of each type; the small one runs two workgroups per
    large-tile slot)."""
    m, n, k = shape
    d = _desc(m, n, k, dtype)
    for sched, mode in [(sk.SCHED_DP, oracle.DP_PERSISTENT), (sk.SCHED_SK_BASIC, oracle.SK),
                        (sk.SCHED_SK_HYBRID2, oracle.HYBRID2), (sk.SCHED_SK_HYBRID1, oracle.HYBRID1)]:
        p = sk.plan_query(d, sk.make_options(schedule=sched, tile=tile), slots)
        assert p.slots == (2 * slots if tile == sk.TILE_SMALL else slots)
        large, small = (128, 64) if dtype == sk.F32 else (256, 128)
        assert p.tile_m == p.tile_n == (small if tile == sk.TILE_SMALL else large)
        slots = p.slots
        t, ipt = p.tiles, p.iters_per_tile
        assert t == -(-m // p.tile_m) * -(-n // p.tile_n) and ipt == -(-k // p.tile_k)
        w, r = t // slots, t % slots
        assert (p.full_waves, p.tail_tiles) == (w, r)
        assert p.group_rows == 0 and p.phase_div == 0 and p.fixup_tree == 0
        if sched == sk.SCHED_SK_HYBRID2 and (w < 1 or r == 0):
            continue  # resolved to another schedule (checked below)
        if sched == sk.SCHED_DP:
            param = p.grid
        elif sched == sk.SCHED_SK_BASIC:
            assert min(t, slots) <= p.grid <= slots
            param = p.grid
        else:
            param = slots
        assert p.schedule == sched
        want = _oracle_records(m, n, k, p.tile_m, p.tile_n, p.tile_k, mode, param)
        assert _lib_plan_records(p) == want
        _check_schedule(p)


@pytest.mark.parametrize("shape", SHAPES + [(4352, 4096, 4096), (9392, 2976, 14144), (3808, 4624, 720),
                                            (2048, 2048, 8192), (512, 512, 30000), (256 * 17, 256 * 16, 256)])
@pytest.mark.parametrize("dtype", [sk.F16, sk.F32])
@pytest.mark.parametrize("slots", [256, 512, 8])
@pytest.mark.parametrize("tile", TILES)
def test_auto_xcd_aligned_schedule_invariants(shape, dtype, slots, tile):
    m, n, k = shape
    d = _desc(m, n, k, dtype)
    p = sk.plan_query(d, sk.make_options(tile=tile), slots)
    slots = p.slots
    assert p.schedule == sk.SCHED_XCD_ALIGNED and p.group_rows == 8
    t, w, r = p.tiles, p.tiles // slots, p.tiles % slots
    if w >= 1 and r == 0:
        assert p.sk_tiles == 0 and p.grid == slots
    if p.sk_tiles:
        D, s = p.phase_div, p.sk_blocks
        assert D % 8 == 0 and slots % D == 0 and s >= 1
        assert p.sk_tiles in (t, slots + r)
        assert p.grid <= slots and p.grid % 8 == 0
        assert (p.sk_iters_q, p.sk_iters_r) == divmod(s * p.iters_per_tile, D)
        if w >= 1:
            assert p.grid == slots and s >= D and p.max_peers <= 1
    else:
        assert p.phase_div == 0 and p.grid == min(t, slots)
    _check_schedule(p)
    for x in range(p.grid):
        assert sum(e - b for _, b, e, *_ in sk.plan_segments(p, x)) <= \
            (-(-p.sk_blocks * p.iters_per_tile // p.phase_div) if p.sk_tiles else 0) + \
            -(-(t - p.sk_tiles) // p.grid) * p.iters_per_tile


@pytest.mark.parametrize("tiles", [(17, 16), (20, 15), (9, 9), (33, 9), (16, 16), (24, 11)])
@pytest.mark.parametrize("slots", [256, 512])
def test_xcd_aligned_data_parallel_waves_spread_over_all_xcds(tiles, slots):
    """Each data-parallel wave, the partial last one too, gives the eight
    XCDs (workgroups x with equal x mod 8) runs of consecutive tiles whose
    lengths differ by at most one."""
    t_m, t_n = tiles
    d = _desc(256 * t_m, 256 * t_n, 64 * 8, sk.F16)
    p = sk.plan_query(d, None, slots)
    # short k: AUTO keeps a partial last wave data-parallel
    assert p.schedule == sk.SCHED_XCD_ALIGNED and p.sk_tiles == 0 and p.group_rows == 8
    waves = -(-p.tiles // p.grid)
    per_wave = [[[] for _ in range(8)] for _ in range(waves)]
    for x in range(p.grid):
        segs = sk.plan_segments(p, x)
        assert len(segs) in (waves - 1, waves)
        for wave, (tile, lb, le, st, en, lp) in enumerate(segs):
            assert (lb, le, lp) == (0, p.iters_per_tile, -1)
            per_wave[wave][x % 8].append(tile)
    for runs in per_wave:
        sizes = [len(r) for r in runs]
        assert max(sizes) - min(sizes) <= 1, sizes
    _check_schedule(p)


@pytest.mark.parametrize("shape", [(4352, 4096, 4096), (9392, 2976, 14144), (3808, 4624, 720),
                                   (2048, 2048, 8192), (1024, 6144, 4096), (6000, 5000, 3000)])
def test_xcd_aligned_workgroups_of_one_class_run_in_lock_step(shape):
    """Workgroups x and x + D (D = phase_div, a multiple of 8, so both sit on
    the same XCD) start at the same k offset and cross tile boundaries at the
    same times: their Stream-K segments have identical k ranges, and at every
    step they work on tiles of one 8-row band."""
    m, n, k = shape
    p = sk.plan_query(_desc(m, n, k), sk.make_options(schedule=sk.SCHED_XCD_ALIGNED), 256)
    assert p.sk_tiles > 0
    D = p.phase_div
    J = -(-p.sk_tiles // p.sk_blocks)
    region = p.sk_tiles * p.iters_per_tile
    for c in range(D):
        members = [c + D * j for j in range(J) if c + D * j < p.grid]
        full = [x for x in members
                if (x + 1) * p.sk_blocks * p.iters_per_tile // D <= region]
        shapes = {tuple((b, e) for _, b, e, *_ in sk.plan_segments(p, x)[:_n_sk(p, x)]) for x in full}
        assert len(shapes) == 1, (c, shapes)
        # tiles processed at the same step: contiguous block of the band order
        nseg = _n_sk(p, full[0])
        for i in range(nseg):
            tiles = [sk.plan_segments(p, x)[i][0] for x in full]
            rows = {tl // p.tiles_n for tl in tiles}
            cols = {tl % p.tiles_n for tl in tiles}
            assert len(rows) + len(cols) <= len(tiles) // 2 + 10, (c, i, rows, cols)


def _n_sk(p, x):
    """Number of Stream-K segments of workgroup x (the rest are whole tiles
    dealt after the region)."""
    b = x * p.sk_blocks * p.iters_per_tile // p.phase_div
    e = min((x + 1) * p.sk_blocks * p.iters_per_tile // p.phase_div, p.sk_tiles * p.iters_per_tile)
    if e <= b:
        return 0
    return (e - 1) // p.iters_per_tile - b // p.iters_per_tile + 1


@pytest.mark.parametrize("shape", SHAPES[:6])
def test_forced_grid_and_explicit_schedules_match_oracle(shape):
    m, n, k = shape
    d = _desc(m, n, k, sk.F32, sk.A_ROW_B_ROW)
    for g in (1, 3, 4, 100, 256, 600):
        p = sk.plan_query(d, sk.make_options(forced_grid=g), 256)
        assert p.schedule == sk.SCHED_SK_BASIC and p.grid == g
        assert _lib_plan_records(p) == _oracle_records(m, n, k, p.tile_m, p.tile_n, p.tile_k,
                                                       oracle.SK, g)
    # explicit schedules on either instance (AUTO tile may pick the small
    # one, whose slot count is twice the large one's)
    p = sk.plan_query(d, sk.make_options(schedule=sk.SCHED_SK_HYBRID1), 256)
    assert _lib_plan_records(p) == _oracle_records(m, n, k, p.tile_m, p.tile_n, p.tile_k,
                                                   oracle.HYBRID1, p.slots)
    p = sk.plan_query(d, sk.make_options(schedule=sk.SCHED_DP), 256)
    assert _lib_plan_records(p) == _oracle_records(m, n, k, p.tile_m, p.tile_n, p.tile_k,
                                                   oracle.DP_PERSISTENT, min(p.slots, p.tiles))


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


def test_auto_keeps_the_stream_k_region_only_when_k_pays_for_the_fixup():
    """t = 272 tiles on 256 slots: the region saves most of a tile's
    iterations per workgroup, which beats one partial + one peer only when
    the tile has enough iterations."""
    short = sk.plan_query(_desc(256 * 17, 256 * 16, 256), None, 256)
    long_ = sk.plan_query(_desc(256 * 17, 256 * 16, 8192), None, 256)
    assert short.schedule == long_.schedule == sk.SCHED_XCD_ALIGNED
    assert short.sk_tiles == 0 and long_.sk_tiles == 272 and long_.grid == 256


def _simulate_tree_fixup(p):
    """Runs the binary-tree combine of sk_gemm.h (fixup_tree) over the plan's
    segments on sets of (workgroup, tile) pieces: every owner must end with
    each piece of its tile exactly once, every stored partial must be
    consumed exactly once, and a workgroup may only wait for a higher one."""
    t, ipt = p.tiles, p.iters_per_tile
    pieces_of = {}
    for x in range(p.grid):
        for tile, lb, le, st, en, lp in sk.plan_segments(p, x):
            pieces_of.setdefault(tile, []).append((lb, x))
    owners = {}
    for tile, lst in pieces_of.items():
        lst.sort()
        xs = [x for _, x in lst]
        assert xs == list(range(xs[0], xs[0] + len(xs))), (tile, xs)  # contiguous workgroups
        owners[tile] = xs
    stored, consumed, final = {}, [], {}
    # process in decreasing workgroup order: every wait targets a higher one
    for tile, xs in owners.items():
        first, n = xs[0], len(xs)
        sums = {x: {(x, tile)} for x in xs}
        for r in reversed(range(n)):
            x = first + r
            l = 0
            while (1 << l) < n:
                if r & (1 << l):
                    stored[(x, tile)] = sums[x]
                    break
                child = r + (1 << l)
                if child < n:
                    assert first + child > x
                    consumed.append((first + child, tile))
                    sums[x] |= stored[(first + child, tile)]
                l += 1
            else:
                final[tile] = sums[x]
                assert r == 0
    assert sorted(final) == list(range(t))
    for tile, xs in owners.items():
        assert final[tile] == {(x, tile) for x in xs}
    assert sorted(consumed) == sorted(stored)
    # one stored partial per workgroup at most (one slot each)
    assert len({x for x, _ in stored}) == len(stored)


@pytest.mark.parametrize("shape", [(256, 4096, 65536), (1000, 1000, 5000), (144, 208, 11952), (600, 520, 3000),
                                   (4352, 4096, 4096), (2048, 2048, 8192), (9392, 2976, 14144)])
@pytest.mark.parametrize("dtype", [sk.F16, sk.F32])
def test_xcd_aligned_tree_fixup_combines_every_piece_once(shape, dtype):
    m, n, k = shape
    slots = 256 if dtype != sk.F32 else 512
    p = sk.plan_query(_desc(m, n, k, dtype), sk.make_options(schedule=sk.SCHED_XCD_ALIGNED), slots)
    assert p.fixup_tree == 1
    _simulate_tree_fixup(p)


def test_schedules_beyond_32_bit_arithmetic():
    """The kernels walk schedules in 32-bit integers.  With 2^20 iterations
    per tile (k = 2^26) the XCD-aware quanta products of a 272-tile region
    pass 2^31: the explicit schedule is refused and AUTO takes the two-tile
    hybrid.  With 2^24 - 1 iterations even that region passes 2^31 and AUTO
    runs data-parallel.  Every plan handed out still covers each iteration
    once."""
    d = _desc(256 * 17, 256 * 16, 1 << 26)
    with pytest.raises(sk.SkError):
        sk.plan_query(d, sk.make_options(schedule=sk.SCHED_XCD_ALIGNED), 256)
    p = sk.plan_query(d, None, 256)
    assert p.schedule == sk.SCHED_SK_HYBRID2 and p.sk_tiles == 272
    _check_schedule(p)
    d = _desc(256 * 17, 256 * 16, (1 << 30) - 64)
    for sched in (sk.SCHED_SK_BASIC, sk.SCHED_SK_HYBRID2, sk.SCHED_XCD_ALIGNED):
        with pytest.raises(sk.SkError):
            sk.plan_query(d, sk.make_options(schedule=sched), 256)
    p = sk.plan_query(d, None, 256)
    assert p.schedule == sk.SCHED_DP and p.sk_tiles == 0
    _check_schedule(p)
    # just inside the limit the aligned schedule is kept
    p = sk.plan_query(_desc(256 * 17, 256 * 16, 1 << 20), None, 256)
    assert p.schedule == sk.SCHED_XCD_ALIGNED and p.sk_tiles > 0
    _check_schedule(p)


def test_auto_below_a_wave_needs_a_clear_iteration_gain():
    """228 tiles of 229 iterations on 256 slots: the split would save about
    11 % of the iterations, less than the single data-parallel wave gains
    from its 28 idle CUs (higher clock), so AUTO keeps the wave; 64 tiles
    split four ways save 75 % and keep the split."""
    large = sk.make_options(tile=sk.TILE_LARGE)
    near = sk.plan_query(_desc(2896, 4816, 14608), large, 256)
    assert near.tiles == 228 and near.sk_tiles == 0 and near.grid == 228
    forced = sk.plan_query(_desc(2896, 4816, 14608),
                           sk.make_options(schedule=sk.SCHED_XCD_ALIGNED, tile=sk.TILE_LARGE), 256)
    assert forced.sk_tiles == 228
    far = sk.plan_query(_desc(2048, 2048, 8192), large, 256)
    assert far.sk_tiles == 64 and far.grid == 256


def test_auto_tile_instance():
    """fp16 AUTO keeps the large tile once its tiles fill the grid and takes
    the small one where the runtime model predicts it faster (few large
    tiles of few iterations); an explicit instance is always honoured.
    fp32 likewise between 128 x 128 and 64 x 64 (1024^3 is one 64 x 64 tile
    per CU), and ABFT keeps the 128 x 128 tile."""
    big = sk.plan_query(_desc(8192, 8192, 8192), None, 256)
    assert (big.tile_m, big.slots) == (256, 256)
    small = sk.plan_query(_desc(512, 512, 512), None, 256)
    assert (small.tile_m, small.slots) == (128, 512)
    for shape in [(512, 512, 512), (8192, 8192, 8192), (300, 5000, 700)]:
        for tile, bm in [(sk.TILE_LARGE, 256), (sk.TILE_SMALL, 128)]:
            assert sk.plan_query(_desc(*shape), sk.make_options(tile=tile), 256).tile_m == bm
        for tile, bm in [(sk.TILE_LARGE, 128), (sk.TILE_SMALL, 64)]:
            assert sk.plan_query(_desc(*shape, sk.F32), sk.make_options(tile=tile), 512).tile_m == bm
        with pytest.raises(sk.SkError) as e:
            sk.plan_query(_desc(*shape, sk.F32), sk.make_options(tile=sk.TILE_SMALL, abft=True), 512)
        assert e.value.status == sk.ERR_UNSUPPORTED
        assert sk.plan_query(_desc(*shape, sk.F32), sk.make_options(abft=True), 512).tile_m == 128
    f32_big = sk.plan_query(_desc(6144, 6144, 6144, sk.F32), None, 512)
    assert (f32_big.tile_m, f32_big.slots) == (128, 512)
    f32_small = sk.plan_query(_desc(1024, 1024, 1024, sk.F32), None, 512)
    assert (f32_small.tile_m, f32_small.slots, f32_small.tiles) == (64, 1024, 256)
    with pytest.raises(sk.SkError):
        sk.plan_query(_desc(512, 512, 512), sk.make_options(tile=3), 256)


@pytest.mark.parametrize("dtype", [sk.F32, sk.F16, sk.BF16])
@pytest.mark.parametrize("m,n,k", [(1, 16384, 16384), (16384, 1, 16384), (1, 1, 1 << 24),
                                   (3, 1, 100003), (1, 5000, 7), (1, 300, 4097)])
def test_matrix_vector_split(dtype, m, n, k):
    """AUTO sends m == 1 or n == 1 to the even split of dot products: the
    chunks are whole 16-byte pieces, S chunks cover k exactly (the last one
    not empty), and there are enough (row, chunk) tasks for every CU."""
    vec = 4 if dtype == sk.F32 else 8
    slots = 512 if dtype == sk.F32 else 256
    for layout in ([sk.A_ROW_B_COL, sk.A_COL_B_COL] if m == 1 else [sk.A_ROW_B_COL, sk.A_ROW_B_ROW]):
        kp = -(-k // vec) * vec  # rows padded to 16 bytes
        lda = kp if layout in (0, 1) else 1
        ldb = kp if layout in (1, 3) else 1
        d = sk.make_desc(m, n, k, 1.0, 1 << 20, lda, 1 << 21, ldb, 0.0, 1 << 22, n, dtype, layout)
        p = sk.plan_query(d, None, slots)
        assert p.schedule == sk.SCHED_GEMV_SPLIT
        rows, S, chunk = p.tiles, p.sk_blocks, p.tile_k
        assert rows == (n if m == 1 else m) and p.total_iters == rows * S
        assert chunk % vec == 0 and S * chunk >= k > (S - 1) * chunk
        assert chunk >= min(k, 8 * 64 * vec) - (vec - 1) or S == 1
        assert rows * S >= min(32 * 256, rows * max(1, k // (8 * 64 * vec)))
        assert 1 <= p.grid <= 8 * 256
        assert sk.plan_segments(p, 0) == []
        assert sk.plan_query(d, sk.make_options(schedule=sk.SCHED_GEMV_SPLIT), slots).schedule == \
            sk.SCHED_GEMV_SPLIT


@pytest.mark.parametrize("dtype", [sk.F32, sk.F16, sk.BF16])
@pytest.mark.parametrize("m,n,k", [(1, 16384, 16384), (16384, 1, 16384), (1, 300, 4097), (5000, 1, 7),
                                   (1, 1, 1 << 20), (1, 100003, 64)])
def test_matrix_vector_output_contiguous_form(dtype, m, n, k):
    """With the matrix operand contiguous along the output (m == 1 with B
    row-major, n == 1 with A column-major) AUTO takes the axpy form of the
    split: tasks are (block of one wave's width of outputs, chunk of k rows),
    the chunks cover k exactly, at least 64 rows each unless there is only
    one, and there are enough tasks for every CU; any vector stride."""
    vec = 4 if dtype == sk.F32 else 8
    slots = 512 if dtype == sk.F32 else 256
    layouts = [sk.A_ROW_B_ROW, sk.A_COL_B_ROW] if m == 1 else [sk.A_COL_B_COL, sk.A_COL_B_ROW]
    for layout in layouts:
        R = n if m == 1 else m
        ldm = -(-R // vec) * vec  # rows padded to 16 bytes
        if m == 1:
            lda = k if layout in (0, 1) else 7
            d = sk.make_desc(m, n, k, 1.0, 1 << 20, lda, 1 << 21, ldm, 0.0, 1 << 22, n, dtype, layout)
        else:
            ldb = 3 if layout in (0, 2) else k
            d = sk.make_desc(m, n, k, 1.0, 1 << 20, ldm, 1 << 21, ldb, 0.0, 1 << 22, 5, dtype, layout)
        p = sk.plan_query(d, None, slots)
        assert p.schedule == sk.SCHED_GEMV_SPLIT and p.tile_n == 64 * vec, (layout, p.schedule, p.tile_n)
        S, chunk, blocks = p.sk_blocks, p.tile_k, -(-R // (64 * vec))
        assert p.tiles == R and p.total_iters == blocks * S
        assert S * chunk >= k > (S - 1) * chunk and (chunk >= 64 or S == 1)
        assert blocks * S >= min(8 * 256, blocks * max(1, k // 64))
        assert sk.plan_segments(p, 0) == []


@pytest.mark.parametrize("dtype", [sk.F32, sk.F16, sk.BF16])
@pytest.mark.parametrize("m,n,k", [(8, 16384, 16384), (16384, 2, 4096), (16, 16, 16), (3, 1000, 4097),
                                   (2, 5, 100003)])
def test_matrix_vector_few_vectors_form(dtype, m, n, k):
    """2 .. 16 vectors (fp16/bf16: 8) against k-contiguous rows (both
    operands k-contiguous, neither m nor n 1) take the multi form: tasks are
    blocks of 64 (fp32) or 16 rows times chunks of whole 64-byte slabs of k
    (the last chunk ends at k), at least eight slabs each unless there is
    only one chunk, and enough of them for every CU; more vectors keep the
    tiled schedules."""
    es = 4 if dtype == sk.F32 else 2
    slab = 64 // es
    slots = 512 if dtype == sk.F32 else 256
    kp = -(-k // (16 // es)) * (16 // es)
    d = sk.make_desc(m, n, k, 1.0, 1 << 20, kp, 1 << 21, kp, 0.0, 1 << 22, n, dtype, sk.A_ROW_B_COL)
    p = sk.plan_query(d, None, slots)
    V, R = (m, n) if m <= 16 else (n, m)
    if V > (16 if dtype == sk.F32 else 8):
        assert p.schedule != sk.SCHED_GEMV_SPLIT
        return
    rows = 64 if dtype == sk.F32 else 16
    assert p.schedule == sk.SCHED_GEMV_SPLIT and p.tile_m == V and p.tile_n == rows
    S, chunk, blocks = p.sk_blocks, p.tile_k, -(-R // rows)
    assert p.tiles == V * R and p.total_iters == blocks * S
    assert chunk % slab == 0 and S * chunk >= k > (S - 1) * chunk
    assert chunk >= 8 * slab or S == 1
    per_cu = 8 if dtype == sk.F32 else 16
    assert 2 * blocks * S >= min(per_cu * 256, blocks * max(1, k // (8 * slab)))  # chunks round up to slabs
    # any other operand order keeps the tiled schedules
    other = sk.make_desc(m, n, k, 1.0, 1 << 20, kp, 1 << 21, n, 0.0, 1 << 22, n, dtype, sk.A_ROW_B_ROW)
    assert sk.plan_query(other, None, slots).schedule != sk.SCHED_GEMV_SPLIT


def test_matrix_vector_fallbacks():
    """Shapes or options the matrix-vector path does not take go to the
    tiled schedules under AUTO, and are refused under an explicit request."""
    gemv = sk.make_options(schedule=sk.SCHED_GEMV_SPLIT)
    cases = [
        sk.make_desc(17, 64, 64, 1.0, 1 << 20, 64, 1 << 21, 64, 0.0, 1 << 22, 64, sk.F16, 1),  # m = 17
        sk.make_desc(2, 64, 64, 1.0, 1 << 20, 64, 1 << 21, 64, 0.0, 1 << 22, 64, sk.F16, 0),  # m = 2, B n-major
        sk.make_desc(4, 64, 64, 1.0, 1 << 20, 66, 1 << 21, 64, 0.0, 1 << 22, 64, sk.F16, 1),  # A rows unaligned
        sk.make_desc(1, 64, 64, 1.0, 1 << 20, 64, 1 << 21, 65, 0.0, 1 << 22, 64, sk.F16, 1),  # rows unaligned
        sk.make_desc(1, 64, 64, 1.0, (1 << 20) + 2, 64, 1 << 21, 64, 0.0, 1 << 22, 64, sk.F16, 1),
        sk.make_desc(64, 1, 64, 1.0, 1 << 20, 64, 1 << 21, 64, 0.0, 1 << 22, 1, sk.F16, 0),  # ldb 64
        sk.make_desc(1, 64, 64, 1.0, 1 << 20, 64, 1 << 21, 65, 0.0, 1 << 22, 64, sk.F16, 0),  # B rows unaligned
        sk.make_desc(64, 1, 64, 1.0, 1 << 20, 66, 1 << 21, 64, 0.0, 1 << 22, 1, sk.F16, 2),  # A columns unaligned
        sk.make_desc(1, 64, 64, 1.0, 1 << 20, 64, (1 << 21) + 4, 64, 0.0, 1 << 22, 64, sk.F16, 0),
    ]
    for d in cases:
        assert sk.plan_query(d, None, 256).schedule != sk.SCHED_GEMV_SPLIT
        with pytest.raises(sk.SkError):
            sk.plan_query(d, gemv, 256)
    d = sk.make_desc(1, 64, 64, 1.0, 1 << 20, 64, 1 << 21, 64, 0.0, 1 << 22, 64, sk.F32, 1)
    assert sk.plan_query(d, None, 512).schedule == sk.SCHED_GEMV_SPLIT
    for o in [sk.make_options(tile=sk.TILE_LARGE), sk.make_options(forced_grid=4),
              sk.make_options(schedule=sk.SCHED_DP)]:
        assert sk.plan_query(d, o, 512).schedule != sk.SCHED_GEMV_SPLIT


def test_two_tile_hybrid_owner_has_one_peer():
    for t_m, t_n in [(17, 17), (23, 12), (16, 17)]:
        d = _desc(256 * t_m, 256 * t_n, 4096, sk.F16)
        p = sk.plan_query(d, sk.make_options(schedule=sk.SCHED_SK_HYBRID2), 256)
        assert p.schedule == sk.SCHED_SK_HYBRID2 and p.max_peers == 1
        p = sk.plan_query(d, None, 256)
        assert p.schedule == sk.SCHED_XCD_ALIGNED and p.sk_tiles > 0 and p.max_peers == 1


def test_grid_model_regimes():
    """Qualitative behaviour of the appendix A.1 model (Fig. 8): large-k
    short-wide shapes use every slot, a medium-k 64-tile shape stays at the
    tile count, a single tile with a huge k stops at a small grid."""
    model = (4.0, 2.0, 1.0, 2.0)
    basic = sk.SCHED_SK_BASIC
    # T(g) ~ c*I/g + d*g/t is minimised near sqrt(c*I*t/d); with t = 16 tiles
    # and I = 16 * 1024 iterations that lies beyond the 256 slots
    p = sk.plan_query(_desc(256, 256 * 16, 65536), sk.make_options(model=model, schedule=basic, tile=sk.TILE_LARGE), 256)
    assert p.grid == 256
    # 64 tiles of 4 iterations: splitting saves at most 2 iterations per
    # workgroup but costs b + d = 4
    p = sk.plan_query(_desc(256 * 8, 256 * 8, 256), sk.make_options(model=model, schedule=basic, tile=sk.TILE_LARGE), 256)
    assert p.grid == 64
    p = sk.plan_query(_desc(256, 256, 64 * 128), sk.make_options(model=model, schedule=basic, tile=sk.TILE_LARGE), 256)
    assert 1 < p.grid <= 16
    # the same regimes under the XCD-aware split (grid = D * ceil(t / s))
    p = sk.plan_query(_desc(256, 256 * 16, 65536), sk.make_options(model=model, tile=sk.TILE_LARGE), 256)
    assert p.sk_tiles == 16 and p.grid == 256
    p = sk.plan_query(_desc(256 * 8, 256 * 8, 256), sk.make_options(model=model, tile=sk.TILE_LARGE), 256)
    assert p.sk_tiles == 0 and p.grid == 64
    # one tile: its partials meet in a binary tree, so the owner waits for
    # only log2(pieces) of them and a deeper split than the page's pays
    p = sk.plan_query(_desc(256, 256, 64 * 128), sk.make_options(model=model, tile=sk.TILE_LARGE), 256)
    assert 16 <= p.grid <= 64 and p.fixup_tree == 1


def test_repack_flags():
    # an n-contiguous 16-bit B is read in place by the 256 and 128 instances
    p = sk.plan_query(_desc(1000, 1000, 1000, sk.F16, sk.A_ROW_B_ROW), None, 256)
    assert p.packs == 0
    p = sk.plan_query(_desc(1000, 1000, 1000, sk.BF16, sk.A_ROW_B_ROW), sk.make_options(tile=sk.TILE_SMALL), 256)
    assert p.packs == 0
    # ... and so is an m-contiguous A
    p = sk.plan_query(_desc(1000, 1000, 1000, sk.F16, sk.A_COL_B_ROW), None, 256)
    assert p.packs == 0
    p = sk.plan_query(_desc(1000, 1000, 1000, sk.F16, sk.A_COL_B_COL), sk.make_options(tile=sk.TILE_SMALL), 256)
    assert p.packs == 0
    # m not a multiple of 8 (lda = m here): A repacked
    p = sk.plan_query(_desc(1004, 1000, 1000, sk.F16, sk.A_COL_B_ROW), None, 256)
    assert p.packs == 1
    # the narrow-m instance reads k-contiguous operands only
    p = sk.plan_query(_desc(96, 1000, 1000, sk.F16, sk.A_ROW_B_ROW), sk.make_options(tile=sk.TILE_NARROW), 256)
    assert p.packs == 2
    p = sk.plan_query(_desc(96, 1000, 1000, sk.F16, sk.A_COL_B_COL), sk.make_options(tile=sk.TILE_NARROW), 256)
    assert p.packs == 1
    # n not a multiple of 8: the last 128-bit chunk of a k-row would straddle n
    d = sk.make_desc(1000, 1004, 1000, 1.0, 1 << 20, 1000, 1 << 21, 1008, 0.0, 1 << 22, 1004, sk.F16,
                     sk.A_ROW_B_ROW)
    assert sk.plan_query(d, None, 256).packs == 2
    # ldb not a multiple of 8, or a misaligned base
    d = sk.make_desc(1000, 1000, 1000, 1.0, 1 << 20, 1000, 1 << 21, 1004, 0.0, 1 << 22, 1000, sk.F16,
                     sk.A_ROW_B_ROW)
    assert sk.plan_query(d, None, 256).packs == 2
    d = sk.make_desc(1000, 1000, 1000, 1.0, 1 << 20, 1000, (1 << 21) + 8, 1000, 0.0, 1 << 22, 1000, sk.F16,
                     sk.A_ROW_B_ROW)
    assert sk.plan_query(d, None, 256).packs == 2
    # k * ldb beyond a 31-bit byte offset: repacked rather than refused
    p = sk.plan_query(_desc(256, 32768, 32768, sk.F16, sk.A_ROW_B_ROW), None, 256)
    assert p.packs == 2
    p = sk.plan_query(_desc(256, 16384, 32768, sk.F16, sk.A_ROW_B_ROW), None, 256)
    assert p.packs == 0
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
    assert sk.gemm_ex(d, sk.make_options(schedule=sk.SCHED_GEMV_SPLIT + 1), stream=0,
                      check=False) == sk.ERR_INVALID_ARG
    assert sk.plan_query(d, sk.make_options(schedule=sk.SCHED_XCD_ALIGNED), 256).schedule == \
        sk.SCHED_XCD_ALIGNED


def test_strerror_texts():
    assert sk.strerror(0) == "success"
    assert "time" in sk.strerror(sk.ERR_FIXUP_TIMEOUT)
    assert sk.version().startswith("sk_gemm")
    # four counters, the records, then max_ratio and checked
    assert ctypes.sizeof(sk.AbftReport) == 16 + 64 * ctypes.sizeof(sk.AbftRecord) + 8
    assert sk.AbftReport.max_ratio.offset == 16 + 64 * ctypes.sizeof(sk.AbftRecord)


def test_noalloc_refusals_before_any_gpu_call():
    """The allocation-free entry point refuses ABFT (its encodings would need
    an allocation) and bad arguments before touching the GPU; its scratch
    size is the header's."""
    d = _desc(256, 256, 256, sk.F32, sk.A_ROW_B_ROW)
    assert sk.gemm_noalloc(d, sk.make_options(abft=True), check=False) == sk.ERR_UNSUPPORTED
    bad = _desc(-1, 256, 256)
    assert sk.gemm_noalloc(bad, None, check=False) == sk.ERR_INVALID_ARG
    assert sk.library().sk_gemm_noalloc(None, None, None) == sk.ERR_INVALID_ARG
    import re
    hdr = open(sk.HEADER_PATH).read()
    mib = int(re.search(r"#define SK_NOALLOC_PARTIAL_BYTES \((\d+)u \* 1024u \* 1024u\)", hdr).group(1))
    assert mib * 1024 * 1024 == sk.NOALLOC_PARTIAL_BYTES
    assert sk.strerror(sk.ERR_TOO_LARGE).startswith("the call needs more scratch")


def test_forced_grid_beyond_the_slots_is_refused_when_a_wait_could_target_an_undispatched_workgroup():
    """A grid above the resident slot count relies on in-order dispatch as
    slots free up; it is planned only while every owner's last peer is fewer
    than slots - 8 workgroups after it."""
    d = _desc(128, 128, 32 * 600, sk.F32, sk.A_ROW_B_ROW)  # one tile of 600 iterations
    p = sk.plan_query(d, sk.make_options(forced_grid=200), 256)  # within the slots: any reach
    assert p.grid == 200 and p.max_peers == 199
    p = sk.plan_query(d, sk.make_options(forced_grid=300), 512)  # above 256 would be refused
    assert p.grid == 300
    with pytest.raises(sk.SkError) as e:
        sk.plan_query(d, sk.make_options(forced_grid=300), 256)
    assert e.value.status == sk.ERR_UNSUPPORTED
    d2 = _desc(8192, 8192, 8192, sk.F16)  # 1024 tiles: g = t is data-parallel, no waits
    assert sk.plan_query(d2, sk.make_options(forced_grid=1024), 256).max_peers == 0
    assert sk.gemm_ex(d, sk.make_options(test_flags=2), check=False) == sk.ERR_INVALID_ARG


def test_two_tile_hybrid_honours_min_waves():
    """hybrid_min_waves = 2 (the page's "w >= 2"): with one full wave and
    leftover tiles the page's two-tile hybrid becomes basic Stream-K over all
    tiles, planned exactly as the oracle's Algorithm 5 on the slot count;
    from two waves on it is the two-tile hybrid again."""
    d = _desc(256 * 17, 256 * 16, 2048)  # 272 tiles on 256 slots: w = 1, r = 16
    p1 = sk.plan_query(d, sk.make_options(schedule=sk.SCHED_SK_HYBRID2), 256)
    assert p1.schedule == sk.SCHED_SK_HYBRID2 and p1.sk_tiles == 272
    p2 = sk.plan_query(d, sk.make_options(schedule=sk.SCHED_SK_HYBRID2, hybrid_min_waves=2), 256)
    assert p2.schedule == sk.SCHED_SK_BASIC and p2.grid == 256 and p2.sk_tiles == p2.tiles
    assert _lib_plan_records(p2) == _oracle_records(256 * 17, 256 * 16, 2048, p2.tile_m, p2.tile_n,
                                                    p2.tile_k, oracle.SK, 256)
    d3 = _desc(256 * 33, 256 * 16, 2048)  # 528 tiles: w = 2, r = 16
    p3 = sk.plan_query(d3, sk.make_options(schedule=sk.SCHED_SK_HYBRID2, hybrid_min_waves=2), 256)
    assert p3.schedule == sk.SCHED_SK_HYBRID2 and p3.sk_tiles == 16 + 256


def test_narrow_tile_plans():
    """The narrow-m instance: the smallest BM of 64, 128, 192, 256 that holds
    m, 256 columns, one tile row; refused above m = 256 and for fp32 (no
    such instance); AUTO never picks it."""
    for m, bm in ((1, 64), (64, 64), (65, 128), (128, 128), (129, 192), (192, 192), (193, 256), (256, 256)):
        for dt in (sk.F16, sk.BF16):
            p = sk.plan_query(_desc(m, 5000, 9000, dt), sk.make_options(tile=sk.TILE_NARROW), slots=256)
            assert (p.tile_m, p.tile_n, p.tile_k, p.tiles_m, p.tiles_n) == (bm, 256, 64, 1, 20), (m, dt)
            auto = sk.plan_query(_desc(m, 5000, 9000, dt), sk.make_options(), slots=256)
            assert auto.tile_n != 256 or auto.tile_m == 256
    with pytest.raises(sk.SkError) as e:
        sk.plan_query(_desc(257, 5000, 9000), sk.make_options(tile=sk.TILE_NARROW), slots=256)
    assert e.value.status == sk.ERR_UNSUPPORTED
    with pytest.raises(sk.SkError) as e:
        sk.plan_query(_desc(100, 5000, 9000, sk.F32, sk.A_ROW_B_ROW), sk.make_options(tile=sk.TILE_NARROW),
                      slots=512)
    assert e.value.status == sk.ERR_UNSUPPORTED
    with pytest.raises(sk.SkError) as e:
        sk.plan_query(_desc(100, 500, 900), sk.make_options(tile=4), slots=256)
    assert e.value.status == sk.ERR_INVALID_ARG
