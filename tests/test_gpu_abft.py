"""GPU tests of the ABFT mode (fault-tolerant GEMM page, threadblock-level
scheme): every injected fault detected, located and corrected, zero false
positives, results within the fp32 tolerance of the oracle.

Faults are injected into the fp32 segment accumulator just before the
segment is verified (sk_fault).  Reading taken for bit flips: a flip whose
size is below ten times the detection threshold of its row or column is
re-drawn (a checksum cannot see a change smaller than the rounding noise).
"""
import ctypes

import numpy as np
import pytest

import sk_synth as S
import work_centric_decomposition_amd as sk

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from gemm_check import TOL, Case, decode, rel_err, sample_indices  # noqa: E402

FAULT_DT = np.dtype([("row", "<i8"), ("col", "<i8"), ("iter", "<i4"), ("kind", "<i4"),
                     ("bit", "<i4"), ("value", "<f4")])
assert FAULT_DT.itemsize == ctypes.sizeof(sk.Fault)
U = 2.0 ** -24


@pytest.fixture(autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    assert sk.device_status() == sk.OK


def _faults_dev(faults):
    arr = np.zeros(max(len(faults), 1), FAULT_DT)
    for i, f in enumerate(faults):
        arr[i] = f
    return torch.from_numpy(arr.view(np.uint8)).cuda()


def _report_dev():
    return torch.zeros(ctypes.sizeof(sk.AbftReport), dtype=torch.uint8, device="cuda")


def _run_abft(c: Case, faults=(), forced=0, schedule=0, alpha=1.0, beta=0.0):
    fd = _faults_dev(faults)
    rep = _report_dev()
    opts = sk.make_options(abft=True, faults=fd if faults else None, n_faults=len(faults),
                           forced_grid=forced, schedule=schedule)
    got = c.run(alpha, beta, opts, rep)
    return got, sk.read_report(rep)


def _records(r):
    return [(r.records[i].row, r.records[i].col, r.records[i].status)
            for i in range(min(r.n_records, sk.ABFT_MAX_RECORDS))]


def _logical(c: Case):
    A = decode(c.A, c.dtype)
    B = decode(c.B, c.dtype)
    if c.layout in (sk.A_ROW_B_ROW, sk.A_ROW_B_COL):
        Al = np.lib.stride_tricks.as_strided(A, (c.m, c.k), (c.lda * 8, 8))
    else:
        Al = np.lib.stride_tricks.as_strided(A, (c.m, c.k), (8, c.lda * 8))
    if c.layout in (sk.A_ROW_B_ROW, sk.A_COL_B_ROW):
        Bl = np.lib.stride_tricks.as_strided(B, (c.k, c.n), (c.ldb * 8, 8))
    else:
        Bl = np.lib.stride_tricks.as_strided(B, (c.k, c.n), (8, c.ldb * 8))
    return np.ascontiguousarray(Al), np.ascontiguousarray(Bl)


def _thresholds(Al, Bl, i, j, tile=128):
    """Detection thresholds the kernel applies to row i and column j of a
    full-k verification domain (a whole tile): 2^-24 sqrt(k) times the bound
    ||a_i||_1 max_k (|B| e)_k of the row's absolute checksum (likewise
    max_k (e^T|A|)_k ||b_j||_1 for the column); used only to re-draw bit
    flips too small to detect."""
    r0, c0 = (i // tile) * tile, (j // tile) * tile
    Ba = np.abs(Bl[:, c0:c0 + tile])
    Aa = np.abs(Al[r0:r0 + tile, :])
    ra = np.abs(Al[i]).sum() * Ba.sum(axis=1).max()
    ca = Aa.sum(axis=0).max() * np.abs(Bl[:, j]).sum()
    scale = U * np.sqrt(Al.shape[1])
    return scale * ra, scale * ca


def _flip(v, bit):
    x = np.array([v], np.float32).view(np.uint32)
    x ^= np.uint32(1 << bit)
    return float(x.view(np.float32)[0])


def _check_corrected(c, got, faults, rep, ref=None, alpha=1.0, beta=0.0):
    assert rep.detected == len(faults), (rep.detected, rep.corrected, rep.uncorrectable, _records(rep))
    assert rep.corrected == len(faults) and rep.uncorrectable == 0
    assert sorted((r, cc) for r, cc, st in _records(rep)) == sorted((f[0], f[1]) for f in faults)
    rows = np.array([f[0] for f in faults], np.int64)
    cols = np.array([f[1] for f in faults], np.int64)
    srow, scol = sample_indices(c.m, c.n, 500, 17)
    rows, cols = np.concatenate([rows, srow]), np.concatenate([cols, scol])
    want, bound = c.reference_entries(rows, cols, alpha, beta)
    g = decode(got[rows, cols], c.dtype)
    assert np.all(np.isfinite(g))
    assert np.max(np.abs(g - want) / bound) <= TOL[sk.F32]


def test_fault_free_runs_report_nothing_and_match_oracle():
    """No false positives: 120 fault-free runs over seeds, layouts and grids."""
    runs = 0
    for seed in range(30):
        layout = seed % 4
        c = Case(384 + 16 * seed, 256 + 8 * seed, 512 + 32 * seed, sk.F32, layout, 5000 + seed)
        ref, bound = c.reference()
        for forced in (0, 3, 7, 64):
            c.reset_c()
            got, rep = _run_abft(c, forced=forced)
            runs += 1
            assert (rep.detected, rep.corrected, rep.uncorrectable, rep.n_records) == (0, 0, 0, 0), \
                (seed, forced, _records(rep))
            assert rel_err(got, sk.F32, ref, bound) <= TOL[sk.F32]
    assert runs == 120


def test_fault_free_4096_with_beta():
    c = Case(4096, 4096, 4096, sk.F32, sk.A_ROW_B_ROW, S.SEED_ABFT)
    got, rep = _run_abft(c, alpha=1.0, beta=1.0)
    assert (rep.detected, rep.n_records) == (0, 0)
    assert c.freivalds(got, 1.0, 1.0) <= TOL[sk.F32]


@pytest.mark.parametrize("layout", [0, 1, 2, 3])
def test_single_additive_fault_every_layout(layout):
    c = Case(300, 260, 640, sk.F32, layout, 77 + layout)
    faults = [(123, 201, 0, 0, 0, 1000.0)]
    got, rep = _run_abft(c, faults)
    _check_corrected(c, got, faults, rep)
    assert abs(rep.records[0].delta - 1000.0) < 1.0


def test_faults_in_stream_k_producer_and_owner_segments():
    """384x384x128 on a forced grid of 4: each tile is split between two
    workgroups; a fault in the producer's segment and one in another tile's
    owner segment are both corrected before the fixup."""
    c = Case(384, 384, 128, sk.F32, sk.A_ROW_B_ROW, S.SEED_SGEMM_SMALL)
    p = sk.plan_query(sk.make_desc(384, 384, 128, 1, c.dA, c.lda, c.dB, c.ldb, 0, c.dC, c.ldc,
                                   sk.F32, 0), sk.make_options(forced_grid=4, abft=True))
    segs = [s for x in range(4) for s in sk.plan_segments(p, x)]
    split = [s for s in segs if not s[3]]
    assert split, "the plan must split a tile"
    t0, b0, e0 = split[0][0], split[0][1], split[0][2]
    tm, tn = divmod(t0, p.tiles_n)
    owner = [s for s in segs if s[3] and not s[4] and s[0] != t0][0]
    t1 = owner[0]
    tm1, tn1 = divmod(t1, p.tiles_n)
    faults = [(tm * 128 + 5, tn * 128 + 77, b0, 0, 0, 1000.0),          # producer segment
              (tm1 * 128 + 100, tn1 * 128 + 3, 0, 0, 0, -1000.0)]      # owner segment
    got, rep = _run_abft(c, faults, forced=4)
    _check_corrected(c, got, faults, rep)
    seg_begins = sorted(rep.records[i].seg_begin for i in range(2))
    assert seg_begins == sorted([b0, 0])


def test_two_faults_in_one_domain_are_uncorrectable():
    c = Case(256, 256, 256, sk.F32, sk.A_ROW_B_ROW, 91)
    faults = [(10, 20, 0, 0, 0, 1000.0), (40, 90, 0, 0, 0, 1000.0)]
    got, rep = _run_abft(c, faults)
    assert rep.detected == 1 and rep.uncorrectable == 1 and rep.corrected == 0


def test_faults_on_ragged_edges_are_corrected():
    """Faults in partial tiles at the matrix edge, every layout: rows of A and
    columns of B past the matrix are left out of the encodings."""
    for layout in range(4):
        c = Case(200, 150, 300, sk.F32, layout, 93 + layout)
        faults = [(199, 149, 0, 0, 0, 1000.0), (130, 20, 0, 0, 0, -1000.0)]
        got, rep = _run_abft(c, faults)
        _check_corrected(c, got, faults, rep)


def test_faults_corrected_before_alpha_and_beta_are_applied():
    """The checksums cover A B; a fault is corrected in the accumulators, and
    the epilogue then applies alpha and beta (C read) as without ABFT."""
    for layout in range(4):
        c = Case(300, 260, 640, sk.F32, layout, 97 + layout)
        faults = [(123, 201, 0, 0, 0, 1000.0), (7, 3, 0, 0, 0, -500.0)]
        got, rep = _run_abft(c, faults, alpha=1.5, beta=-0.75)
        _check_corrected(c, got, faults, rep, alpha=1.5, beta=-0.75)


def test_abft_on_repacked_operands():
    """k-major rows that are not 16-byte aligned are repacked before the GEMM;
    the encodings are formed from the copies the kernel reads."""
    for layout in range(4):
        c = Case(300, 260, 333, sk.F32, layout, 95 + layout, pad=1)
        d = sk.make_desc(c.m, c.n, c.k, 1.0, c.dA, c.lda, c.dB, c.ldb, 0.0, c.dC, c.ldc, sk.F32,
                         layout)
        p = sk.plan_query(d, sk.make_options(abft=True))
        ref, bound = c.reference()
        c.reset_c()
        got, rep = _run_abft(c)
        assert (rep.detected, rep.n_records) == (0, 0), (layout, p.packs, _records(rep))
        assert rel_err(got, sk.F32, ref, bound) <= TOL[sk.F32]
        if layout == sk.A_ROW_B_COL:
            assert p.packs == 3, p.packs
        c.reset_c()
        faults = [(123, 201, 0, 0, 0, 1000.0)]
        got, rep = _run_abft(c, faults)
        _check_corrected(c, got, faults, rep)


@pytest.mark.parametrize("bit", [31, 30, 29, 28, 27, 26, 25, 24, 23, 22, 21])
def test_bit_flips_of_large_effect(bit):
    c = Case(512, 512, 1024, sk.F32, sk.A_ROW_B_ROW, 300 + bit)
    Al, Bl = _logical(c)
    i, j = 200 + bit, 333 - bit
    v = float(Al[i] @ Bl[:, j])
    tr, tc = _thresholds(Al, Bl, i, j)
    fv = _flip(v, bit)
    if np.isfinite(fv) and abs(fv - v) < 10 * max(tr, tc):
        pytest.skip("this flip changes the value by less than 10x the threshold (re-drawn below)")
    faults = [(i, j, 0, 1, bit, 0.0)]
    got, rep = _run_abft(c, faults)
    _check_corrected(c, got, faults, rep)


def _seeded_faults(run, c, Al, Bl, tile=128):
    """1..8 faults at seeded positions, at most one per tile, additive 1e3 or
    a bit flip; flips below ten times the threshold are re-drawn."""
    raw = S.u64(S.SEED_ABFT, 1000 + run, 0, 512)
    pos = [0]

    def nxt(mod):
        v = int(raw[pos[0]] % np.uint64(mod))
        pos[0] += 1
        return v

    nf = 1 + nxt(8)
    faults, tiles, redraws = [], set(), 0
    while len(faults) < nf:
        i, j = nxt(c.m), nxt(c.n)
        if (i // tile, j // tile) in tiles:
            continue
        if nxt(2) == 0:
            faults.append((i, j, 0, 0, 0, 1000.0))
        else:
            bit = nxt(32)
            v = float(Al[i] @ Bl[:, j])
            fv = _flip(v, bit)
            tr, tc = _thresholds(Al, Bl, i, j)
            if np.isfinite(fv) and abs(fv - v) < 10 * max(tr, tc):
                redraws += 1
                continue
            faults.append((i, j, 0, 1, bit, 0.0))
        tiles.add((i // tile, j // tile))
    return faults, redraws


def test_abft_4096_seeded_fault_runs():
    """4096^3 fp32, U[-1,1], 1-8 faults per run at seeded positions, 50 runs:
    every fault detected, located at its element and corrected."""
    c = Case(4096, 4096, 4096, sk.F32, sk.A_ROW_B_ROW, S.SEED_ABFT, with_c=False)
    Al, Bl = _logical(c)
    total, total_redraws = 0, 0
    for run in range(50):
        faults, redraws = _seeded_faults(run, c, Al, Bl)
        total_redraws += redraws
        got, rep = _run_abft(c, faults)
        print(f"run {run}: {len(faults)} faults, {redraws} re-drawn flips", flush=True)
        _check_corrected(c, got, faults, rep)
        total += len(faults)
    assert total >= 50


def test_abft_4096_fault_free_runs_margin():
    """100 fault-free 4096^3 fp32 runs (10 seeds, 5 with beta = 0 and 5 with
    beta = 1 each; U[-1,1] inputs): zero detections in every run, every row
    and column of every tile checked, and the largest |residual| / threshold
    seen over all of them (the margin of the sqrt(k_seg) threshold) is
    printed and must stay below 1."""
    n, runs, worst = 4096, 0, 0.0
    for seed in range(10):
        c = Case(n, n, n, sk.F32, sk.A_ROW_B_ROW, S.SEED_ABFT + 100 + seed)
        rep_dev = _report_dev()
        opts = sk.make_options(abft=True)
        d = sk.make_desc(n, n, n, 1.0, c.dA, c.lda, c.dB, c.ldb, 0.0, c.dC, c.ldc, sk.F32, sk.A_ROW_B_ROW)
        for r in range(10):
            beta = 0.0 if r < 5 else 1.0
            d.beta = beta
            c.reset_c()
            sk.gemm_ex(d, opts, rep_dev)
            torch.cuda.synchronize()
            rep = sk.read_report(rep_dev)
            assert (rep.detected, rep.corrected, rep.uncorrectable, rep.n_records) == (0, 0, 0, 0), \
                (seed, r, _records(rep))
            assert rep.checked == (n // 128) ** 2 * 256, rep.checked
            worst = max(worst, rep.max_ratio)
            runs += 1
        got = c.result()
        assert c.freivalds(got, 1.0, 1.0) <= TOL[sk.F32]  # the last run (beta = 1) is right
        print(f"seed {seed}: largest |residual| / threshold so far {worst:.4f}", flush=True)
    print(f"{runs} fault-free 4096^3 runs: largest |residual| / threshold = {worst:.4f}", flush=True)
    assert runs == 100 and 0.0 < worst < 1.0


def test_abft_workspace_buffers_grow_between_calls():
    """The encodings, threshold inputs and per-tile counters live in the
    stream's workspace and grow when a call needs more: a small call, one
    whose encodings pass the initial 4 MiB (16384 x 16384 x 4096, 256 + 256
    tiles at 128 k-iterations), one with more tiles than the initial 1024
    counters (n = 140000: 1094 tile columns), then the small one again.
    Fault-free, each equals the same call without ABFT bit for bit (the
    checksum updates do not touch the accumulators) and reports nothing."""
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    for (m, n, k) in [(300, 260, 640), (16384, 16384, 4096), (64, 140000, 96), (300, 260, 640)]:
        print("case abft growth", m, n, k, flush=True)
        A = torch.rand(m * k, generator=g, device="cuda") * 2 - 1
        B = torch.rand(k * n, generator=g, device="cuda") * 2 - 1
        C0 = torch.zeros(m * n, device="cuda")
        C1 = torch.zeros(m * n, device="cuda")
        rep = _report_dev()
        for C, opts, r in ((C0, sk.make_options(), None), (C1, sk.make_options(abft=True), rep)):
            d = sk.make_desc(m, n, k, 1.0, A, k, B, n, 0.0, C, n, sk.F32, sk.A_ROW_B_ROW)
            sk.gemm_ex(d, opts, r)
        torch.cuda.synchronize()
        r = sk.read_report(rep)
        assert (r.detected, r.n_records) == (0, 0), (m, n, k, _records(r))
        assert r.checked > 0 and r.max_ratio < 1.0, (m, n, k, r.checked, r.max_ratio)
        assert torch.equal(C0.view(torch.int32), C1.view(torch.int32)), (m, n, k)
        del A, B, C0, C1
