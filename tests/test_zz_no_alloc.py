"""The allocation-free entry point (sk_gemm_noalloc) against sk_gemm_ex:
same plans and kernels, so the same bits; scratch from the library's static
per-GPU array, reused from one call to the next (two calls in a row, the
second smaller); refusals with clear codes."""
import numpy as np
import pytest

import work_centric_decomposition_amd as sk

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from gemm_check import TOL, Case, rel_err  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    assert sk.device_status() == sk.OK


def _both(c: Case, opts, alpha=1.0, beta=0.0):
    """C from sk_gemm_ex, then C from sk_gemm_noalloc on the same input C."""
    d = sk.make_desc(c.m, c.n, c.k, alpha, c.dA, c.lda, c.dB, c.ldb, beta, c.dC, c.ldc, c.dtype, c.layout)
    c.reset_c()
    sk.gemm_ex(d, opts)
    torch.cuda.synchronize()
    ref = c.result()
    c.reset_c()
    sk.gemm_noalloc(d, opts)
    torch.cuda.synchronize()
    return ref, c.result()


# (m, n, k, dtype, layout, options, alpha, beta): a forced Stream-K grid
# (partials in the scratch), the XCD-aware split on both fp16/bf16 tiles,
# mn-contiguous fp16 operands, fp32 with a split, matrix-vector products
# with chunk sums in the scratch
CASES = [
    ("fp16 forced grid 200", (1000, 900, 3000, sk.F16, sk.A_ROW_B_COL), dict(forced_grid=200), 1.0, 0.0),
    ("bf16 xcd large tile", (256 * 17, 256 * 16, 1024, sk.BF16, sk.A_ROW_B_COL),
     dict(schedule=sk.SCHED_XCD_ALIGNED, tile=sk.TILE_LARGE), 1.0, 0.0),
    ("fp16 auto small tile", (1000, 1000, 5000, sk.F16, sk.A_ROW_B_COL), dict(tile=sk.TILE_SMALL), 0.5, 1.0),
    # m-contiguous A and n-contiguous B read in place (m and n stay
    # multiples of 8 after the shrink)
    ("fp16 mn-contiguous operands", (1032, 1008, 3000, sk.F16, sk.A_COL_B_ROW), dict(forced_grid=100), 1.0, 1.0),
    ("fp32 forced grid 7", (520, 600, 3000, sk.F32, sk.A_ROW_B_ROW), dict(forced_grid=7), 1.0, 1.0),
    ("fp32 auto", (3000, 2960, 200, sk.F32, sk.A_ROW_B_ROW), {}, 1.0, 0.0),
    ("fp32 small tile", (1024, 1000, 1024, sk.F32, sk.A_ROW_B_ROW), dict(tile=sk.TILE_SMALL), 1.0, 1.0),
    ("fp32 dot products", (1, 2048, 16384, sk.F32, sk.A_ROW_B_COL), {}, 1.0, 0.0),
]


def _shrink(shape):
    m, n, k, dt, lay = shape
    # k stays a multiple of 8 elements, so the operands are read in place
    return (max(1, m // 3), max(1, n // 2 + 8 * (n > 1)), max(8, k // 32 * 8), dt, lay)


@pytest.mark.parametrize("name,shape,kw,alpha,beta", CASES)
def test_noalloc_matches_sk_gemm_ex_two_calls(name, shape, kw, alpha, beta):
    """Two calls in a row, the second on a smaller input: each equals the
    allocating entry point bit for bit and the oracle within tolerance."""
    for i, shp in enumerate((shape, _shrink(shape))):
        m, n, k, dtype, layout = shp
        print("case noalloc", name, "call", i, shp, flush=True)
        c = Case(m, n, k, dtype, layout, 300 + i + m, dist="normal", scale=1 / np.sqrt(k))
        opts = sk.make_options(**kw)
        ref, got = _both(c, opts, alpha, beta)
        assert np.array_equal(ref.view(np.uint8), got.view(np.uint8)), (name, i)
        want, bound = c.reference(alpha, beta)
        assert rel_err(got, dtype, want, bound) <= TOL[dtype], (name, i)


def test_noalloc_refusals():
    c = Case(300, 260, 333, sk.F32, sk.A_ROW_B_COL, 5, pad=1)  # unaligned k-major rows: repack
    d = sk.make_desc(c.m, c.n, c.k, 1.0, c.dA, c.lda, c.dB, c.ldb, 0.0, c.dC, c.ldc, sk.F32, sk.A_ROW_B_COL)
    assert sk.plan_query(d).packs != 0
    assert sk.gemm_noalloc(d, None, check=False) == sk.ERR_UNSUPPORTED
    assert sk.gemm_noalloc(d, sk.make_options(abft=True), check=False) == sk.ERR_UNSUPPORTED
    c = Case(2048, 2048, 512, sk.F16, sk.A_ROW_B_COL, 6, with_c=False)
    d = sk.make_desc(c.m, c.n, c.k, 1.0, c.dA, c.lda, c.dB, c.ldb, 0.0, c.dC, c.ldc, sk.F16, sk.A_ROW_B_COL)
    opts = sk.make_options(forced_grid=300, tile=sk.TILE_LARGE)  # 300 partials of 256 KiB > 64 MiB
    assert sk.gemm_noalloc(d, opts, check=False) == sk.ERR_TOO_LARGE
    # the refusals launched nothing; a fitting call still works afterwards
    sk.gemm_noalloc(d, sk.make_options(forced_grid=200, tile=sk.TILE_LARGE))
    torch.cuda.synchronize()
