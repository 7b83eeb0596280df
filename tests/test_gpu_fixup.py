"""GPU tests of the fixup's bounded wait: a time-out is forced from the host
(producers store their partials without signalling them, and a short wait
limit), every kernel still exits, and the time-out is reported once, by the
next call on the device (which launches nothing) or by sk_device_status."""
import numpy as np
import pytest

import sk_synth as S
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


def _desc(c):
    return sk.make_desc(c.m, c.n, c.k, 1.0, c.dA, c.lda, c.dB, c.ldb, 0.0, c.dC, c.ldc, c.dtype, c.layout)


@pytest.mark.parametrize("dtype", [sk.F32, sk.F16])
def test_forced_time_out_is_reported_by_the_next_call(dtype):
    print("case fixup time-out", dtype, flush=True)
    c = Case(384, 384, 128, dtype, sk.A_ROW_B_COL, S.SEED_SGEMM_SMALL)
    d = _desc(c)
    broken = sk.make_options(forced_grid=5, spin_limit_us=50, test_flags=sk.TEST_NO_SIGNAL)
    assert sk.plan_query(d, broken).max_peers >= 1  # owners wait on peers
    sk.gemm_ex(d, broken)
    torch.cuda.synchronize()  # every wait gave up after 50 us; the kernel exited
    c.reset_c()
    before = c.result()
    rc = sk.gemm_ex(d, sk.make_options(forced_grid=5), check=False)
    assert rc == sk.ERR_FIXUP_TIMEOUT
    torch.cuda.synchronize()
    assert np.array_equal(c.result().view(np.uint8), before.view(np.uint8))  # nothing launched
    # reported once: the next call runs and matches the oracle
    got = c.run(1.0, 0.0, sk.make_options(forced_grid=5))
    ref, bound = c.reference()
    assert rel_err(got, dtype, ref, bound) <= TOL[dtype]
    assert sk.device_status() == sk.OK


def test_forced_time_out_is_reported_by_device_status():
    c = Case(384, 384, 128, sk.F32, sk.A_ROW_B_ROW, S.SEED_SGEMM_SMALL)
    d = _desc(c)
    sk.gemm_ex(d, sk.make_options(forced_grid=5, spin_limit_us=50, test_flags=sk.TEST_NO_SIGNAL))
    assert sk.device_status() == sk.ERR_FIXUP_TIMEOUT
    assert sk.device_status() == sk.OK  # cleared
    got = c.run(1.0, 0.0, sk.make_options(forced_grid=5))  # not reported again
    ref, bound = c.reference()
    assert rel_err(got, sk.F32, ref, bound) <= TOL[sk.F32]


def test_forced_time_out_in_the_allocation_free_entry_point():
    """Its error word is device memory: sk_device_status reports it."""
    c = Case(384, 384, 128, sk.F32, sk.A_ROW_B_ROW, S.SEED_SGEMM_SMALL)
    d = _desc(c)
    sk.gemm_noalloc(d, sk.make_options(forced_grid=5, spin_limit_us=50, test_flags=sk.TEST_NO_SIGNAL))
    assert sk.device_status() == sk.ERR_FIXUP_TIMEOUT
    c.reset_c()
    sk.gemm_noalloc(d, sk.make_options(forced_grid=5))
    torch.cuda.synchronize()
    ref, bound = c.reference()
    assert rel_err(c.result(), sk.F32, ref, bound) <= TOL[sk.F32]
