"""Stream-K GEMM for AMD MI355X (gfx950): Python binding of libskgemm.so.

This module only marshals arguments into the C ABI declared in
``include/sk_gemm.h``; every step of the GEMM runs in the library's HIP
kernels.  Device memory and streams may come from PyTorch: any object with
``data_ptr()`` is accepted where a device pointer is expected, and ``stream``
may be a ``torch.cuda.Stream``, a raw ``hipStream_t`` value (int) or None (the
current PyTorch stream if torch is loaded, else the default stream).

The library is loaded on first use; if it is not built, that first call
raises ImportError: there is no fallback.
"""
from __future__ import annotations

import ctypes
import importlib.util
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libskgemm.so")
HEADER_PATH = os.path.join(HERE, "..", "include", "sk_gemm.h")

F32, F16, BF16 = 0, 1, 2
A_ROW_B_ROW, A_ROW_B_COL, A_COL_B_ROW, A_COL_B_COL = 0, 1, 2, 3
SCHED_AUTO, SCHED_DP, SCHED_SK_BASIC, SCHED_SK_HYBRID2, SCHED_SK_HYBRID1 = 0, 1, 2, 3, 4
SCHED_XCD_ALIGNED, SCHED_GEMV_SPLIT = 5, 6
TILE_AUTO, TILE_LARGE, TILE_SMALL, TILE_NARROW = 0, 1, 2, 3
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NO_MEMORY, ERR_HIP, ERR_FIXUP_TIMEOUT, ERR_NO_DEVICE = \
    0, -1, -2, -3, -4, -5, -6
ERR_TOO_LARGE = -7
TEST_NO_SIGNAL = 1
NOALLOC_PARTIAL_BYTES = 64 * 1024 * 1024
ABFT_MAX_RECORDS = 64

# PyTorch-ROCm ships its own HIP runtime, which its libraries reference by the
# unversioned file name.  If libskgemm.so (which needs libamdhip64.so.7) were
# loaded first, torch would then load a second runtime into the process and
# one of the two would see no device.  Loading torch first makes the library
# bind to the runtime torch already holds.
if importlib.util.find_spec("torch") is not None:
    import torch  # noqa: F401

i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class GemmDesc(ctypes.Structure):
    _fields_ = [("m", i64), ("n", i64), ("k", i64), ("alpha", f32), ("A", vp), ("lda", i64),
                ("B", vp), ("ldb", i64), ("beta", f32), ("C", vp), ("ldc", i64),
                ("dtype", ctypes.c_int), ("layout", ctypes.c_int)]


class Fault(ctypes.Structure):
    _fields_ = [("row", i64), ("col", i64), ("iter", i32), ("kind", i32), ("bit", i32),
                ("value", f32)]


class AbftRecord(ctypes.Structure):
    _fields_ = [("row", i64), ("col", i64), ("delta", f32), ("status", i32), ("tile", i32),
                ("seg_begin", i32)]


class AbftReport(ctypes.Structure):
    _fields_ = [("detected", i32), ("corrected", i32), ("uncorrectable", i32), ("n_records", i32),
                ("records", AbftRecord * ABFT_MAX_RECORDS), ("max_ratio", f32), ("checked", i32)]


class Options(ctypes.Structure):
    _fields_ = [("schedule", i32), ("forced_grid", i32), ("abft", i32), ("hybrid_min_waves", i32),
                ("faults", vp), ("n_faults", i32), ("abft_tau", f32), ("model_a", f32),
                ("model_b", f32), ("model_c", f32), ("model_d", f32), ("spin_limit_us", i32),
                ("tile", i32), ("test_flags", i32)]


class Plan(ctypes.Structure):
    _fields_ = [("tile_m", i32), ("tile_n", i32), ("tile_k", i32), ("slots", i32), ("grid", i32),
                ("schedule", i32), ("tiles_m", i64), ("tiles_n", i64), ("tiles", i64),
                ("iters_per_tile", i64), ("total_iters", i64), ("sk_tiles", i64),
                ("sk_iters_q", i64), ("sk_iters_r", i64), ("dp_tiles", i64), ("full_waves", i32),
                ("tail_tiles", i32), ("max_peers", i32), ("packs", i32), ("phase_div", i32),
                ("sk_blocks", i32), ("group_rows", i32), ("fixup_tree", i32)]


class Segment(ctypes.Structure):
    _fields_ = [("tile", i64), ("iter_begin", i64), ("iter_end", i64), ("started", i32),
                ("ended", i32), ("last_peer", i64)]


class _Library:
    """libskgemm.so, loaded on first use: importing the package (for example
    to build the library) never needs it, while every call through the ABI
    fails loudly when it is missing.  There is no fallback of any kind."""

    def __init__(self):
        self._cdll = None

    def _load(self):
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              f"`python -m work_centric_decomposition_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.sk_gemm.argtypes = [i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, ctypes.c_int,
                                 ctypes.c_int, vp]
        lib.sk_gemm.restype = ctypes.c_int
        lib.sk_gemm_ex.argtypes = [ctypes.POINTER(GemmDesc), ctypes.POINTER(Options), vp, vp]
        lib.sk_gemm_ex.restype = ctypes.c_int
        lib.sk_gemm_noalloc.argtypes = [ctypes.POINTER(GemmDesc), ctypes.POINTER(Options), vp]
        lib.sk_gemm_noalloc.restype = ctypes.c_int
        lib.sk_plan_query.argtypes = [ctypes.POINTER(GemmDesc), ctypes.POINTER(Options), i32,
                                       ctypes.POINTER(Plan)]
        lib.sk_plan_query.restype = ctypes.c_int
        lib.sk_plan_segments.argtypes = [ctypes.POINTER(Plan), i64, ctypes.POINTER(Segment), i64]
        lib.sk_plan_segments.restype = i64
        lib.sk_device_status.argtypes = []
        lib.sk_device_status.restype = ctypes.c_int
        lib.sk_strerror.argtypes = [ctypes.c_int]
        lib.sk_strerror.restype = ctypes.c_char_p
        lib.sk_last_hip_error.argtypes = []
        lib.sk_last_hip_error.restype = ctypes.c_char_p
        lib.sk_release_workspace.argtypes = []
        lib.sk_release_workspace.restype = ctypes.c_int
        lib.sk_version.argtypes = []
        lib.sk_version.restype = ctypes.c_char_p
        self._cdll = lib
        return lib

    def __getattr__(self, name):
        lib = self.__dict__.get("_cdll") or self._load()
        return getattr(lib, name)


_lib = _Library()


class SkError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        msg = f"{what}: {strerror(status)} ({status})"
        if status == ERR_HIP:
            msg += f" [{last_hip_error()}]"
        super().__init__(msg)
        self.status = status


def library():
    """The loaded ctypes library (for tests of the exported symbols)."""
    return _lib._cdll or _lib._load()


def header_functions():
    """Names of the functions declared in include/sk_gemm.h."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(sk_[a-z_]+)\s*\(", text, re.M)))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    raise TypeError(f"expected a device pointer, got {type(x)}")


def _stream(stream):
    if stream is None:
        torch = sys.modules.get("torch")
        if torch is not None and torch.cuda.is_available():
            return int(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def strerror(status: int) -> str:
    return _lib.sk_strerror(status).decode()


def last_hip_error() -> str:
    return _lib.sk_last_hip_error().decode()


def version() -> str:
    return _lib.sk_version().decode()


def gemm(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, dtype, layout, stream=None,
         check=True) -> int:
    """C = alpha*A*B + beta*C through ``sk_gemm`` (asynchronous on `stream`)."""
    rc = _lib.sk_gemm(m, n, k, alpha, _ptr(A), lda, _ptr(B), ldb, beta, _ptr(C), ldc, dtype,
                      layout, _stream(stream))
    if check and rc != OK:
        raise SkError(rc, "sk_gemm")
    return rc


def make_options(schedule=SCHED_AUTO, forced_grid=0, abft=False, hybrid_min_waves=0,
                 faults=None, n_faults=0, abft_tau=0.0, model=(0.0, 0.0, 0.0, 0.0),
                 spin_limit_us=0, tile=0, test_flags=0) -> Options:
    o = Options()
    o.schedule, o.forced_grid, o.abft, o.hybrid_min_waves = schedule, forced_grid, int(abft), \
        hybrid_min_waves
    o.faults, o.n_faults, o.abft_tau = _ptr(faults), n_faults, abft_tau
    o.model_a, o.model_b, o.model_c, o.model_d = model
    o.spin_limit_us = spin_limit_us
    o.tile = tile
    o.test_flags = test_flags
    return o


def make_desc(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, dtype, layout) -> GemmDesc:
    return GemmDesc(m, n, k, alpha, _ptr(A), lda, _ptr(B), ldb, beta, _ptr(C), ldc, dtype, layout)


def gemm_ex(desc: GemmDesc, opts: Options | None = None, report=None, stream=None,
            check=True) -> int:
    """``sk_gemm_ex``: schedule/grid/ABFT options; `report` is a device buffer
    of ``ctypes.sizeof(AbftReport)`` bytes (needed in ABFT mode)."""
    rc = _lib.sk_gemm_ex(ctypes.byref(desc), ctypes.byref(opts) if opts is not None else None,
                         _ptr(report), _stream(stream))
    if check and rc != OK:
        raise SkError(rc, "sk_gemm_ex")
    return rc


def gemm_noalloc(desc: GemmDesc, opts: Options | None = None, stream=None, check=True) -> int:
    """``sk_gemm_noalloc``: the allocation-free form of ``sk_gemm_ex`` (no
    ABFT; scratch is the library's static per-GPU array)."""
    rc = _lib.sk_gemm_noalloc(ctypes.byref(desc), ctypes.byref(opts) if opts is not None else None,
                              _stream(stream))
    if check and rc != OK:
        raise SkError(rc, "sk_gemm_noalloc")
    return rc


def plan_query(desc: GemmDesc, opts: Options | None = None, slots: int = 0) -> Plan:
    """``sk_plan_query``; with slots > 0 no GPU is touched."""
    p = Plan()
    rc = _lib.sk_plan_query(ctypes.byref(desc), ctypes.byref(opts) if opts is not None else None,
                            slots, ctypes.byref(p))
    if rc != OK:
        raise SkError(rc, "sk_plan_query")
    return p


def plan_segments(plan: Plan, wg: int):
    """Segments of workgroup `wg` as tuples
    (tile, iter_begin, iter_end, started, ended, last_peer)."""
    n = _lib.sk_plan_segments(ctypes.byref(plan), wg, None, 0)
    if n < 0:
        raise SkError(int(n), "sk_plan_segments")
    buf = (Segment * max(int(n), 1))()
    _lib.sk_plan_segments(ctypes.byref(plan), wg, buf, n)
    return [(s.tile, s.iter_begin, s.iter_end, s.started, s.ended, s.last_peer)
            for s in buf[:n]]


def device_status() -> int:
    return _lib.sk_device_status()


def release_workspace() -> int:
    return _lib.sk_release_workspace()


def read_report(buf) -> AbftReport:
    """Copies a device-side report (a torch uint8 tensor) into an AbftReport."""
    host = bytes(buf.cpu().numpy().tobytes())
    return AbftReport.from_buffer_copy(host[:ctypes.sizeof(AbftReport)])
