// sk_api.cpp -- the C ABI of the Stream-K GEMM library (host side).
//
// Validates arguments, handles the BLAS quick returns, plans the work
// decomposition, manages the per-(device, stream) workspace that holds the
// partial tiles and flags of the cross-workgroup fixup, repacks operands the
// kernels cannot read directly, and launches the kernels.  Every arithmetic
// step of the GEMM runs in the HIP kernels of sk_kernels.hip.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "sk_internal.h"

namespace sk {
namespace {

thread_local std::string g_last_hip_error = "no error";

int hip_fail(hipError_t e, const char *what) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  g_last_hip_error = buf;
  return SK_ERR_HIP;
}

struct DeviceInfo {
  bool ok = false;
  int cus = 0;
  int slots[3] = {0, 0, 0};        // per dtype, large tiles
  int slots_small[3] = {0, 0, 0};  // per dtype, small tiles
  int slots_narrow[3] = {0, 0, 0}; // fp16/bf16 narrow-m instances (the fewest of the four)
  int slots_abft = 0;              // fp32 with ABFT
  int64_t wall_khz = 100000;
};

struct Workspace {
  float *partials = nullptr;
  size_t partial_bytes = 0;
  uint32_t *flags = nullptr;
  int flag_count = 0;
  // the error word, in pinned host memory mapped into the device's address
  // space: a kernel's time-out is seen by the host without a synchronisation
  int32_t *status_host = nullptr;
  int32_t *status = nullptr;  // its device address
  uint32_t epoch = 0;
  // ABFT preparation: one completion counter per tile of A and of B, zero
  // between calls (the kernel's last workgroup of a tile clears its own),
  // and the encodings and threshold inputs (calls on one stream run in
  // order, so each reuses them)
  uint32_t *abft_ctr = nullptr;
  int64_t abft_ctr_count = 0;
  float *abft_buf = nullptr;
  int64_t abft_floats = 0;
  // k-contiguous copies of A and B for operands the kernels cannot read in
  // place (calls on one stream run in order, so each reuses them)
  void *pack[2] = {nullptr, nullptr};
  size_t pack_bytes[2] = {0, 0};
};

std::mutex g_mu;
std::map<int, DeviceInfo> g_dev;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

int device_info(int dev, DeviceInfo **out) {
  auto it = g_dev.find(dev);
  if (it != g_dev.end()) {
    *out = &it->second;
    return it->second.ok ? SK_OK : SK_ERR_NO_DEVICE;
  }
  DeviceInfo &d = g_dev[dev];
  *out = &d;
  struct Forget {  // a failed probe is retried on the next call
    int dev;
    bool armed = true;
    ~Forget() { if (armed) g_dev.erase(dev); }
  } forget{dev};
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    g_last_hip_error = std::string("device is ") + prop.gcnArchName + ", the kernels are built for gfx950";
    return SK_ERR_NO_DEVICE;
  }
  d.cus = prop.multiProcessorCount;
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0)
    d.wall_khz = khz;
  // large and small tiles per dtype, and fp32 with ABFT (large tiles)
  struct Query {
    int dtype, inst;
    bool abft;
    int *slots;
  };
  const Query queries[] = {{SK_F32, 0, false, &d.slots[SK_F32]},        {SK_F16, 0, false, &d.slots[SK_F16]},
                           {SK_BF16, 0, false, &d.slots[SK_BF16]},      {SK_F32, 0, true, &d.slots_abft},
                           {SK_F32, 1, false, &d.slots_small[SK_F32]},  {SK_F16, 1, false, &d.slots_small[SK_F16]},
                           {SK_BF16, 1, false, &d.slots_small[SK_BF16]}};
  for (const Query &q : queries) {
    int occ = 0;
    e = (hipError_t)kernel_occupancy(q.dtype, q.abft, q.inst, &occ);
    if (e != hipSuccess) return hip_fail(e, "occupancy query");
    const int want = tile_cfg(q.dtype, q.inst).occupancy;
    if (occ < 1) {
      g_last_hip_error = "kernel does not fit on a CU";
      return SK_ERR_HIP;
    }
    *q.slots = d.cus * (occ < want ? occ : want);
  }
  // fp16, bf16 narrow-m instances: one workgroup per CU each
  for (int dtype = SK_F16; dtype <= SK_BF16; ++dtype) {
    int fewest = 1 << 30;
    for (int inst = 2; inst <= 5; ++inst) {
      int occ = 0;
      e = (hipError_t)kernel_occupancy(dtype, false, inst, &occ);
      if (e != hipSuccess) return hip_fail(e, "occupancy query");
      if (occ < 1) {
        g_last_hip_error = "kernel does not fit on a CU";
        return SK_ERR_HIP;
      }
      const int want = tile_cfg(dtype, inst).occupancy;
      fewest = std::min(fewest, occ < want ? occ : want);
    }
    d.slots_narrow[dtype] = d.cus * fewest;
  }
  d.ok = true;
  forget.armed = false;
  return SK_OK;
}

__global__ void init_flags_kernel(uint32_t *flags, int n, int32_t *status) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) flags[i] = 0;
  if (status != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *status = 0;
}

// Scratch of the allocation-free entry point (sk_gemm_noalloc): one static
// device array per GPU, held until the process ends.  Layout: the status
// word at byte 0, kScratchFlags flags from byte 256, the partial-tile slots
// from byte kScratchHead.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device with hipGetSymbolAddress and kept.
constexpr int kScratchFlags = 16384;
constexpr size_t kScratchHead = 128 * 1024;
constexpr size_t kScratchPartialBytes = SK_NOALLOC_PARTIAL_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchHead + kScratchPartialBytes];

struct NoAlloc {
  char *ptr = nullptr;  // device address of `scratch` on this device
  uint32_t epoch = 0;
};
std::map<int, NoAlloc> g_noalloc;

// Set-up of the scratch on device `dev` (current), once: its address, and
// the flags and status word cleared by a fill kernel on `stream`.  Caller
// holds g_mu.
int noalloc_state(int dev, hipStream_t stream, NoAlloc **out) {
  NoAlloc &s = g_noalloc[dev];
  if (s.ptr == nullptr) {
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      g_noalloc.erase(dev);
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    }
    char *base = static_cast<char *>(p);
    hipLaunchKernelGGL(init_flags_kernel, dim3(16), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t *>(base + 256), kScratchFlags,
                       reinterpret_cast<int32_t *>(base));
    e = hipGetLastError();
    if (e != hipSuccess) {
      g_noalloc.erase(dev);
      return hip_fail(e, "scratch set-up");
    }
    s.ptr = base;
  }
  *out = &s;
  return SK_OK;
}

// Workspace of (dev, stream) with room for `slots` partial tiles of
// `tile_bytes` each.  Caller holds g_mu.
int get_workspace(int dev, hipStream_t stream, int64_t slots, size_t tile_bytes, Workspace **out) {
  Workspace &w = g_ws[{dev, stream}];
  const size_t need = (size_t)slots * tile_bytes;
  const size_t base = (size_t)256 * 256 * 256 * 4;  // 256 slots of the largest tile: 64 MiB
  if (w.partials == nullptr || w.partial_bytes < need || w.flag_count < slots) {
    int32_t *keep_host = nullptr, *keep_dev = nullptr;
    if (w.partials) {  // growth: wait for work that may still use the old buffers
      hipError_t e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      (void)hipFree(w.partials);
      (void)hipFree(w.flags);
      keep_host = w.status_host;  // the error word survives growth (it may hold a report)
      keep_dev = w.status;
      Workspace keep_abft;  // so do the ABFT buffers (the counters are zero) and the repack copies
      keep_abft.abft_ctr = w.abft_ctr;
      keep_abft.abft_ctr_count = w.abft_ctr_count;
      keep_abft.abft_buf = w.abft_buf;
      keep_abft.abft_floats = w.abft_floats;
      for (int i = 0; i < 2; ++i) {
        keep_abft.pack[i] = w.pack[i];
        keep_abft.pack_bytes[i] = w.pack_bytes[i];
      }
      w = keep_abft;
    }
    size_t bytes = need > base ? need : base;
    int nflags = slots > 1024 ? (int)slots : 1024;
    hipError_t e = hipMalloc(&w.partials, bytes);
    if (e != hipSuccess) {
      w.partials = nullptr;
      w.status_host = keep_host;
      w.status = keep_dev;
      (void)hipGetLastError();
      return SK_ERR_NO_MEMORY;
    }
    e = hipMalloc(&w.flags, sizeof(uint32_t) * nflags);
    if (e == hipSuccess && keep_host == nullptr) {
      e = hipHostMalloc(reinterpret_cast<void **>(&keep_host), sizeof(int32_t),
                        hipHostMallocMapped | hipHostMallocCoherent);
      if (e == hipSuccess) {
        *keep_host = 0;
        e = hipHostGetDevicePointer(reinterpret_cast<void **>(&keep_dev), keep_host, 0);
        if (e != hipSuccess) {
          (void)hipHostFree(keep_host);
          keep_host = nullptr;
        }
      }
    }
    if (e != hipSuccess) {
      (void)hipFree(w.partials);
      (void)hipFree(w.flags);
      w.partials = nullptr;
      w.flags = nullptr;
      (void)hipGetLastError();
      return SK_ERR_NO_MEMORY;
    }
    w.status_host = keep_host;
    w.status = keep_dev;
    w.partial_bytes = bytes;
    w.flag_count = nflags;
    w.epoch = 0;
    hipLaunchKernelGGL(init_flags_kernel, dim3(4), dim3(256), 0, stream, w.flags, nflags, nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "workspace init");
  }
  *out = &w;
  return SK_OK;
}

// Repack copy `which` (0: A, 1: B) of at least `bytes` in workspace `w` of
// `stream`, grown (never shrunk) after the stream's earlier work is done with
// the old one.  Caller holds g_mu.
int get_pack_buffer(Workspace &w, hipStream_t stream, int which, size_t bytes, void **out) {
  if (w.pack[which] == nullptr || w.pack_bytes[which] < bytes) {
    if (w.pack[which] != nullptr) {
      hipError_t e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      (void)hipFree(w.pack[which]);
      w.pack[which] = nullptr;
      w.pack_bytes[which] = 0;
    }
    const size_t n = (bytes + ((size_t)1 << 20) - 1) >> 20 << 20;  // whole MiB
    hipError_t e = hipMalloc(&w.pack[which], n);
    if (e != hipSuccess) {
      w.pack[which] = nullptr;
      (void)hipGetLastError();
      return SK_ERR_NO_MEMORY;
    }
    w.pack_bytes[which] = n;
  }
  *out = w.pack[which];
  return SK_OK;
}

// Workgroups of the ABFT preparation launch (four per compute unit): enough
// loads in flight to stream the operands, each workgroup walking several
// chunks so that its completion count is paid once per group.
constexpr int64_t kPrepBlocks = 1024;

// At least `count` zeroed ABFT counters and `floats` floats of ABFT buffer
// in workspace `w` of `stream`.  Caller holds g_mu.
int get_abft_buffers(Workspace &w, hipStream_t stream, int64_t count, int64_t floats) {
  if (count > INT32_MAX) return SK_ERR_TOO_LARGE;
  const bool grow_ctr = w.abft_ctr == nullptr || w.abft_ctr_count < count;
  const bool grow_buf = w.abft_buf == nullptr || w.abft_floats < floats;
  if (!grow_ctr && !grow_buf) return SK_OK;
  if (w.abft_ctr != nullptr || w.abft_buf != nullptr) {  // growth: wait for work that may still use them
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  }
  if (grow_buf) {
    (void)hipFree(w.abft_buf);
    w.abft_buf = nullptr;
    w.abft_floats = 0;
    const int64_t n = floats > (1 << 20) ? floats : (1 << 20);
    hipError_t e = hipMalloc(reinterpret_cast<void **>(&w.abft_buf), sizeof(float) * (size_t)n);
    if (e != hipSuccess) {
      w.abft_buf = nullptr;
      (void)hipGetLastError();
      return SK_ERR_NO_MEMORY;
    }
    w.abft_floats = n;
  }
  if (grow_ctr) {
    (void)hipFree(w.abft_ctr);
    w.abft_ctr = nullptr;
    w.abft_ctr_count = 0;
    const int64_t n = count > 1024 ? count : 1024;
    hipError_t e = hipMalloc(reinterpret_cast<void **>(&w.abft_ctr), sizeof(uint32_t) * n);
    if (e != hipSuccess) {
      w.abft_ctr = nullptr;
      (void)hipGetLastError();
      return SK_ERR_NO_MEMORY;
    }
    hipLaunchKernelGGL(init_flags_kernel, dim3(4), dim3(256), 0, stream, w.abft_ctr, (int)n, nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "ABFT counter init");
    w.abft_ctr_count = n;
  }
  return SK_OK;
}

// A fixup time-out that a kernel of this device has written to a
// workspace's (host-mapped) error word since the last report: reported once,
// by the next call that starts after the word was written (the call then
// launches nothing), or by sk_device_status.  Caller holds g_mu.
int take_timeout_report(int dev) {
  for (auto &kv : g_ws) {
    if (kv.first.first != dev || kv.second.status_host == nullptr) continue;
    volatile int32_t *w = kv.second.status_host;
    if (*w & 1) {
      *w = 0;
      return SK_ERR_FIXUP_TIMEOUT;
    }
  }
  return SK_OK;
}

bool a_kmajor_of(int layout) { return layout == SK_A_ROW_B_ROW || layout == SK_A_ROW_B_COL; }
bool b_kmajor_of(int layout) { return layout == SK_A_ROW_B_COL || layout == SK_A_COL_B_COL; }

int validate(const sk_gemm_desc &d, const sk_options &o, const sk_abft_report *report) {
  if (d.m < 0 || d.n < 0 || d.k < 0) return SK_ERR_INVALID_ARG;
  if (d.dtype != SK_F32 && d.dtype != SK_F16 && d.dtype != SK_BF16) return SK_ERR_INVALID_ARG;
  if (d.layout < SK_A_ROW_B_ROW || d.layout > SK_A_COL_B_COL) return SK_ERR_INVALID_ARG;
  if (o.schedule < SK_SCHED_AUTO || o.schedule > SK_SCHED_GEMV_SPLIT) return SK_ERR_INVALID_ARG;
  if (o.forced_grid < 0 || o.hybrid_min_waves < 0 || o.n_faults < 0 || o.spin_limit_us < 0)
    return SK_ERR_INVALID_ARG;
  if (o.n_faults > 0 && o.faults == nullptr) return SK_ERR_INVALID_ARG;
  if (o.test_flags & ~SK_TEST_NO_SIGNAL) return SK_ERR_INVALID_ARG;
  if (o.abft && d.dtype != SK_F32) return SK_ERR_UNSUPPORTED;
  if (o.abft && report == nullptr) return SK_ERR_INVALID_ARG;
  if (d.m == 0 || d.n == 0) return SK_OK;
  if (d.C == nullptr || d.ldc < d.n) return SK_ERR_INVALID_ARG;
  if (d.k > 0 && d.alpha != 0.f) {
    if (d.A == nullptr || d.B == nullptr) return SK_ERR_INVALID_ARG;
    const int64_t a_min = a_kmajor_of(d.layout) ? d.k : d.m;
    const int64_t b_min = b_kmajor_of(d.layout) ? d.k : d.n;
    if (d.lda < (a_min > 1 ? a_min : 1) || d.ldb < (b_min > 1 ? b_min : 1)) return SK_ERR_INVALID_ARG;
  }
  return SK_OK;
}

// noalloc: the allocation-free form (sk_gemm_noalloc): partials, flags and
// status come from the static scratch; nothing is allocated, and calls that
// would need an allocation (ABFT encodings, repacked operands) or more
// scratch than it holds are refused.
int gemm_impl(const sk_gemm_desc &d, const sk_options &o, sk_abft_report *report, hipStream_t stream,
              bool noalloc = false) {
  if (noalloc && o.abft) return SK_ERR_UNSUPPORTED;
  int rc = validate(d, o, report);
  if (rc != SK_OK) return rc;
  if (d.m == 0 || d.n == 0) return SK_OK;  // nothing to compute or write
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceInfo *info = nullptr;
  rc = device_info(dev, &info);
  if (rc != SK_OK) return rc;
  NoAlloc *na = nullptr;
  if (noalloc) {
    rc = noalloc_state(dev, stream, &na);
    if (rc != SK_OK) return rc;
  } else {
    rc = take_timeout_report(dev);
    if (rc != SK_OK) return rc;
  }
  if (d.k == 0 || d.alpha == 0.f) {  // C = beta * C
    if (o.abft) {  // (the GEMM path zeroes the report in its ABFT preparation)
      rc = launch_zero_report(report, stream);
      if (rc != hipSuccess) return hip_fail((hipError_t)rc, "report reset");
    }
    rc = launch_scale(d.dtype, d.m, d.n, d.beta, d.C, d.ldc, stream);
    return rc == hipSuccess ? SK_OK : hip_fail((hipError_t)rc, "scale kernel");
  }
  // matrix-vector products: the even split of dot products
  if (o.schedule == SK_SCHED_GEMV_SPLIT ||
      (o.schedule == SK_SCHED_AUTO && !o.abft && o.forced_grid == 0 && o.tile == SK_TILE_AUTO)) {
    GemvPlan g;
    if (!o.abft && gemv_plan(d, info->cus, g)) {
      float *part = nullptr;
      if (g.S > 1) {
        const size_t need = (size_t)(g.S * g.R * g.V) * sizeof(float);
        if (noalloc) {
          if (need > kScratchPartialBytes) return SK_ERR_TOO_LARGE;
          part = reinterpret_cast<float *>(na->ptr + kScratchHead);
        } else {
          Workspace *ws = nullptr;
          rc = get_workspace(dev, stream, 1, need, &ws);
          if (rc != SK_OK) return rc;
          part = ws->partials;
        }
      }
      rc = launch_gemv(d.dtype, g, part, d.alpha, d.beta, stream);
      return rc == hipSuccess ? SK_OK : hip_fail((hipError_t)rc, "matrix-vector kernel launch");
    }
    if (o.schedule == SK_SCHED_GEMV_SPLIT) return SK_ERR_UNSUPPORTED;
  }
  Plan P;
  const int slots[3] = {o.abft && d.dtype == SK_F32 ? info->slots_abft : info->slots[d.dtype],
                        info->slots_small[d.dtype], d.dtype == SK_F32 ? 1 : info->slots_narrow[d.dtype]};
  rc = make_plan(d, o, slots, P);
  if (rc != SK_OK) return rc;
  const int es = d.dtype == SK_F32 ? 4 : 2;
  const bool ak = a_kmajor_of(d.layout), bk = b_kmajor_of(d.layout);
  if (noalloc) {
    if (P.pack_a || P.pack_b) return SK_ERR_UNSUPPORTED;
    if (P.grid > kScratchFlags || (size_t)P.grid * P.cfg.bm * P.cfg.bn * 4 > kScratchPartialBytes)
      return SK_ERR_TOO_LARGE;
  }

  // operands: direct, or repacked into a k-contiguous copy
  const int64_t kp = (d.k + 63) / 64 * 64;
  const TileCfg &c = P.cfg;
  KernelArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = d.A; a.lda = d.lda; a.a_kmajor = ak; a.a_kext = (int32_t)d.k;
  a.B = d.B; a.ldb = d.ldb; a.b_kmajor = bk; a.b_kext = (int32_t)d.k;
  // 32-bit buffer offsets inside a k-major tile: rows * ld * es must fit
  auto offsets_fit = [&](bool kmaj, int64_t ld, int rows) {
    const int64_t span = kmaj ? (int64_t)rows * ld * es : (int64_t)c.bk * ld * es;
    return span + 1024 < 0x7FFFFFFF;
  };
  if (!offsets_fit(P.pack_a ? true : ak, P.pack_a ? kp : d.lda, c.bm) ||
      !offsets_fit(P.pack_b ? true : bk, P.pack_b ? kp : d.ldb, c.bn))
    return SK_ERR_UNSUPPORTED;

  float *partials = nullptr;
  uint32_t *flags = nullptr, epoch = 0;
  int32_t *status = nullptr;
  Workspace *ws = nullptr;  // (every call but the allocation-free one)
  if (noalloc) {
    partials = reinterpret_cast<float *>(na->ptr + kScratchHead);
    flags = reinterpret_cast<uint32_t *>(na->ptr + 256);
    status = reinterpret_cast<int32_t *>(na->ptr);
    if (++na->epoch == 0) na->epoch = 1;
    epoch = na->epoch;
  } else {
    const int64_t slots_needed = P.grid;
    rc = get_workspace(dev, stream, slots_needed, (size_t)c.bm * c.bn * 4, &ws);
    if (rc != SK_OK) return rc;
    if (++ws->epoch == 0) ws->epoch = 1;
    partials = ws->partials; flags = ws->flags; status = ws->status; epoch = ws->epoch;
  }
  if (P.pack_a) {  // (never in the allocation-free form: refused above)
    void *pa = nullptr;
    rc = get_pack_buffer(*ws, stream, 0, (size_t)d.m * kp * es, &pa);
    if (rc != SK_OK) return rc;
    rc = launch_pack(d.dtype, d.A, d.lda, ak, d.m, d.k, pa, kp, stream);
    if (rc != hipSuccess) return hip_fail((hipError_t)rc, "pack A");
    a.A = pa; a.lda = kp; a.a_kmajor = 1; a.a_kext = (int32_t)kp;
  }
  if (P.pack_b) {
    void *pb = nullptr;
    rc = get_pack_buffer(*ws, stream, 1, (size_t)d.n * kp * es, &pb);
    if (rc != SK_OK) return rc;
    rc = launch_pack(d.dtype, d.B, d.ldb, bk, d.n, d.k, pb, kp, stream);
    if (rc != hipSuccess) return hip_fail((hipError_t)rc, "pack B");
    a.B = pb; a.ldb = kp; a.b_kmajor = 1; a.b_kext = (int32_t)kp;
  }

  a.C = d.C; a.ldc = d.ldc;
  a.m = (int32_t)d.m; a.n = (int32_t)d.n; a.k = (int32_t)d.k;
  a.alpha = d.alpha; a.beta = d.beta;
  a.tiles_m = (int32_t)P.tiles_m; a.tiles_n = (int32_t)P.tiles_n;
  a.tiles = (int32_t)P.tiles; a.ipt = (int32_t)P.ipt;
  a.sched = P.sched();
  a.partials = partials; a.flags = flags; a.epoch = epoch; a.status = status;
  const int64_t us = o.spin_limit_us > 0 ? o.spin_limit_us : 2000000;
  a.spin_limit = us * info->wall_khz / 1000;
  a.no_signal = (o.test_flags & SK_TEST_NO_SIGNAL) ? 1 : 0;
  a.abft = o.abft; a.n_faults = o.n_faults; a.faults = o.faults; a.report = report;
  a.abft_tau = o.abft_tau > 0 ? o.abft_tau : 1.0f;

  // ABFT: the encodings of every tile row of A and tile column of B and the
  // detection-threshold inputs, formed once from the operands the kernel
  // reads, in the stream's workspace, by one preparation launch
  if (o.abft) {
    const int64_t kb = P.ipt, chunks = (kb * 32 + 63) / 64;
    // about kPrepBlocks workgroups, each walking a group of chunks
    const int64_t tiles2 = P.tiles_m + P.tiles_n;
    int64_t groups = (kPrepBlocks + tiles2 - 1) / tiles2;
    if (groups > chunks) groups = chunks;
    const int64_t gsize = (chunks + groups - 1) / groups;
    groups = (chunks + gsize - 1) / gsize;
    const int64_t ea = P.tiles_m * kb * 32, eb = P.tiles_n * kb * 32;
    const int64_t ra_ = d.m * groups, rb_ = d.n * groups, ta = P.tiles_m * groups, tb = P.tiles_n * groups;
    const int64_t floats = ea + eb + ra_ + rb_ + ta + tb + d.m + d.n + P.tiles_m + P.tiles_n;
    rc = get_abft_buffers(*ws, stream, P.tiles_m + P.tiles_n, floats);
    if (rc != SK_OK) return rc;
    float *p_ea = ws->abft_buf, *p_eb = p_ea + ea, *p_ra = p_eb + eb, *p_rb = p_ra + ra_, *p_ta = p_rb + rb_,
          *p_tb = p_ta + ta, *p_na = p_tb + tb, *p_nb = p_na + d.m, *p_ma = p_nb + d.n, *p_mb = p_ma + P.tiles_m;
    AbftPrepArgs pr;
    pr.op[0] = AbftPrepOperand{static_cast<const float *>(a.A), a.lda, a.a_kmajor, d.m, P.tiles_m,
                               p_ea, p_ra, p_ta, p_na, p_ma};
    pr.op[1] = AbftPrepOperand{static_cast<const float *>(a.B), a.ldb, a.b_kmajor, d.n, P.tiles_n,
                               p_eb, p_rb, p_tb, p_nb, p_mb};
    pr.k = d.k; pr.kb = kb; pr.chunks = chunks; pr.group_chunks = gsize; pr.groups = groups;
    pr.counters = ws->abft_ctr;
    pr.report = report;
    rc = launch_abft_prep(pr, stream);
    if (rc != hipSuccess) return hip_fail((hipError_t)rc, "ABFT preparation kernel");
    a.enc_a = p_ea; a.enc_b = p_eb; a.enc_kb = (int32_t)kb;
    a.norm_a = p_na; a.norm_b = p_nb; a.emax_a = p_ma; a.emax_b = p_mb;
  }

  rc = launch_gemm(P, a, stream);
  if (rc != hipSuccess) return hip_fail((hipError_t)rc, "GEMM kernel launch");
  return SK_OK;
}

const sk_options kDefaultOpts = {};

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

int sk_gemm(int64_t m, int64_t n, int64_t k, float alpha, const void *A, int64_t lda, const void *B,
            int64_t ldb, float beta, void *C, int64_t ldc, sk_dtype dtype, sk_layout layout,
            hipStream_t stream) {
  sk_gemm_desc d{m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, dtype, layout};
  try {
    return gemm_impl(d, kDefaultOpts, nullptr, stream);
  } catch (...) {
    return SK_ERR_NO_MEMORY;
  }
}

int sk_gemm_ex(const sk_gemm_desc *desc, const sk_options *opts, sk_abft_report *report,
               hipStream_t stream) {
  if (!desc) return SK_ERR_INVALID_ARG;
  try {
    return gemm_impl(*desc, opts ? *opts : kDefaultOpts, report, stream);
  } catch (...) {
    return SK_ERR_NO_MEMORY;
  }
}

int sk_gemm_noalloc(const sk_gemm_desc *desc, const sk_options *opts, hipStream_t stream) {
  if (!desc) return SK_ERR_INVALID_ARG;
  try {
    return gemm_impl(*desc, opts ? *opts : kDefaultOpts, nullptr, stream, true);
  } catch (...) {
    return SK_ERR_NO_MEMORY;
  }
}

int sk_plan_query(const sk_gemm_desc *desc, const sk_options *opts, int32_t slots, sk_plan *out) {
  if (!desc || !out || slots < 0) return SK_ERR_INVALID_ARG;
  const sk_options &o = opts ? *opts : kDefaultOpts;
  try {
    int slots2 = 0, slots3 = 0;  // small-tile and narrow-m instances
    if (slots == 0) {
      int dev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
      std::lock_guard<std::mutex> lock(g_mu);
      DeviceInfo *info = nullptr;
      int rc = device_info(dev, &info);
      if (rc != SK_OK) return rc;
      if (desc->dtype < 0 || desc->dtype > 2) return SK_ERR_INVALID_ARG;
      slots = o.abft && desc->dtype == SK_F32 ? info->slots_abft : info->slots[desc->dtype];
      slots2 = info->slots_small[desc->dtype];
      slots3 = desc->dtype == SK_F32 ? 1 : info->slots_narrow[desc->dtype];
    }
    if (slots2 == 0) slots2 = 2 * slots;
    if (slots3 == 0) slots3 = slots;
    GemvPlan g;
    if ((o.schedule == SK_SCHED_GEMV_SPLIT ||
         (o.schedule == SK_SCHED_AUTO && !o.abft && o.forced_grid == 0 && o.tile == SK_TILE_AUTO)) &&
        desc->dtype >= 0 && desc->dtype <= 2 && desc->layout >= 0 && desc->layout <= 3 && !o.abft &&
        desc->m >= 0 && desc->n >= 0 && gemv_plan(*desc, desc->dtype == SK_F32 ? slots / 2 : slots, g)) {
      std::memset(out, 0, sizeof(*out));
      out->schedule = SK_SCHED_GEMV_SPLIT;
      out->slots = slots;
      out->grid = g.grid;
      out->tile_k = (int32_t)g.chunk;
      out->tiles = g.R;
      out->iters_per_tile = 1;
      out->sk_blocks = (int32_t)g.S;
      if (g.form == kGemvAxpy) {  // outputs per task: one wave's width
        out->tile_n = (desc->dtype == SK_F32 ? 4 : 8) * 64;
        out->total_iters = (g.R + out->tile_n - 1) / out->tile_n * g.S;
      } else if (g.form == kGemvMulti) {  // vectors x rows per task
        out->tile_m = g.V;
        out->tile_n = desc->dtype == SK_F32 ? 64 : 16;
        out->tiles = (int64_t)g.V * g.R;
        out->total_iters = (g.R + out->tile_n - 1) / out->tile_n * g.S;
      } else {
        out->total_iters = g.R * g.S;
      }
      return SK_OK;
    }
    const int both[3] = {slots, slots2, slots3};
    Plan P;
    int rc = make_plan(*desc, o, both, P);
    if (rc != SK_OK) return rc;
    std::memset(out, 0, sizeof(*out));
    out->tile_m = P.cfg.bm; out->tile_n = P.cfg.bn; out->tile_k = P.cfg.bk;
    out->slots = P.slots; out->grid = P.grid; out->schedule = P.schedule;
    out->tiles_m = P.tiles_m; out->tiles_n = P.tiles_n; out->tiles = P.tiles;
    out->iters_per_tile = P.ipt; out->total_iters = P.total;
    out->sk_tiles = P.sk_tiles; out->sk_iters_q = P.sk_q; out->sk_iters_r = P.sk_r;
    out->dp_tiles = P.dp_tiles; out->full_waves = P.w; out->tail_tiles = P.r;
    out->max_peers = plan_max_peers(P);
    out->packs = (P.pack_a ? 1 : 0) | (P.pack_b ? 2 : 0);
    out->phase_div = P.phase_div; out->sk_blocks = P.blocks; out->group_rows = P.group_rows;
    out->fixup_tree = P.sched().tree ? 1 : 0;
    return SK_OK;
  } catch (...) {
    return SK_ERR_NO_MEMORY;
  }
}

int sk_device_status(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SK_ERR_HIP;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  int result = take_timeout_report(dev);
  for (auto &kv : g_ws)  // every workspace's word is read and cleared
    if (kv.first.first == dev && kv.second.status_host) {
      if (*static_cast<volatile int32_t *>(kv.second.status_host) & 1) result = SK_ERR_FIXUP_TIMEOUT;
      *static_cast<volatile int32_t *>(kv.second.status_host) = 0;
    }
  auto na = g_noalloc.find(dev);
  if (na != g_noalloc.end() && na->second.ptr) {  // the allocation-free entry point's word: device memory
    int32_t *w = reinterpret_cast<int32_t *>(na->second.ptr);
    int32_t v = 0;
    e = hipMemcpy(&v, w, sizeof(v), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "status read");
    if (v & 1) result = SK_ERR_FIXUP_TIMEOUT;
    if (v) {
      const int32_t zero = 0;
      e = hipMemcpy(w, &zero, sizeof(zero), hipMemcpyHostToDevice);
      if (e != hipSuccess) return hip_fail(e, "status clear");
    }
  }
  return result;
}

const char *sk_strerror(int status) {
  switch (status) {
    case SK_OK: return "success";
    case SK_ERR_INVALID_ARG: return "invalid argument";
    case SK_ERR_UNSUPPORTED: return "unsupported argument combination";
    case SK_ERR_NO_MEMORY: return "workspace allocation failed";
    case SK_ERR_HIP: return "HIP runtime error";
    case SK_ERR_FIXUP_TIMEOUT: return "a workgroup timed out waiting for a partial tile";
    case SK_ERR_NO_DEVICE: return "no usable gfx950 device";
    case SK_ERR_TOO_LARGE: return "the call needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

const char *sk_last_hip_error(void) { return g_last_hip_error.c_str(); }

int sk_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ws.empty()) return SK_OK;
  hipError_t e = hipDeviceSynchronize();
  for (auto &kv : g_ws) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(kv.first.first);
    (void)hipFree(kv.second.partials);
    (void)hipFree(kv.second.flags);
    (void)hipFree(kv.second.abft_ctr);
    (void)hipFree(kv.second.abft_buf);
    (void)hipFree(kv.second.pack[0]);
    (void)hipFree(kv.second.pack[1]);
    (void)hipHostFree(kv.second.status_host);
    (void)hipSetDevice(cur);
  }
  g_ws.clear();
  return e == hipSuccess ? SK_OK : hip_fail(e, "hipDeviceSynchronize");
}

const char *sk_version(void) { return "sk_gemm 0.1 (gfx950)"; }

}  // extern "C"
