// sk_kernels.hip -- Stream-K GEMM kernels for CDNA4 (gfx950).
//
// One persistent kernel per element type runs every work segment of its
// workgroup (Stream-K page, Algorithm 5 and the section 5.2 hybrids): first
// the Stream-K segments, then the data-parallel tiles.  A segment is the
// MacLoop of Algorithm 3 over k-iterations [lb, le) of one output tile,
// followed by
//  * a partial store + flag release when the segment does not hold the
//    tile's first iteration (Algorithm 5, StorePartials / Signal), or
//  * an acquire-wait on each peer's flag and the sum of its partial (Wait /
//    LoadPartials) when it holds the first iteration but not the last, then
//  * the epilogue C = alpha * acc + beta * C (StoreTile).
//
// Data movement (the fault-tolerant GEMM page's SGEMM ladder -- shared-memory
// tiling, 128-bit accesses, double-buffered prefetch -- recast for CDNA4):
//  * global -> LDS: 128-bit buffer loads that write straight into LDS (no
//    register staging), two LDS stages, one barrier per k-iteration; the
//    loads of iteration i+1 are in flight while iteration i computes;
//  * out-of-range rows and k-chunks are fetched with an offset beyond the
//    buffer's range, which the buffer unit answers with zeros;
//  * LDS layouts are XOR-swizzled at 16-byte granularity so that the
//    fragment reads of 16 lanes (one 256-byte LDS cycle on gfx950's 64 banks)
//    touch 16 distinct bank groups;
//  * LDS -> registers -> MFMA: each wave64 owns a register tile of C; the
//    product is formed as C^T = B^T A^T so that every lane holds four
//    consecutive columns of one row of C (vector epilogue stores).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sk_internal.h"

namespace sk {
namespace dev {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef __bf16 b4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void *lds_vptr;

constexpr uint32_t kOOB = 0x80000000u;  // offset past every buffer range (ranges are < 2^31)
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

extern __shared__ __attribute__((aligned(1024))) char smem[];

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char *base, int64_t bytes) {
  int32_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, n, kRsrcWord3);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int lds_off, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(smem + lds_off), 16, voff, 0, 0, 0);
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// ---------------------------------------------------------------- elements

template <int DT> struct Elem;
template <> struct Elem<SK_F16> {
  using T = _Float16;
  using V8 = h8_t;
  static __device__ __forceinline__ f4_t mfma(V8 a, V8 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float ld(const void *p, int64_t i) {
    return (float)static_cast<const T *>(p)[i];
  }
  static __device__ __forceinline__ void st(void *p, int64_t i, float v) {
    static_cast<T *>(p)[i] = (T)v;
  }
  static __device__ __forceinline__ void st4(void *p, int64_t i, f4_t v) {
    h4_t h = {(T)v[0], (T)v[1], (T)v[2], (T)v[3]};
    *reinterpret_cast<h4_t *>(static_cast<T *>(p) + i) = h;
  }
  static __device__ __forceinline__ f4_t ld4(const void *p, int64_t i) {
    h4_t h = *reinterpret_cast<const h4_t *>(static_cast<const T *>(p) + i);
    return f4_t{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  }
};
template <> struct Elem<SK_BF16> {
  using T = __bf16;
  using V8 = b8_t;
  static __device__ __forceinline__ f4_t mfma(V8 a, V8 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float ld(const void *p, int64_t i) {
    return (float)static_cast<const T *>(p)[i];
  }
  static __device__ __forceinline__ void st(void *p, int64_t i, float v) {
    static_cast<T *>(p)[i] = (T)v;
  }
  static __device__ __forceinline__ void st4(void *p, int64_t i, f4_t v) {
    b4_t h = {(T)v[0], (T)v[1], (T)v[2], (T)v[3]};
    *reinterpret_cast<b4_t *>(static_cast<T *>(p) + i) = h;
  }
  static __device__ __forceinline__ f4_t ld4(const void *p, int64_t i) {
    b4_t h = *reinterpret_cast<const b4_t *>(static_cast<const T *>(p) + i);
    return f4_t{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  }
};
template <> struct Elem<SK_F32> {
  using T = float;
  static __device__ __forceinline__ float ld(const void *p, int64_t i) {
    return static_cast<const float *>(p)[i];
  }
  static __device__ __forceinline__ void st(void *p, int64_t i, float v) {
    static_cast<float *>(p)[i] = v;
  }
  static __device__ __forceinline__ void st4(void *p, int64_t i, f4_t v) {
    *reinterpret_cast<f4_t *>(static_cast<float *>(p) + i) = v;
  }
  static __device__ __forceinline__ f4_t ld4(const void *p, int64_t i) {
    return *reinterpret_cast<const f4_t *>(static_cast<const float *>(p) + i);
  }
};

// ------------------------------------------------------ cross-WG fixup
//
// Partial tiles live in the workgroup's slot in the same per-lane order as
// the accumulators (float4 i of thread t at slot[i * NT + t]), so the store
// and the owner's load are both fully coalesced 16-byte accesses.
// Ordering: every thread's stores complete before the workgroup barrier; the
// flag is then published with an agent-scope release (which writes the
// XCD's L2 back, so that a workgroup on another XCD sees the data), and the
// owner reads the flag with agent-scope acquire semantics (invalidating its
// own stale cached copies) before any thread loads the partial.

template <int NT, int NACC>
__device__ __forceinline__ void store_partial(const KernelArgs &a, int x, const f4_t (&acc)[NACC]) {
  f4_t *slot = reinterpret_cast<f4_t *>(a.partials) + (int64_t)x * NACC * NT;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NACC; ++i) slot[i * NT + t] = acc[i];
  __syncthreads();
  if (t == 0) __hip_atomic_store(a.flags + x, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns false if the wait timed out (the status word is set).
__device__ __forceinline__ bool wait_flag(const KernelArgs &a, int peer) {
  __shared__ int ok_s;
  if (threadIdx.x == 0) {
    int ok = 1;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(a.flags + peer, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.epoch) {
      __builtin_amdgcn_s_sleep(1);
      if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > a.spin_limit) {
        atomicOr(a.status, 1);
        ok = 0;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    ok_s = ok;
  }
  __syncthreads();
  return ok_s != 0;
}

template <int NT, int NACC>
__device__ __forceinline__ void add_partial(const KernelArgs &a, int peer, f4_t (&acc)[NACC]) {
  const f4_t *slot = reinterpret_cast<const f4_t *>(a.partials) + (int64_t)peer * NACC * NT;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] += slot[i * NT + t];
}

// ------------------------------------------------------------ epilogue
//
// Lane (l) of a wave holds, for accumulator block (mb, nb), row
// r0 + mb*16 + (l & 15) and columns c0 + nb*16 + 4*(l >> 4) + {0..3}.
template <int DT, int MB, int NB>
__device__ __forceinline__ void epilogue(const KernelArgs &a, bool vec_ok, int row0, int col0,
                                         const f4_t (&acc)[MB * NB]) {
  using E = Elem<DT>;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int i = row0 + mb * 16 + (lane & 15);
    if (i >= a.m) continue;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int j = col0 + nb * 16 + 4 * (lane >> 4);
      if (j >= a.n) continue;
      const int64_t off = (int64_t)i * a.ldc + j;
      f4_t v = acc[mb * NB + nb] * a.alpha;
      if (vec_ok && j + 3 < a.n) {
        if (a.beta != 0.f) v += a.beta * E::ld4(a.C, off);
        E::st4(a.C, off, v);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (j + e < a.n) {
            float o = v[e];
            if (a.beta != 0.f) o += a.beta * E::ld(a.C, off + e);
            E::st(a.C, off + e, o);
          }
        }
      }
    }
  }
}

// --------------------------------------------------------- tile loaders
//
// K-major operand tile: R rows (m or n) x BKB bytes of k per row, row-major
// in LDS with 16-byte chunk c of row r stored at chunk position
// c ^ ((r >> 1) & 7) (8 chunks per 128-byte row).  One 1 KiB direct-to-LDS
// instruction per wave covers 8 rows; lane L writes position L & 7 of row
// L >> 3 and therefore fetches the chunk that belongs there.
//   base: element (row0, k0) of the operand; rows_left = rows of the operand
//   from row0; kbytes_left = bytes of k from k0; total: bytes from base to
//   the end of the operand.
template <int R, int NT>
__device__ __forceinline__ void load_kmajor_128(int lds_off, const char *base, int64_t ld_bytes,
                                                int rows_left, int kbytes_left, int64_t total) {
  static_assert(R * 128 % (NT / 64 * 1024) == 0, "tile must split evenly over the waves");
  constexpr int PER_WAVE = R * 128 / 1024 / (NT / 64);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, total);
  const int w = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int inst = w * PER_WAVE + j;
    const int row = inst * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    const bool ok = row < rows_left && c * 16 < kbytes_left;
    const uint32_t voff = ok ? (uint32_t)(row * ld_bytes + c * 16) : kOOB;
    dma16(rs, lds_off + inst * 1024, voff);
  }
}

// MN-major fp32 operand tile: BK rows (k) x 128 floats (512 bytes) per row,
// 16-byte chunk c of row k stored at position c ^ (4 * ((k >> 2) & 3)).  One
// instruction covers two rows.
template <int BK, int NT>
__device__ __forceinline__ void load_mnmajor_f32x128(int lds_off, const char *base, int64_t ld_bytes,
                                                     int krows_left, int mn_left, int64_t total) {
  constexpr int PER_WAVE = BK * 512 / 1024 / (NT / 64);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, total);
  const int w = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int inst = w * PER_WAVE + j;
    const int kr = inst * 2 + (lane >> 5);
    const int c = (lane & 31) ^ (4 * ((kr >> 2) & 3));
    const bool ok = kr < krows_left && c * 4 < mn_left;
    const uint32_t voff = ok ? (uint32_t)(kr * ld_bytes + c * 16) : kOOB;
    dma16(rs, lds_off + inst * 1024, voff);
  }
}

// ============================================================== HGEMM
// 256 x 256 x 64 tiles, 8 waves as 2 (m) x 4 (n), wave tile 128 x 64,
// v_mfma_f32_16x16x32_{f16,bf16}: 8 x 4 blocks per wave.
struct HCfg {
  static constexpr int BM = 256, BN = 256, BK = 64, NT = 512;
  static constexpr int WTM = 128, WTN = 64, MB = 8, NB = 4, NACC = MB * NB;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
};

template <int DT>
__device__ __forceinline__ void h_load(const KernelArgs &a, int stage, int m0, int n0, int kit) {
  constexpr int ES = 2;
  const int k0 = kit * HCfg::BK;
  const int64_t lda_b = a.lda * ES, ldb_b = a.ldb * ES;
  const char *Ab = static_cast<const char *>(a.A) + (int64_t)m0 * lda_b + (int64_t)k0 * ES;
  const char *Bb = static_cast<const char *>(a.B) + (int64_t)n0 * ldb_b + (int64_t)k0 * ES;
  const int64_t a_total = (int64_t)(a.m - 1 - m0) * lda_b + (int64_t)(a.a_kext - k0) * ES;
  const int64_t b_total = (int64_t)(a.n - 1 - n0) * ldb_b + (int64_t)(a.b_kext - k0) * ES;
  const int kb = (a.k - k0) * ES;
  load_kmajor_128<HCfg::BM, HCfg::NT>(stage * HCfg::STAGE, Ab, lda_b, a.m - m0, kb, a_total);
  load_kmajor_128<HCfg::BN, HCfg::NT>(stage * HCfg::STAGE + HCfg::A_BYTES, Bb, ldb_b, a.n - n0, kb,
                                      b_total);
}

template <int DT>
__device__ __forceinline__ void h_compute(int stage, int wm, int wn, f4_t (&acc)[HCfg::NACC]) {
  using E = Elem<DT>;
  using V8 = typename E::V8;
  const int lane = threadIdx.x & 63;
  const int As = stage * HCfg::STAGE, Bs = As + HCfg::A_BYTES;
#pragma unroll
  for (int ks = 0; ks < HCfg::BK / 32; ++ks) {
    V8 bf[HCfg::NB], af[HCfg::MB];
    const int c = ks * 4 + (lane >> 4);
#pragma unroll
    for (int nb = 0; nb < HCfg::NB; ++nb) {
      const int row = wn * HCfg::WTN + nb * 16 + (lane & 15);
      bf[nb] = *reinterpret_cast<const V8 *>(smem + Bs + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int mb = 0; mb < HCfg::MB; ++mb) {
      const int row = wm * HCfg::WTM + mb * 16 + (lane & 15);
      af[mb] = *reinterpret_cast<const V8 *>(smem + As + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int mb = 0; mb < HCfg::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < HCfg::NB; ++nb)
        acc[mb * HCfg::NB + nb] = E::mfma(bf[nb], af[mb], acc[mb * HCfg::NB + nb]);
  }
}

// MacLoop over iterations [lb, le) of the tile at (m0, n0).
template <int DT>
__device__ __forceinline__ void h_macloop(const KernelArgs &a, int m0, int n0, int lb, int le,
                                          f4_t (&acc)[HCfg::NACC]) {
  const int w = wave_id();
  const int wm = w / 4, wn = w % 4;
#pragma unroll
  for (int i = 0; i < HCfg::NACC; ++i) acc[i] = f4_t{0.f, 0.f, 0.f, 0.f};
  if (lb >= le) return;
  h_load<DT>(a, 0, m0, n0, lb);
  for (int it = lb; it < le; ++it) {
    const int cur = (it - lb) & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of stage `cur` have landed
    __syncthreads();
    if (it + 1 < le) h_load<DT>(a, cur ^ 1, m0, n0, it + 1);
    h_compute<DT>(cur, wm, wn, acc);
  }
  __syncthreads();  // the next segment's loads reuse the stages
}

// ============================================================== SGEMM
// 128 x 128 x 32 tiles, 4 waves as 2 x 2, wave tile 64 x 64,
// v_mfma_f32_16x16x4_f32: 4 x 4 blocks per wave.  Within a group of 16 k,
// MFMA step q of lane group h = lane >> 4 multiplies k = 16 g + 4 h + q for
// both operands; a k-major operand reads its 4 values with one 128-bit LDS
// read, an mn-major operand reads one 32-bit value per step.
struct SCfg {
  static constexpr int BM = 128, BN = 128, BK = 32, NT = 256;
  static constexpr int WTM = 64, WTN = 64, MB = 4, NB = 4, NACC = MB * NB;
  static constexpr int A_BYTES = BM * BK * 4, B_BYTES = BN * BK * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES;
};

template <bool KMAJOR>
__device__ __forceinline__ void s_load_operand(int lds_off, const void *ptr, int64_t ld, int mn0,
                                               int mn_total, int k0, int k_total, int k_ext) {
  constexpr int ES = 4;
  const int64_t ldb = ld * ES;
  const char *p = static_cast<const char *>(ptr);
  if (KMAJOR) {
    const char *base = p + (int64_t)mn0 * ldb + (int64_t)k0 * ES;
    const int64_t total = (int64_t)(mn_total - 1 - mn0) * ldb + (int64_t)(k_ext - k0) * ES;
    load_kmajor_128<SCfg::BM, SCfg::NT>(lds_off, base, ldb, mn_total - mn0, (k_total - k0) * ES, total);
  } else {
    const char *base = p + (int64_t)k0 * ldb + (int64_t)mn0 * ES;
    const int64_t total = (int64_t)(k_total - 1 - k0) * ldb + (int64_t)(mn_total - mn0) * ES;
    load_mnmajor_f32x128<SCfg::BK, SCfg::NT>(lds_off, base, ldb, k_total - k0, mn_total - mn0, total);
  }
}

template <bool AK, bool BKM>
__device__ __forceinline__ void s_load(const KernelArgs &a, int stage, int m0, int n0, int kit) {
  const int k0 = kit * SCfg::BK;
  s_load_operand<AK>(stage * SCfg::STAGE, a.A, a.lda, m0, a.m, k0, a.k, a.a_kext);
  s_load_operand<BKM>(stage * SCfg::STAGE + SCfg::A_BYTES, a.B, a.ldb, n0, a.n, k0, a.k, a.b_kext);
}

// Value of operand element (mn_local, k_local) for MFMA step q, lane group h.
template <bool KMAJOR>
__device__ __forceinline__ f4_t s_frag4(int base_off, int row, int g) {
  // k-major: row `row`, chunk 4g + h (the caller's lane group is folded into
  // `row`'s lane part and into the chunk below)
  const int lane = threadIdx.x & 63;
  const int c = 4 * g + (lane >> 4);
  return *reinterpret_cast<const f4_t *>(smem + base_off + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
}

__device__ __forceinline__ float s_mn_elem(int base_off, int mn, int k) {
  const int c = mn >> 2, e = mn & 3;
  const int p = c ^ (4 * ((k >> 2) & 3));
  return *reinterpret_cast<const float *>(smem + base_off + k * 512 + p * 16 + e * 4);
}

template <bool AK, bool BKM>
__device__ __forceinline__ void s_compute(int stage, int wm, int wn, f4_t (&acc)[SCfg::NACC]) {
  const int lane = threadIdx.x & 63;
  const int As = stage * SCfg::STAGE, Bs = As + SCfg::A_BYTES;
  const int h = lane >> 4, li = lane & 15;
#pragma unroll
  for (int g = 0; g < SCfg::BK / 16; ++g) {
    f4_t av[SCfg::MB], bv[SCfg::NB];
#pragma unroll
    for (int mb = 0; mb < SCfg::MB; ++mb) {
      const int mn = wm * SCfg::WTM + mb * 16 + li;
      if (AK) {
        av[mb] = s_frag4<true>(As, mn, g);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) av[mb][q] = s_mn_elem(As, mn, 16 * g + 4 * h + q);
      }
    }
#pragma unroll
    for (int nb = 0; nb < SCfg::NB; ++nb) {
      const int mn = wn * SCfg::WTN + nb * 16 + li;
      if (BKM) {
        bv[nb] = s_frag4<true>(Bs, mn, g);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) bv[nb][q] = s_mn_elem(Bs, mn, 16 * g + 4 * h + q);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int mb = 0; mb < SCfg::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < SCfg::NB; ++nb)
          acc[mb * SCfg::NB + nb] =
              __builtin_amdgcn_mfma_f32_16x16x4f32(bv[nb][q], av[mb][q], acc[mb * SCfg::NB + nb], 0, 0, 0);
  }
}

template <bool AK, bool BKM>
__device__ __forceinline__ void s_macloop(const KernelArgs &a, int m0, int n0, int lb, int le,
                                          f4_t (&acc)[SCfg::NACC]) {
  const int w = wave_id();
  const int wm = w / 2, wn = w % 2;
#pragma unroll
  for (int i = 0; i < SCfg::NACC; ++i) acc[i] = f4_t{0.f, 0.f, 0.f, 0.f};
  if (lb >= le) return;
  s_load<AK, BKM>(a, 0, m0, n0, lb);
  for (int it = lb; it < le; ++it) {
    const int cur = (it - lb) & 1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < le) s_load<AK, BKM>(a, cur ^ 1, m0, n0, it + 1);
    s_compute<AK, BKM>(cur, wm, wn, acc);
  }
  __syncthreads();
}

// ======================================================= work iteration

// Runs one segment: MacLoop, then partial store or fixup + epilogue.
template <class Cfg, class MacLoop, int DT>
__device__ __forceinline__ void run_segment(const KernelArgs &a, bool vec_ok, int x, int tile, int lb,
                                            int le, bool started, int last_peer, MacLoop macloop) {
  f4_t acc[Cfg::NACC];
  const int tm = tile / a.tiles_n, tn = tile % a.tiles_n;
  const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
  macloop(m0, n0, lb, le, acc);
  if (!started) {
    store_partial<Cfg::NT, Cfg::NACC>(a, x, acc);
    return;
  }
  for (int p = x + 1; p <= last_peer; ++p) {
    if (wait_flag(a, p)) add_partial<Cfg::NT, Cfg::NACC>(a, p, acc);
  }
  const int w = wave_id();
  constexpr int WN = Cfg::BN / Cfg::WTN;
  epilogue<DT, Cfg::MB, Cfg::NB>(a, vec_ok, m0 + (w / WN) * Cfg::WTM, n0 + (w % WN) * Cfg::WTN, acc);
}

template <class Cfg, int DT, class MacLoop>
__device__ __forceinline__ void run_workgroup(const KernelArgs &a, bool vec_ok, MacLoop macloop) {
  const int x = blockIdx.x;
  if (a.sk_tiles > 0) {
    int64_t it = (int64_t)x * a.sk_q + (x < a.sk_r ? x : a.sk_r);
    const int64_t end = (int64_t)(x + 1) * a.sk_q + (x + 1 < a.sk_r ? x + 1 : a.sk_r);
    while (it < end) {
      const int tile = (int)(it / a.ipt);
      const int64_t ts = (int64_t)tile * a.ipt, te = ts + a.ipt;
      const int lb = (int)(it - ts), le = (int)((end < te ? end : te) - ts);
      const bool started = lb == 0, ended = end >= te;
      int last_peer = -1;
      if (started && !ended) {
        const int64_t big = a.sk_r * (a.sk_q + 1), l = te - 1;
        last_peer = (int)(l < big ? l / (a.sk_q + 1) : a.sk_r + (l - big) / a.sk_q);
      }
      run_segment<Cfg, MacLoop, DT>(a, vec_ok, x, tile, lb, le, started, last_peer, macloop);
      it = te;
    }
  }
  for (int tile = a.sk_tiles + x; tile < a.tiles; tile += a.grid)
    run_segment<Cfg, MacLoop, DT>(a, vec_ok, x, tile, 0, a.ipt, true, -1, macloop);
}

template <int DT>
__global__ __launch_bounds__(HCfg::NT) void hgemm_kernel(KernelArgs a, int vec_ok) {
  run_workgroup<HCfg, DT>(a, vec_ok != 0, [&](int m0, int n0, int lb, int le, f4_t(&acc)[HCfg::NACC]) {
    h_macloop<DT>(a, m0, n0, lb, le, acc);
  });
}

template <bool AK, bool BKM>
__global__ __launch_bounds__(SCfg::NT) void sgemm_kernel(KernelArgs a, int vec_ok) {
  run_workgroup<SCfg, SK_F32>(a, vec_ok != 0, [&](int m0, int n0, int lb, int le, f4_t(&acc)[SCfg::NACC]) {
    s_macloop<AK, BKM>(a, m0, n0, lb, le, acc);
  });
}

// ========================================================= small kernels

template <int DT>
__global__ void scale_kernel(int64_t m, int64_t n, float beta, void *C, int64_t ldc) {
  using E = Elem<DT>;
  const int64_t total = m * n;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / n, j = e % n;
    const float v = beta == 0.f ? 0.f : beta * E::ld(C, i * ldc + j);
    E::st(C, i * ldc + j, v);
  }
}

// Repack: dst[r * ldd + l] = src(r, l) for l < k, 0 for k <= l < ldd.  A
// 64 x 64 tile goes through LDS so that both the read (along the source's
// contiguous index) and the write (along l) are coalesced.
template <typename U>
__global__ __launch_bounds__(256) void pack_kernel(const U *src, int64_t lds, int src_kmajor,
                                                   int64_t rows, int64_t k, U *dst, int64_t ldd) {
  __shared__ U tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, l0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
  for (int yy = ty; yy < 64; yy += 4) {
    if (src_kmajor) {  // row r = r0 + yy, l = l0 + tx
      const int64_t r = r0 + yy, l = l0 + tx;
      tile[yy][tx] = (r < rows && l < k) ? src[r * lds + l] : U(0);
    } else {  // src(r, l) at l * lds + r: read along r
      const int64_t l = l0 + yy, r = r0 + tx;
      tile[tx][yy] = (r < rows && l < k) ? src[l * lds + r] : U(0);
    }
  }
  __syncthreads();
  for (int yy = ty; yy < 64; yy += 4) {
    const int64_t r = r0 + yy, l = l0 + tx;
    if (r < rows && l < ldd) dst[r * ldd + l] = tile[yy][tx];
  }
}

__global__ void zero_words_kernel(int32_t *p, int64_t words) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace dev

// ============================================================ launchers

static bool c_vec_ok(const KernelArgs &a, int dtype) {
  const int es = dtype == SK_F32 ? 4 : 2;
  const uintptr_t align = (uintptr_t)(4 * es);
  return (reinterpret_cast<uintptr_t>(a.C) % align == 0) && (a.ldc % 4 == 0);
}

int launch_gemm(const Plan &p, const KernelArgs &a, hipStream_t stream) {
  dim3 grid(p.grid), block(p.cfg.threads);
  const int vec_ok = c_vec_ok(a, p.dtype) ? 1 : 0;
  const size_t lds = p.cfg.lds_bytes;
  if (p.dtype == SK_F16) {
    hipLaunchKernelGGL(dev::hgemm_kernel<SK_F16>, grid, block, lds, stream, a, vec_ok);
  } else if (p.dtype == SK_BF16) {
    hipLaunchKernelGGL(dev::hgemm_kernel<SK_BF16>, grid, block, lds, stream, a, vec_ok);
  } else {
    if (a.a_kmajor && a.b_kmajor)
      hipLaunchKernelGGL((dev::sgemm_kernel<true, true>), grid, block, lds, stream, a, vec_ok);
    else if (a.a_kmajor)
      hipLaunchKernelGGL((dev::sgemm_kernel<true, false>), grid, block, lds, stream, a, vec_ok);
    else if (a.b_kmajor)
      hipLaunchKernelGGL((dev::sgemm_kernel<false, true>), grid, block, lds, stream, a, vec_ok);
    else
      hipLaunchKernelGGL((dev::sgemm_kernel<false, false>), grid, block, lds, stream, a, vec_ok);
  }
  return (int)hipGetLastError();
}

int launch_scale(int dtype, int64_t m, int64_t n, float beta, void *C, int64_t ldc,
                 hipStream_t stream) {
  const int64_t total = m * n;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (dtype == SK_F32)
    hipLaunchKernelGGL(dev::scale_kernel<SK_F32>, dim3(blocks), dim3(256), 0, stream, m, n, beta, C, ldc);
  else if (dtype == SK_F16)
    hipLaunchKernelGGL(dev::scale_kernel<SK_F16>, dim3(blocks), dim3(256), 0, stream, m, n, beta, C, ldc);
  else
    hipLaunchKernelGGL(dev::scale_kernel<SK_BF16>, dim3(blocks), dim3(256), 0, stream, m, n, beta, C, ldc);
  return (int)hipGetLastError();
}

int launch_pack(int dtype, const void *src, int64_t lds, bool src_kmajor, int64_t rows, int64_t k,
                void *dst, int64_t ldd, hipStream_t stream) {
  dim3 grid((unsigned)((ldd + 63) / 64), (unsigned)((rows + 63) / 64)), block(256);
  if (dtype == SK_F32)
    hipLaunchKernelGGL(dev::pack_kernel<uint32_t>, grid, block, 0, stream,
                       static_cast<const uint32_t *>(src), lds, src_kmajor ? 1 : 0, rows, k,
                       static_cast<uint32_t *>(dst), ldd);
  else
    hipLaunchKernelGGL(dev::pack_kernel<uint16_t>, grid, block, 0, stream,
                       static_cast<const uint16_t *>(src), lds, src_kmajor ? 1 : 0, rows, k,
                       static_cast<uint16_t *>(dst), ldd);
  return (int)hipGetLastError();
}

int launch_zero_report(sk_abft_report *report, hipStream_t stream) {
  const int64_t words = (int64_t)(sizeof(sk_abft_report) / 4);
  hipLaunchKernelGGL(dev::zero_words_kernel, dim3(1), dim3(256), 0, stream,
                     reinterpret_cast<int32_t *>(report), words);
  return (int)hipGetLastError();
}

int kernel_occupancy(int dtype, int *blocks_per_cu) {
  const TileCfg c = tile_cfg(dtype);
  hipError_t e;
  int nb = 0;
  if (dtype == SK_F32) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&dev::sgemm_kernel<true, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, c.lds_bytes);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, dev::sgemm_kernel<true, false>, c.threads,
                                                       c.lds_bytes);
    for (auto f : {reinterpret_cast<const void *>(&dev::sgemm_kernel<true, true>),
                   reinterpret_cast<const void *>(&dev::sgemm_kernel<false, true>),
                   reinterpret_cast<const void *>(&dev::sgemm_kernel<false, false>)})
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, c.lds_bytes);
  } else {
    const void *f16 = reinterpret_cast<const void *>(&dev::hgemm_kernel<SK_F16>);
    const void *bf16 = reinterpret_cast<const void *>(&dev::hgemm_kernel<SK_BF16>);
    e = hipFuncSetAttribute(f16, hipFuncAttributeMaxDynamicSharedMemorySize, c.lds_bytes);
    if (e == hipSuccess) e = hipFuncSetAttribute(bf16, hipFuncAttributeMaxDynamicSharedMemorySize, c.lds_bytes);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &nb, dtype == SK_F16 ? dev::hgemm_kernel<SK_F16> : dev::hgemm_kernel<SK_BF16>, c.threads,
          c.lds_bytes);
  }
  *blocks_per_cu = nb;
  return (int)e;
}

}  // namespace sk
