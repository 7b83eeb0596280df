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
typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef __bf16 b4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void *lds_vptr;
typedef short v4s_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kOOB = 0x80000000u;  // offset past every buffer range (ranges are < 2^31)
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

extern __shared__ __attribute__((aligned(1024))) char smem[];

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char *base, int64_t bytes) {
  int32_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, n, kRsrcWord3);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (LDS/scalar and export counters unchecked).
constexpr int vmcnt_le(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Transposing 64-bit LDS read of 16-bit values (ds_read_b64_tr_b16): within
// each group of 16 lanes, lane i receives value i % 4 of the 8 bytes at the
// addresses of lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 (in that
// order) of its group.
//
// The read goes through a restrict-qualified parameter so that, once
// inlined, it carries alias-scope information.  Without it the compiler's
// wait insertion puts a wait for every outstanding vector-memory load in
// front of each such read (it cannot tell the read from one of LDS bytes a
// direct-to-LDS load may still be writing), which empties the load
// pipeline inside the MAC loop; ordinary LDS loads are not held that way.
// The loop orders its LDS reads after the direct-to-LDS loads of a stage
// with its own waits and barriers, as it does for the ordinary loads.
typedef __attribute__((address_space(3))) v4s_t *lds_v4s_t;
__device__ __attribute__((always_inline)) inline v4s_t ds_read_tr16_at(lds_v4s_t __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}
// (at LDS byte address `addr`)
__device__ __forceinline__ v4s_t ds_read_tr16_abs(int addr) {
  return ds_read_tr16_at((lds_v4s_t)(uintptr_t)(uint32_t)addr);
}
__device__ __forceinline__ int lds_addr(const char *p) {
  return (int)(uint32_t)(uintptr_t)(lds_vptr)p;
}

// ---------------------------------------------------------------- elements

template <int DT> struct Elem;
template <> struct Elem<SK_F16> {
  using T = _Float16;
  using V8 = h8_t;
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
// Ordering without whole-cache maintenance.  The L2 of each XCD is not
// coherent with the others, and an agent-scope release or acquire in the
// language memory model writes back or invalidates the entire L2 of the XCD
// (disturbing every workgroup that shares it, and costing tens of
// microseconds per fixup on a busy chip).  In the LLVM AMDGPU memory model
// for GFX942 (followed by gfx950), relaxed agent-scope atomics are plain
// accesses with the sc1 bit, coherent across the XCDs' L2 caches, and the
// release/acquire maintenance (write-back before, invalidation after) exists
// only for data accessed without sc1.  Here the partial tile is written and
// read with agent-coherent (sc1) 128-bit buffer accesses, which the L2
// passes through to the memory side, so only the order of the accesses
// matters:
//   producer: sc1 stores; wait for this wave's stores to complete; workgroup
//     barrier; thread 0 stores the flag (relaxed, agent scope, also sc1);
//   owner: thread 0 reads the flag (relaxed, agent scope) until it holds the
//     epoch; workgroup barrier; sc1 loads of the partial.
constexpr int kAuxSc1 = 16;  // cache-policy operand: sc1 (agent coherence)

template <class P>
__device__ __forceinline__ void store_partial(const KernelArgs &a, int x, const typename P::Acc &acc) {
  constexpr int BYTES = P::NACC4 * P::NT * 16;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(reinterpret_cast<const char *>(a.partials) + (int64_t)x * BYTES, BYTES);
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < P::NACC4; ++i) {
    const f4_t v = P::get4(acc, i);
    // lane offset in a register, slice offset as a scalar constant
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, v), r, t * 16, i * P::NT * 16, kAuxSc1);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
  __syncthreads();
  if (t == 0 && !a.no_signal) __hip_atomic_store(a.flags + x, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        // the error word may be host memory: a plain system-scope store
        __hip_atomic_store(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        ok = 0;
        break;
      }
    }
    ok_s = ok;
  }
  __syncthreads();
  return ok_s != 0;
}

// The owner's loads go through LDS: every wave fetches its own lanes' 16-byte
// entries of up to LDS_BYTES of the partial with direct-to-LDS loads (no
// registers held while they are in flight, so they all overlap), waits for
// its own loads only (no other wave reads them) and adds them from LDS.  The
// caller has passed a workgroup barrier since the last MAC-loop LDS read; a
// barrier at the end keeps the next segment's tile loads from overwriting
// entries another wave has not read yet.
template <class P>
__device__ __forceinline__ void add_partial(const KernelArgs &a, int peer, typename P::Acc &acc) {
  constexpr int SLICE = P::NT * 16;                       // bytes of one accumulator slice
  constexpr int BYTES = P::NACC4 * SLICE;
  constexpr int CHUNK = P::LDS_BYTES / SLICE < P::NACC4 ? P::LDS_BYTES / SLICE : P::NACC4;
  static_assert(CHUNK > 0 && P::NACC4 % CHUNK == 0, "partial staging");
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(reinterpret_cast<const char *>(a.partials) + (int64_t)peer * BYTES, BYTES);
  const int t = threadIdx.x, wbase = wave_id() * 1024;
#pragma unroll
  for (int c0 = 0; c0 < P::NACC4; c0 += CHUNK) {
#pragma unroll
    for (int i = 0; i < CHUNK; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(smem + i * SLICE + wbase), 16, t * 16,
                                               (c0 + i) * SLICE, 0, kAuxSc1);
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
#pragma unroll
    for (int i = 0; i < CHUNK; ++i)
      P::add4(acc, c0 + i, *reinterpret_cast<const f4_t *>(smem + i * SLICE + t * 16));
    if (c0 + CHUNK < P::NACC4) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this chunk read
  }
  __syncthreads();
}

// ------------------------------------------------------------ epilogue
//
// Stores alpha * v + beta * C for the four consecutive columns j..j+3 of row
// i (columns at or beyond n are skipped; C is not read when beta == 0).
template <int DT>
__device__ __forceinline__ void store4(const KernelArgs &a, bool vec_ok, int i, int j, f4_t v) {
  using E = Elem<DT>;
  if (i >= a.m || j >= a.n) return;
  const int64_t off = (int64_t)i * a.ldc + j;
  v *= a.alpha;
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


typedef float f16v_t __attribute__((ext_vector_type(16)));

// ============================================================== HGEMM
// 256 x 256 x BK tiles (BK = 64 by default), 8 waves (two per SIMD) as
// 2 (m) x 4 (n), wave tile 128 x 64 = 4 x 2 blocks of
// v_mfma_f32_32x32x16_{f16,bf16} (16 fp32 per lane per block, 128 per lane).
// A k-iteration is BK/16 k-substeps; the fragments of one substep are 6 LDS
// reads (24 VGPRs).  NSTAGE LDS stages (two of 64 KiB by default): loads are
// issued NSTAGE-1 iterations ahead of their use.
// 32x32 block layout, with the product formed as C^T = B^T A^T: register r
// of lane l holds row (l & 31) and column 8*(r/4) + 4*(l >> 5) + (r & 3) of
// the block, i.e. four consecutive columns per register quad.
// HGEMM instances: 256 x 256 tiles with 8 waves (2 x 4, 128 x 64 each;
// one workgroup per CU) and 128 x 128 tiles with 4 waves (2 x 2, 64 x 64
// each; two workgroups per CU) for shapes with few large tiles.  W = 4 with
// 256 x 256 tiles (128 x 128 per wave, one wave per SIMD, a third fewer LDS
// fragment reads per MFMA) also builds and gives the same bits, but one wave
// per SIMD cannot hide its own LDS and barrier waits: about 6 % slower on
// large squares, so it is not instantiated.
template <int DT, int TILE, int W = (TILE == 256 ? 8 : 4), bool BMN_ = false, bool AMN_ = false>
struct HPolicy {
  static constexpr int ET = DT;
  // BMN / AMN: B stored n-contiguous (row-major k x n) / A stored
  // m-contiguous (column-major m x k), staged in LDS as BK rows of BN / BM
  // values and read into the MFMA layout with transposing LDS reads
  static constexpr bool BMN = BMN_, AMN = AMN_;
  static constexpr int BM = TILE, BN = TILE, BK = 64, NSTAGE = 2;
  static constexpr int WAVES = W, NT = 64 * WAVES;
  // waves per SIMD the register budget is sized for
  static constexpr int WPE = TILE == 256 && W == 4 ? 1 : 2;
  static constexpr int SUBS = BK / 16;  // k-substeps of one iteration
  static_assert(TILE == 256 || TILE == 128, "tile");
  static constexpr int WTM = BM / 2, WTN = BN / (WAVES / 2), MB = WTM / 32, NB = WTN / 32;
  static constexpr int WAVES_N = BN / WTN;
  static constexpr int NACC4 = MB * NB * 4;
  static constexpr int ROW = BK * 2;  // bytes of one LDS row (k-contiguous)
  static constexpr int A_BYTES = BM * ROW, B_BYTES = BN * ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  // LDS holds the A tiles of all stages, then the B tiles of all stages, so
  // that every fragment read lies within 64 KiB (the reach of an LDS
  // instruction's offset field) of one A base and one B base
  static __device__ __forceinline__ constexpr int a_off(int stage) { return stage * A_BYTES; }
  static __device__ __forceinline__ constexpr int b_off(int stage) { return NSTAGE * A_BYTES + stage * B_BYTES; }
  static constexpr int LOADS = A_BYTES / 1024 / (NT / 64);  // per operand per wave and stage
  static constexpr int ROWS_PER_LOAD = 1024 / ROW;
  // 16-byte chunk c of LDS row r is stored at chunk position c ^ swz(r):
  // the 16 lanes of one LDS cycle (rows r..r+15, one chunk) then touch 16
  // distinct 16-byte bank groups of gfx950's 64 banks (256 bytes hold
  // 256/ROW rows; consecutive groups of them get distinct XOR masks).
  static __device__ __forceinline__ int swz(int r) { return (r / (256 / ROW)) % (ROW / 16); }
  // mn-contiguous stages (BMN, AMN): k-row r holds TILE values (TILE / 8
  // chunks of 16 bytes); chunk c sits at position c ^ (4 (r & 3)).  A
  // transposing read fetches a 4 (k) x 16 (m or n) block per 16 lanes, 8
  // bytes per lane; with this XOR the 8 blocks of 32 lanes (two column
  // halves x four rows) fall in distinct 32-byte bank windows, since a row
  // is a multiple of 256 bytes.  BM == BN, so A and B stages of this form
  // share the layout and the lanes' load positions.
  static constexpr int MNROW = BN * 2;                // bytes of one k-row of an mn-contiguous stage
  static constexpr int MNCPR = BN / 8;                // chunks per k-row
  static constexpr int MNRPL = 1024 / MNROW;          // k-rows per 1 KiB load
  static __device__ __forceinline__ int mnpos(int r, int c) { return c ^ (4 * (r & 3)); }
  static_assert(!(BMN || AMN) || (BM == BN && MNROW % 256 == 0 && MNCPR >= 16), "mn-contiguous stage layout");
  struct Acc { f16v_t v[MB * NB]; };
  static __device__ __forceinline__ f4_t get4(const Acc &c, int i) {
    const f16v_t &b = c.v[i >> 2];
    const int g = i & 3;
    return f4_t{b[4 * g], b[4 * g + 1], b[4 * g + 2], b[4 * g + 3]};
  }
  static __device__ __forceinline__ void add4(Acc &c, int i, f4_t x) {
    f16v_t &b = c.v[i >> 2];
    const int g = i & 3;
    b[4 * g] += x[0]; b[4 * g + 1] += x[1]; b[4 * g + 2] += x[2]; b[4 * g + 3] += x[3];
  }
  static __device__ __forceinline__ void zero(Acc &c) {
#pragma unroll
    for (int i = 0; i < MB * NB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) c.v[i][e] = 0.f;
  }
};

// Direct-to-LDS loads of one tile's A and B k-slices.  The per-lane byte
// offsets (row * ld + swizzled chunk, or an out-of-range offset for rows
// past the matrix) are computed once per tile; each k-iteration only adds
// the scalar offset k0 * 2.  In the iteration that holds the end of k,
// chunks at or past k are fetched out of range (zeros).
template <class P>
struct HLoader {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t va[P::LOADS], vb[P::LOADS];
  // 16-byte k-chunk load j fetches (same for A and B): rows of load j are
  // 8 j further on, which with 128-byte rows changes the swizzle only with
  // the parity of j, so two values hold every load's chunk
  int chunk2[2];
  __device__ __forceinline__ int chunk(int j) const { return chunk2[j & 1]; }
  int lds_a;            // LDS byte offset of this wave's first A load (stage 0)
  // mn-contiguous operands: k-row of this lane's first load within a stage
  // (load j: + j MNRPL), and the bytes A and B advance per k-iteration
  int krow0;
  int astep, bstep;
  // does load j of this lane fetch k-row krow0 + j MNRPL of the iteration
  // (a row before k)?
  __device__ __forceinline__ bool krow_ok(int j, int left) const { return (krow0 + j * P::MNRPL) * 2 < left; }

  __device__ __forceinline__ void init(const KernelArgs &a, int m0, int n0) {
    static_assert(P::ROW == 128 && P::LOADS % 2 == 0, "chunk of load j depends only on j & 1");
    constexpr int ES = 2;
    const int w = wave_id(), lane = threadIdx.x & 63;
    const int64_t lda_b = a.lda * ES, ldb_b = a.ldb * ES;
    // mn-contiguous operands: element (k, n) of B at B + (k ldb + n) 2
    // (element (i, k) of A at A + (k lda + i) 2); the descriptor starts at
    // column n0 (row m0) and ends at the last element, the iteration's
    // k-rows go in soffset
    const char *Ab = static_cast<const char *>(a.A) + (int64_t)m0 * (P::AMN ? ES : lda_b);
    const char *Bb = static_cast<const char *>(a.B) + (int64_t)n0 * (P::BMN ? ES : ldb_b);
    if constexpr (P::AMN)
      ra = make_rsrc(Ab, ((int64_t)(a.k - 1) * a.lda + (a.m - m0)) * ES);
    else
      ra = make_rsrc(Ab, (int64_t)(a.m - 1 - m0) * lda_b + (int64_t)a.a_kext * ES);
    if constexpr (P::BMN)
      rb = make_rsrc(Bb, ((int64_t)(a.k - 1) * a.ldb + (a.n - n0)) * ES);
    else
      rb = make_rsrc(Bb, (int64_t)(a.n - 1 - n0) * ldb_b + (int64_t)a.b_kext * ES);
    if constexpr (P::AMN || P::BMN) {
      astep = (int)(P::BK * lda_b);
      bstep = (int)(P::BK * ldb_b);
      // lane L of load j fills position L % MNCPR of k-row krow0 + j MNRPL;
      // the chunk stored there is the inverse of the XOR
      krow0 = w * P::LOADS * P::MNRPL + lane / P::MNCPR;
#pragma unroll
      for (int j = 0; j < P::LOADS; ++j) {
        const int kr = krow0 + j * P::MNRPL;
        const int c = P::mnpos(kr, lane % P::MNCPR);
        if constexpr (P::AMN) va[j] = m0 + c * 8 < a.m ? (uint32_t)((int64_t)kr * lda_b + c * 16) : kOOB;
        if constexpr (P::BMN) vb[j] = n0 + c * 8 < a.n ? (uint32_t)((int64_t)kr * ldb_b + c * 16) : kOOB;
      }
    }
    constexpr int CPR = P::ROW / 16;  // chunks per row
#pragma unroll
    for (int j = 0; j < P::LOADS; ++j) {
      const int row = (w * P::LOADS + j) * P::ROWS_PER_LOAD + lane / CPR;
      const int c = (lane % CPR) ^ P::swz(row);
      if (j < 2) chunk2[j] = c;
      if constexpr (!P::AMN) va[j] = row < a.m - m0 ? (uint32_t)(row * lda_b + c * 16) : kOOB;
      if constexpr (!P::BMN) vb[j] = row < a.n - n0 ? (uint32_t)(row * ldb_b + c * 16) : kOOB;
    }
    lds_a = w * P::LOADS * 1024;
  }

  // Load q of this wave's share of iteration kit (q even: A, q odd: B,
  // block q / 2), without a branch: chunks at or past k, and every chunk
  // when `live` is false, are fetched out of range, i.e. written to LDS as
  // zeros.
  __device__ __forceinline__ void load_one(const KernelArgs &a, int stage, int kit, bool live, int q) const {
    const int j = q >> 1;
    const int k0b = kit * P::BK * 2;
    const int left = live ? (a.k - kit * P::BK) * 2 : 0;
    const int dst = ((q & 1) ? P::b_off(stage) : P::a_off(stage)) + lds_a + j * 1024;
    if (P::BMN && (q & 1)) {  // k-rows at or past k read as zeros
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_vptr)(smem + dst), 16, krow_ok(j, left) ? vb[j] : kOOB,
                                               kit * bstep, 0, 0);
      return;
    }
    if (P::AMN && !(q & 1)) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_vptr)(smem + dst), 16, krow_ok(j, left) ? va[j] : kOOB,
                                               kit * astep, 0, 0);
      return;
    }
    const bool ok = chunk(j) * 16 < left;
    __builtin_amdgcn_raw_ptr_buffer_load_lds((q & 1) ? rb : ra, (lds_vptr)(smem + dst), 16,
                                             ok ? ((q & 1) ? vb[j] : va[j]) : kOOB, k0b, 0, 0);
  }

  __device__ __forceinline__ void load(const KernelArgs &a, int stage, int kit) const {
    const int k0b = kit * P::BK * 2;
    const int left = (a.k - kit * P::BK) * 2;  // bytes of k from k0
    const int abase = P::a_off(stage) + lds_a, bbase = P::b_off(stage) + lds_a;
    const int k0ba = P::AMN ? kit * astep : k0b;  // A's and B's soffsets
    const int k0bb = P::BMN ? kit * bstep : k0b;
    if (left >= P::BK * 2) {
#pragma unroll
      for (int j = 0; j < P::LOADS; ++j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_vptr)(smem + abase + j * 1024), 16, va[j], k0ba, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_vptr)(smem + bbase + j * 1024), 16,
                                                 vb[j], k0bb, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < P::LOADS; ++j) {
        const bool ok = chunk(j) * 16 < left;
        const bool oka = P::AMN ? krow_ok(j, left) : ok;
        const bool okb = P::BMN ? krow_ok(j, left) : ok;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_vptr)(smem + abase + j * 1024), 16,
                                                 oka ? va[j] : kOOB, k0ba, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_vptr)(smem + bbase + j * 1024), 16,
                                                 okb ? vb[j] : kOOB, k0bb, 0, 0);
      }
    }
  }
};

template <int DT>
__device__ __forceinline__ f16v_t h_mfma(typename Elem<DT>::V8 a, typename Elem<DT>::V8 b, f16v_t c);
template <>
__device__ __forceinline__ f16v_t h_mfma<SK_F16>(h8_t a, h8_t b, f16v_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f16v_t h_mfma<SK_BF16>(b8_t a, b8_t b, f16v_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt immediate: at most n vector-memory operations of this wave
// outstanding and no LDS read outstanding.
constexpr int vmcnt_le_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

// MacLoop with fragments read two substeps ahead (three fragment sets in
// rotation) for the two-stage, four-substep configuration.  The stage
// switch moves to the middle of each iteration: after substep 1 every
// fragment of stage i has been read, so after this wave's loads of stage
// i+1 have landed and its LDS reads have returned, one workgroup barrier
// both publishes stage i+1 and frees stage i for the loads of iteration
// i+2.
template <class P>
struct HFrag {
  typename Elem<P::ET>::V8 a[P::MB], b[P::NB];
};

// One fragment read (q < NB: B block q, else A block q - NB) and one MFMA
// (block row q / NB, column q % NB) of a substep, for the pinned
// interleaving below.
template <class P>
__device__ __forceinline__ void h_frag_one(int stage, int sub, int wm, int wn, int q, HFrag<P> &F) {
  using V8 = typename Elem<P::ET>::V8;
  const int lane = threadIdx.x & 63;
  const int As = P::a_off(stage), Bs = P::b_off(stage);
  const int c = sub * 2 + (lane >> 5);
  if ((q < P::NB && P::BMN) || (q >= P::NB && P::AMN)) {
    // lane 16 g + j addresses the four values (k, x .. x + 3) with
    // k = 16 sub + 8 (g / 2) + j / 4 and x = 16 (g % 2) + 4 (j % 4) within
    // the 32-wide block (x: n for B, m for A); the transposing read hands
    // lane 16 g + i the values (k0 .. k0 + 3, x0 + i) of its 16-lane group.
    // A second read 4 rows further completes the eight k of the
    // k-contiguous fragment.
    //
    // Chunk (32 blk + xl) / 8 of k-row k sits at position 4 (blk ^ (k & 3))
    // + xl / 8 (blk: the 32-wide block within the tile, xl < 32), so the
    // address is the lane's part, bits outside 6..8, plus 64 (blk ^ (k & 3))
    // in bits 6..8: one lane base XORed with 64 blk for every block, so
    // that the blocks of a wave share one address register.  The LDS
    // address of the stage (whose bits are all above bit 8) is added first;
    // the XOR is an explicit instruction at each read, which the compiler
    // cannot hoist out of the loop into one register per block.
    const int g = lane >> 4, j = lane & 15;
    const int kl = 8 * (g >> 1) + (j >> 2), xl = 16 * (g & 1) + 4 * (j & 3);
    const int lp = kl * P::MNROW + (xl >> 3) * 16 + (xl & 4) * 2 + 64 * (kl & 3);
    const int blk = q < P::NB ? wn * (P::WTN / 32) + q : wm * (P::WTM / 32) + (q - P::NB);
    static_assert(P::MNROW >= 512 || P::BN / 32 <= 4, "block bits below the k-row bits");
    static_assert(P::A_BYTES % (16 * P::MNROW) == 0 && P::B_BYTES % (16 * P::MNROW) == 0,
                  "stage bases above the lane part");
    const int base = lds_addr(smem) + (q < P::NB ? Bs : As) + lp;
    int xb;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(xb) : "s"(64 * blk), "v"(base));
    const int addr = xb + sub * 16 * P::MNROW;
    const v4s_t lo = ds_read_tr16_abs(addr), hi = ds_read_tr16_abs(addr + 4 * P::MNROW);
    const V8 v = __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    if (q < P::NB)
      F.b[q] = v;
    else
      F.a[q - P::NB] = v;
  } else if (q < P::NB) {
    const int row = wn * P::WTN + q * 32 + (lane & 31);
    F.b[q] = *reinterpret_cast<const V8 *>(smem + Bs + row * P::ROW + ((c ^ P::swz(row)) << 4));
  } else {
    const int row = wm * P::WTM + (q - P::NB) * 32 + (lane & 31);
    F.a[q - P::NB] = *reinterpret_cast<const V8 *>(smem + As + row * P::ROW + ((c ^ P::swz(row)) << 4));
  }
}

template <class P>
__device__ __forceinline__ void h_mfma_one(const HFrag<P> &F, typename P::Acc &acc, int q) {
  const int mb = q / P::NB, nb = q % P::NB;
  acc.v[q] = h_mfma<P::ET>(F.b[nb], F.a[mb], acc.v[q]);
}

// One substep: the MFMAs of fragment set M, interleaved (in this exact
// order: the scheduler may not regroup them) with the fragment reads of
// substep `sub` of stage `stage` into set R and with loads lo .. lo+nl-1 of
// this wave's share of iteration `kit` into stage `lstage`, both spread
// evenly over the MFMAs.  Spreading the reads and loads this way keeps a
// single wave issuing MFMAs back to back: grouped loads stall its issue for
// longer than an MFMA takes.
template <class P>
__device__ __forceinline__ void h_substep(const KernelArgs &a, const HLoader<P> &ld, const HFrag<P> &M,
                                          HFrag<P> &R, int stage, int sub, int wm, int wn,
                                          typename P::Acc &acc, int nl, int lstage, int kit, bool live,
                                          int lo) {
  constexpr int NM = P::MB * P::NB, NR = P::MB + P::NB;
  static_assert(NR <= NM, "one fragment read per MFMA at most");
#pragma unroll
  for (int q = 0; q < NM; ++q) {
    h_mfma_one<P>(M, acc, q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int l = q * nl / NM; l < (q + 1) * nl / NM; ++l) ld.load_one(a, lstage, kit, live, lo + l);
#pragma unroll
    for (int r = (q * NR + NM - 1) / NM; r < ((q + 1) * NR + NM - 1) / NM; ++r)
      h_frag_one<P>(stage, sub, wm, wn, r, R);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Iteration i of the lookahead-2 loop.  Global substep g = 4 i + s uses
// fragment set F[g % 3]; with i = PH (mod 3), 4 i = PH (mod 3).
template <class P, int PH>
__device__ __forceinline__ void h_iter_la2(const KernelArgs &a, const HLoader<P> &ld, int i, int n, int lb,
                                           int wm, int wn, HFrag<P> (&F)[3], typename P::Acc &acc) {
  constexpr int f0 = (PH + 0) % 3, f1 = (PH + 1) % 3, f2 = (PH + 2) % 3;
  const int buf = i & 1;
  h_substep<P>(a, ld, F[f0], F[f2], buf, 2, wm, wn, acc, 0, 0, 0, false, 0);
  h_substep<P>(a, ld, F[f1], F[f0], buf, 3, wm, wn, acc, 0, 0, 0, false, 0);
  // stage switch: stage i+1 complete (its loads were the only ones in
  // flight) and every read of stage i returned
  __builtin_amdgcn_s_waitcnt(vmcnt_le_lgkm0(0));
  __syncthreads();
  // no branches from here to the next stage switch: in the last two
  // iterations the loads fetch nothing (zeros into the stage just freed)
  // and the last iteration's reads of stage i+1 go unused.  The loads of
  // iteration i+2 are split over the two substeps before the next switch.
  h_substep<P>(a, ld, F[f2], F[f1], buf ^ 1, 0, wm, wn, acc, P::LOADS, buf, lb + i + 2, i + 2 < n, 0);
  h_substep<P>(a, ld, F[f0], F[f2], buf ^ 1, 1, wm, wn, acc, P::LOADS, buf, lb + i + 2, i + 2 < n, P::LOADS);
}

template <class P>
__device__ __forceinline__ void h_macloop_la2(const KernelArgs &a, int m0, int n0, int lb, int le,
                                              typename P::Acc &acc) {
  static_assert(P::NSTAGE == 2 && P::SUBS == 4, "lookahead-2 loop: two stages of four substeps");
  constexpr int LPS = 2 * P::LOADS;
  const int w = wave_id();
  const int wm = w / P::WAVES_N, wn = w % P::WAVES_N;
  P::zero(acc);
  const int n = le - lb;
  if (n <= 0) return;
  HLoader<P> ld;
  ld.init(a, m0, n0);
  ld.load(a, 0, lb);
  if (n > 1) {
    ld.load(a, 1, lb + 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_le_lgkm0(LPS));
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_le_lgkm0(0));
  }
  __syncthreads();
  HFrag<P> F[3];
#pragma unroll
  for (int q = 0; q < P::MB + P::NB; ++q) {
    h_frag_one<P>(0, 0, wm, wn, q, F[0]);
    h_frag_one<P>(0, 1, wm, wn, q, F[1]);
  }
  int i = 0;
  for (; i + 3 <= n; i += 3) {
    h_iter_la2<P, 0>(a, ld, i, n, lb, wm, wn, F, acc);
    h_iter_la2<P, 1>(a, ld, i + 1, n, lb, wm, wn, F, acc);
    h_iter_la2<P, 2>(a, ld, i + 2, n, lb, wm, wn, F, acc);
  }
  if (i < n) h_iter_la2<P, 0>(a, ld, i, n, lb, wm, wn, F, acc);
  if (i + 1 < n) h_iter_la2<P, 1>(a, ld, i + 1, n, lb, wm, wn, F, acc);
  // the last iterations' (empty) loads and reads have landed in every wave
  // before the caller reuses LDS
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Epilogue of one tile.  A tile that lies wholly inside C (16-byte aligned,
// ldc a multiple of 8) is written through LDS in whole cache lines, else,
// with rows that allow 4-element vector accesses, by straight-line accesses;
// edge tiles take the per-element bounds checks of store4.  The kernel is
// built twice: BZ for beta == 0 (C never read) and !BZ for beta != 0, so
// that neither carries the other's staging code (the beta != 0 staging
// would otherwise cost the beta == 0 kernel registers and start-up time).
template <class P, bool BZ>
__device__ __forceinline__ void h_epilogue(const KernelArgs &a, bool vec_ok, int m0, int n0,
                                           const typename P::Acc &acc) {
  using T = typename Elem<P::ET>::T;
  const int w = wave_id(), lane = threadIdx.x & 63;
  const int r0 = m0 + (w / P::WAVES_N) * P::WTM, c0 = n0 + (w % P::WAVES_N) * P::WTN;
  const bool full = m0 + P::BM <= a.m && n0 + P::BN <= a.n;
  if (full && a.beta == 0.f && reinterpret_cast<uintptr_t>(a.C) % 16 == 0 && a.ldc % 8 == 0) {
    // Through LDS, half of the wave's block at a time: each lane holds 4
    // consecutive columns of one row, so direct stores would touch 32 rows
    // per instruction; read back as whole rows of the wave's block (2 WTN
    // contiguous bytes, 64 / (WTN / 8) rows per instruction) they cover whole
    // cache lines.  Rows of RS = 2 WTN + 8 bytes (an odd number of 8-byte
    // bank pairs apart) put the 32 rows of one 8-byte LDS write on distinct
    // banks.  Each wave uses only its own region (MB / 2 x 32 rows) and a
    // wave's LDS accesses complete in order, so the passes need no barrier;
    // the caller has passed a workgroup barrier since the last MAC-loop LDS
    // read, and one at the end keeps the next tile's loads (which land in
    // every wave's region) from overwriting rows another wave has not read
    // yet.
    constexpr int RS = P::WTN * 2 + 8, HALF = P::MB / 2;
    constexpr int LPR = P::WTN * 2 / 16, RPI = 64 / LPR;  // lanes per row, rows per read
    // per-lane bases; every other offset is a compile-time constant
    char *const wr = smem + w * (HALF * 32 * RS) + (lane & 31) * RS + 8 * (lane >> 5);
    const char *const rd = smem + w * (HALF * 32 * RS) + (lane / LPR) * RS + (lane % LPR) * 16;
    char *cp = static_cast<char *>(a.C) + ((int64_t)(r0 + lane / LPR) * a.ldc + c0 + (lane % LPR) * 8) * sizeof(T);
    const int64_t step = (int64_t)RPI * a.ldc * sizeof(T);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int mb = 0; mb < HALF; ++mb)
#pragma unroll
        for (int nb = 0; nb < P::NB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            Elem<P::ET>::st4(wr + mb * 32 * RS + (nb * 32 + 8 * g) * 2, 0,
                          a.alpha * P::get4(acc, ((h * HALF + mb) * P::NB + nb) * 4 + g));
#pragma unroll
      for (int it = 0; it < HALF * 32 / RPI; ++it) {
        *reinterpret_cast<u4_t *>(cp) = *reinterpret_cast<const u4_t *>(rd + it * RPI * RS);
        cp += step;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads returned
    __syncthreads();
    return;
  }
  if constexpr (!BZ) {
  if (full && reinterpret_cast<uintptr_t>(a.C) % 16 == 0 && a.ldc % 8 == 0) {
    // beta != 0: alpha * acc goes through LDS in fp32, one 32-row block of
    // the wave at a time, and is read back as whole rows (8 columns per
    // lane) beside 16-byte loads and stores of C that cover whole cache
    // lines (the MFMA layout would touch 32 rows per access); alpha * acc +
    // beta * C is rounded once, as on the other paths.  Rows of RS = 4 WTN +
    // 16 bytes: the 8 lanes of one LDS cycle of a 16-byte write (8 rows)
    // start on distinct 4-bank groups.  Same region and barrier rules as
    // above.
    using V8 = typename Elem<P::ET>::V8;
    constexpr int RS = P::WTN * 4 + 16;
    constexpr int LPR = P::WTN / 8, RPI = 64 / LPR;  // lanes per row, rows per read
    static_assert(P::NT / 64 * 32 * RS <= P::LDS_BYTES && 32 % RPI == 0, "epilogue staging");
    // the lane index made opaque here, so that these addresses are formed
    // here and not hoisted out of the tile loop (where they would hold
    // registers through the MAC loop)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    char *const wr = smem + w * (32 * RS) + (ln & 31) * RS + 16 * (ln >> 5);
    const char *const rd = smem + w * (32 * RS) + (ln / LPR) * RS + (ln % LPR) * 32;
    T *cp = static_cast<T *>(a.C) + (int64_t)(r0 + ln / LPR) * a.ldc + c0 + (ln % LPR) * 8;
    const int64_t step = (int64_t)RPI * a.ldc;
#pragma unroll
    for (int mb = 0; mb < P::MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < P::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f4_t *>(wr + (nb * 32 + 8 * g) * 4) = a.alpha * P::get4(acc, (mb * P::NB + nb) * 4 + g);
      // one row group at a time (a rolled loop: the accumulators of the
      // other blocks leave no registers for several in flight)
#pragma unroll 1
      for (int it = 0; it < 32 / RPI; ++it) {
        const char *rp = rd + it * RPI * RS;
        const f4_t x0 = *reinterpret_cast<const f4_t *>(rp), x1 = *reinterpret_cast<const f4_t *>(rp + 16);
        T *const q = cp;
        cp += step;
        const V8 c = *reinterpret_cast<const V8 *>(q);
        V8 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = (T)(x0[e] + a.beta * (float)c[e]);
          o[e + 4] = (T)(x1[e] + a.beta * (float)c[e + 4]);
        }
        *reinterpret_cast<V8 *>(q) = o;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads returned
    __syncthreads();
    return;
  }
  }
  if (vec_ok && full) {
    // C rows not 16-byte aligned: straight-line 4-element accesses at fixed
    // offsets from one row pointer per 32-row block
    T *cb = static_cast<T *>(a.C) + (int64_t)(r0 + (lane & 31)) * a.ldc + c0 + 4 * (lane >> 5);
    const int64_t rstep = (int64_t)32 * a.ldc;
#pragma unroll
    for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < P::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          T *q = cb + mb * rstep;
          const int o = nb * 32 + 8 * g;
          f4_t v = a.alpha * P::get4(acc, (mb * P::NB + nb) * 4 + g);
          if (a.beta != 0.f) v += a.beta * Elem<P::ET>::ld4(q, o);
          Elem<P::ET>::st4(q, o, v);
        }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < P::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4<P::ET>(a, vec_ok, r0 + mb * 32 + (lane & 31), c0 + nb * 32 + 8 * g + 4 * (lane >> 5),
                   P::get4(acc, (mb * P::NB + nb) * 4 + g));
}

// ========================================================= narrow-m HGEMM
// GEMMs with m of at most 256 and long k (HBM-bound once n and k are large:
// the Stream-K page's evaluation singles out such memory-bound shapes).  One
// tile covers every row of C, so B -- the large operand -- is read once, and
// it streams straight into registers D iterations ahead rather than through
// LDS.  Tiles of BM = 32 MB rows (MB = 2, 4, 6 or 8: the smallest that holds
// m) by 256 columns, 8 waves of 32 columns each, every wave over all BM
// rows: per iteration of 64 k a wave holds its 32 x 64 slice of B in
// registers (four 16-byte loads per lane, issued D iterations ahead) and
// reads the tile's A, staged in LDS for all waves (D + 1 stages), one
// 32-row fragment per MFMA.  Order of k inside an iteration: lane half h at
// k-step s takes the 16-byte chunk 4 h + s (8 values of k) of the 64, in A
// and B alike, so that a lane's four B loads cover 64 contiguous bytes of
// its column.  The MFMA is the HGEMM kernels' 32x32x16 (C^T = B^T A^T, the
// same accumulator layout), one 32 x 32 block per row block.
template <int DT, int MB_>
struct NPolicy {
  static constexpr int ET = DT;
  static constexpr int MB = MB_, NB = 1;
  static constexpr int BM = 32 * MB, BN = 256, BK = 64;
  static constexpr int WAVES = 8, NT = 64 * WAVES, WPE = 1;
  static constexpr int D = 3;           // iterations of B and A in flight
  static constexpr int NSTAGE = D + 1;  // A stages in LDS
  static constexpr int ROW = BK * 2;    // bytes of one A row in a stage
  static constexpr int A_BYTES = BM * ROW;
  static constexpr int LDS_BYTES = NSTAGE * A_BYTES;
  static constexpr int LA = A_BYTES / 1024 / WAVES;  // A loads per wave and iteration
  static constexpr int NACC4 = MB * 4;
  static_assert(LA >= 1 && A_BYTES % (1024 * WAVES) == 0, "A staging");
  // 16-byte chunk c of A row r sits at chunk position c ^ swz(r): the 16
  // lanes of one LDS cycle (16 consecutive rows, one chunk) hit 16 distinct
  // 16-byte bank groups
  static __device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
  struct Acc { f16v_t v[MB]; };
  static __device__ __forceinline__ f4_t get4(const Acc &c, int i) {
    const f16v_t &b = c.v[i >> 2];
    const int g = i & 3;
    return f4_t{b[4 * g], b[4 * g + 1], b[4 * g + 2], b[4 * g + 3]};
  }
  static __device__ __forceinline__ void add4(Acc &c, int i, f4_t x) {
    f16v_t &b = c.v[i >> 2];
    const int g = i & 3;
    b[4 * g] += x[0]; b[4 * g + 1] += x[1]; b[4 * g + 2] += x[2]; b[4 * g + 3] += x[3];
  }
  static __device__ __forceinline__ void zero(Acc &c) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) c.v[i][e] = 0.f;
  }
};

// Per-lane offsets of the narrow-m kernel's loads, computed once per tile.
// A: load j of wave w fills rows (w LA + j) * 8 + lane / 8 of a stage
// (direct-to-LDS, 1 KiB per load).  B: lane l reads column w * 32 + (l & 31)
// at bytes 64 (l >> 5) + 16 s of each 128-byte k-slice.  Rows and columns
// past the matrix, and chunks at or past k, are fetched out of range (zeros).
template <class P>
struct NLoader {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t va[P::LA];
  int ca[P::LA];  // k-chunk of A load j
  uint32_t vb;
  int lds_a;      // this wave's first A load within a stage

  __device__ __forceinline__ void init(const KernelArgs &a, int m0, int n0) {
    constexpr int ES = 2;
    const int w = wave_id(), lane = threadIdx.x & 63;
    const int64_t lda_b = a.lda * ES, ldb_b = a.ldb * ES;
    const char *Ab = static_cast<const char *>(a.A) + (int64_t)m0 * lda_b;
    const char *Bb = static_cast<const char *>(a.B) + (int64_t)n0 * ldb_b;
    ra = make_rsrc(Ab, (int64_t)(a.m - 1 - m0) * lda_b + (int64_t)a.a_kext * ES);
    rb = make_rsrc(Bb, (int64_t)(a.n - 1 - n0) * ldb_b + (int64_t)a.b_kext * ES);
#pragma unroll
    for (int j = 0; j < P::LA; ++j) {
      const int row = (w * P::LA + j) * 8 + lane / 8;
      const int c = (lane % 8) ^ P::swz(row);
      ca[j] = c;
      va[j] = row < a.m - m0 ? (uint32_t)(row * lda_b + c * 16) : kOOB;
    }
    const int col = w * 32 + (lane & 31);
    vb = col < a.n - n0 ? (uint32_t)(col * ldb_b + (lane >> 5) * 64) : kOOB;
    lds_a = w * P::LA * 1024;
  }

  // A of iteration kit into `stage`; every chunk when `live` is false is
  // fetched out of range
  __device__ __forceinline__ void load_a(const KernelArgs &a, int stage, int kit, bool live) const {
    const int k0b = kit * P::BK * 2;
    const int left = live ? (a.k - kit * P::BK) * 2 : 0;
    const int dst = stage * P::A_BYTES + lds_a;
#pragma unroll
    for (int j = 0; j < P::LA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_vptr)(smem + dst + j * 1024), 16,
                                               ca[j] * 16 < left ? va[j] : kOOB, k0b, 0, 0);
  }

  // this lane's B of iteration kit, one 16-byte chunk per k-step
  __device__ __forceinline__ void load_b(const KernelArgs &a, int kit, bool live,
                                         typename Elem<P::ET>::V8 (&b)[4]) const {
    using V8 = typename Elem<P::ET>::V8;
    const int k0b = kit * P::BK * 2;
    const int left = live ? (a.k - kit * P::BK) * 2 : 0;
    const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool ok = (4 * h + s) * 16 < left;
      b[s] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rb, ok ? vb + s * 16 : kOOB, k0b, 0));
    }
  }
};

// Iteration i (= PH mod D) of the narrow-m MAC loop.  On entry this wave
// has issued the loads of iterations up to i + D - 1, A then B per
// iteration; those of iteration i have landed once at most D - 1
// iterations' loads are outstanding.  The barrier then publishes A stage
// i mod (D + 1) and frees stage (i - 1) mod (D + 1), whose readers (the
// MFMAs of iteration i - 1) are done, for A of iteration i + D; B of
// iteration i + D goes into the registers this iteration's MFMAs have just
// read.
template <class P, int PH>
__device__ __forceinline__ void n_iter(const KernelArgs &a, const NLoader<P> &ld, int i, int n, int lb,
                                       typename Elem<P::ET>::V8 (&B)[P::D][4], typename P::Acc &acc) {
  using V8 = typename Elem<P::ET>::V8;
  __builtin_amdgcn_s_waitcnt(vmcnt_le((P::D - 1) * (P::LA + 4)));
  // a plain barrier: __syncthreads() would also wait for every load in
  // flight; the memory clobber keeps the compiler from moving LDS accesses
  // across it
  asm volatile("s_barrier" ::: "memory");
  ld.load_a(a, (i + P::D) % P::NSTAGE, lb + i + P::D, i + P::D < n);
  const int lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
  const char *As = smem + (i % P::NSTAGE) * P::A_BYTES + r * P::ROW;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    V8 af[P::MB];
    const int pos = ((4 * h + s) ^ P::swz(r)) << 4;  // swz(mb * 32 + r) = swz(r)
#pragma unroll
    for (int mb = 0; mb < P::MB; ++mb) af[mb] = *reinterpret_cast<const V8 *>(As + mb * 32 * P::ROW + pos);
#pragma unroll
    for (int mb = 0; mb < P::MB; ++mb) acc.v[mb] = h_mfma<P::ET>(B[PH][s], af[mb], acc.v[mb]);
  }
  ld.load_b(a, lb + i + P::D, i + P::D < n, B[PH]);
}

template <class P>
__device__ __forceinline__ void n_macloop(const KernelArgs &a, int m0, int n0, int lb, int le,
                                          typename P::Acc &acc) {
  using V8 = typename Elem<P::ET>::V8;
  static_assert(P::D == 3, "the loop below is unrolled for three iterations in flight");
  P::zero(acc);
  const int n = le - lb;
  if (n <= 0) return;
  NLoader<P> ld;
  ld.init(a, m0, n0);
  V8 B[P::D][4];
#pragma unroll
  for (int d = 0; d < P::D; ++d) {
    ld.load_a(a, d, lb + d, d < n);
    ld.load_b(a, lb + d, d < n, B[d]);
  }
  int i = 0;
  for (; i + 3 <= n; i += 3) {
    n_iter<P, 0>(a, ld, i, n, lb, B, acc);
    n_iter<P, 1>(a, ld, i + 1, n, lb, B, acc);
    n_iter<P, 2>(a, ld, i + 2, n, lb, B, acc);
  }
  if (i < n) n_iter<P, 0>(a, ld, i, n, lb, B, acc);
  if (i + 1 < n) n_iter<P, 1>(a, ld, i + 1, n, lb, B, acc);
  // every wave's loads (the last ones fetch nothing) and LDS reads are done
  // before the caller reuses LDS
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Epilogue of a narrow-m tile: lane l of wave w holds rows mb * 32 + (l & 31)
// and columns w * 32 + 8 g + 4 (l >> 5) + e of the tile.
template <class P>
__device__ __forceinline__ void n_epilogue(const KernelArgs &a, bool vec_ok, int m0, int n0,
                                           const typename P::Acc &acc) {
  const int w = wave_id(), lane = threadIdx.x & 63;
  const int c0 = n0 + w * 32 + 4 * (lane >> 5);
#pragma unroll
  for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4<P::ET>(a, vec_ok, m0 + mb * 32 + (lane & 31), c0 + 8 * g, P::get4(acc, mb * 4 + g));
}

// ============================================================== SGEMM
// TILE x TILE x 32 tiles, 4 waves as 2 x 2, wave tile TILE/2 x TILE/2,
// v_mfma_f32_16x16x4_f32: (TILE/32)^2 blocks per wave.  Two instances:
// 128 x 128 (4 x 4 blocks per wave, two workgroups per CU) and 64 x 64
// (2 x 2 blocks, for shapes with few 128 x 128 tiles: 1024^3 is one 64 x 64
// tile per CU with no partial exchange).  Within a group of 16 k, MFMA step
// q of lane group h = lane >> 4 multiplies k = 16 g + 4 h + q for both
// operands; a k-major operand reads its 4 values with one 128-bit LDS read,
// an mn-major operand reads one 32-bit value per step.
template <int TILE>
struct SCfgT {
  static_assert(TILE == 128 || TILE == 64, "fp32 tile");
  static constexpr int BM = TILE, BN = TILE, BK = 32, NT = 256;
  static constexpr int WTM = TILE / 2, WTN = TILE / 2, MB = WTM / 16, NB = WTN / 16, NACC = MB * NB;
  static constexpr int A_BYTES = BM * BK * 4, B_BYTES = BN * BK * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int MN_ROW = TILE * 4;  // bytes of one k row of an mn-major slice
};
using SCfg = SCfgT<128>;  // the instance ABFT runs on

// Direct-to-LDS loads of one operand's tile slices (fp32), with per-lane
// offsets computed once per tile; each k-iteration advances a scalar base.
//  k-major: BM rows (m or n) of BK fp32 (128 bytes), chunk c of row r at
//    position c ^ ((r >> 1) & 7); one 1 KiB load covers 8 rows; the base
//    of iteration kit is kit * BK * 4 bytes further.
//  mn-major: BK rows (k) of TILE fp32 (MN_ROW bytes), chunk c of row k at
//    position c ^ (4 * ((k >> 2) & 3)); one load covers 1024 / MN_ROW rows;
//    the base advances kit * BK * ld * 4 bytes.
// Rows past the matrix (and, in the iteration holding the end of k, k
// chunks or rows at or past k) are fetched out of range, i.e. as zeros.
template <class C, bool KMAJOR>
struct SLoader {
  static constexpr int LOADS = C::BM * C::BK * 4 / 1024 / (C::NT / 64);
  static constexpr int LPR = C::MN_ROW / 16;  // mn-major: lanes per k row
  static_assert(LOADS >= 1 && 64 % LPR == 0, "fp32 staging");
  const char *base;     // element (mn0, 0) of the operand
  int64_t range;        // bytes from base to the end of the operand
  int64_t kstep;        // bytes the slice advances per k-iteration
  uint32_t v[LOADS];
  int key[LOADS];       // k-major: chunk index; mn-major: k row within the slice
  int lds_first;        // LDS offset of this wave's first load within the operand's stage area

  __device__ __forceinline__ void init(const void *ptr, int64_t ld, int mn0, int mn_total, int k_total,
                                       int k_ext) {
    const int w = wave_id(), lane = threadIdx.x & 63;
    const int64_t ldb = ld * 4;
    lds_first = w * LOADS * 1024;
    if (KMAJOR) {
      base = static_cast<const char *>(ptr) + (int64_t)mn0 * ldb;
      range = (int64_t)(mn_total - 1 - mn0) * ldb + (int64_t)k_ext * 4;
      kstep = C::BK * 4;
#pragma unroll
      for (int j = 0; j < LOADS; ++j) {
        const int row = (w * LOADS + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        key[j] = c;
        v[j] = row < mn_total - mn0 ? (uint32_t)(row * ldb + c * 16) : kOOB;
      }
    } else {
      base = static_cast<const char *>(ptr) + (int64_t)mn0 * 4;
      range = (int64_t)(k_total - 1) * ldb + (int64_t)(mn_total - mn0) * 4;
      kstep = C::BK * ldb;
#pragma unroll
      for (int j = 0; j < LOADS; ++j) {
        const int kr = (w * LOADS + j) * (64 / LPR) + lane / LPR;
        const int c = (lane % LPR) ^ (4 * ((kr >> 2) & 3));
        key[j] = kr;
        v[j] = c * 4 < mn_total - mn0 ? (uint32_t)(kr * ldb + c * 16) : kOOB;
      }
    }
  }

  // Slice of k-iteration kit into the operand's area at LDS offset lds_off.
  // The buffer descriptor is rebuilt from the advanced base (scalar work),
  // so the hardware range check ends exactly at the operand's last element.
  __device__ __forceinline__ void load(int lds_off, int kit, int k_total) const {
    const int64_t adv = (int64_t)kit * kstep;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + adv, range - adv);
    const int left = k_total - kit * C::BK;  // k values from the slice start
    const int dst = lds_off + lds_first;
    if (left >= C::BK) {
#pragma unroll
      for (int j = 0; j < LOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(smem + dst + j * 1024), 16, v[j], 0, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < LOADS; ++j) {
        const bool ok = KMAJOR ? key[j] * 4 < left : key[j] < left;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(smem + dst + j * 1024), 16, ok ? v[j] : kOOB,
                                                 0, 0, 0);
      }
    }
  }
};

// Element (mn, k) of an mn-major fp32 stage area.
template <class C>
__device__ __forceinline__ float s_mn_elem(int base_off, int mn, int k) {
  const int c = mn >> 2, e = mn & 3;
  const int p = c ^ (4 * ((k >> 2) & 3));
  return *reinterpret_cast<const float *>(smem + base_off + k * C::MN_ROW + p * 16 + e * 4);
}

// Fragments of k-group g (16 values of k) of an LDS stage.  Within the
// group, MFMA step q of lane group h = lane >> 4 multiplies k = 16 g + 4 h + q
// for both operands: a k-major operand reads its four values with one
// 128-bit LDS read, an mn-major operand with one 32-bit read per step.
template <class C, bool AK, bool BKM>
__device__ __forceinline__ void s_frags(int stage, int g, int wm, int wn, f4_t (&av)[C::MB],
                                        f4_t (&bv)[C::NB]) {
  const int lane = threadIdx.x & 63;
  const int As = stage * C::STAGE, Bs = As + C::A_BYTES;
  const int h = lane >> 4, li = lane & 15;
  const int c = 4 * g + h;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    const int mn = wm * C::WTM + mb * 16 + li;
    if (AK) {
      av[mb] = *reinterpret_cast<const f4_t *>(smem + As + mn * 128 + ((c ^ ((mn >> 1) & 7)) << 4));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) av[mb][q] = s_mn_elem<C>(As, mn, 16 * g + 4 * h + q);
    }
  }
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    const int mn = wn * C::WTN + nb * 16 + li;
    if (BKM) {
      bv[nb] = *reinterpret_cast<const f4_t *>(smem + Bs + mn * 128 + ((c ^ ((mn >> 1) & 7)) << 4));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) bv[nb][q] = s_mn_elem<C>(Bs, mn, 16 * g + 4 * h + q);
    }
  }
}

template <class C>
__device__ __forceinline__ void s_mfmas(const f4_t (&av)[C::MB], const f4_t (&bv)[C::NB],
                                        f4_t (&acc)[C::NACC]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
        acc[mb * C::NB + nb] =
            __builtin_amdgcn_mfma_f32_16x16x4f32(bv[nb][q], av[mb][q], acc[mb * C::NB + nb], 0, 0, 0);
}

// ---------------------------------------------------------------- ABFT
//
// Threadblock-level ABFT of the fault-tolerant GEMM page, per work segment:
//   encodings   (e^T A)_k = sum_i A_ik,  (B e)_k = sum_j B_kj
//               over the tile's rows of A and columns of B;
//   checksums   rc_i += sum_k A_ik (B e)_k     -- row checksum of C = A B
//               cc_j += sum_k (e^T A)_k B_kj   -- column checksum.
// The encodings depend only on the operands, and every workgroup of a tile
// row (column) needs the same ones, so they are formed once per call by
// abft_prep_kernel, read from memory into LDS with the tiles two iterations
// ahead, and only the checksum updates run in the MAC loop, from the MFMA
// fragments already in registers.  At the end of the segment (before its
// partial store, or before the owner adds its peers' partials) the row and
// column sums of the accumulators are compared with the checksums: a row
// mismatches when |sum - rc_i| exceeds tau * 2^-24 * sqrt(k_seg) * ra_i or
// is not finite (likewise columns), where k_seg is the number of k values
// the segment accumulated: the rounding error of an fp32 dot product of
// length k grows like sqrt(k) u sum|a||b|.  ra_i stands for
// sum_k |a_ik| (|B| e)_k; the kernel uses its bound ||a_i||_1 max_k (|B| e)_k
// (row norm and tile maximum over all of k, formed once per call with the
// encodings), and likewise max_k (e^T|A|)_k ||b_j||_1 for columns, so the
// MAC loop carries no absolute checksums.  One mismatching row and one
// mismatching column locate the fault; the element is recomputed from its
// row checksum, c_ij = rc_i - sum_{l != j} c_il.  Any other pattern is
// reported as uncorrectable.  All reductions run in a fixed order.
struct AbftLds {
  alignas(16) float e[2][2][SCfg::BK];  // per stage: e^T A, B e
  float part[2][4][128];      // rc, cc: per lane group l >> 4 (a quarter of k)
  float sums[2][2][128];      // row sums per wave column, column sums per wave row
  float others[SCfg::NT / 64];
  int bad[4];                 // mismatching rows, one such row, columns, one such column
};

// Checksums of one lane (rows wm*64 + mb*16 + (l & 15) in a row wave,
// columns wn*64 + nb*16 + (l & 15) in a column wave) over the k values
// 4 (l >> 4) .. + 3 modulo 16.
struct AbftPart {
  float c[4];
};

// The ABFT working set in LDS (allocated only in kernels that use it).
__device__ __forceinline__ AbftLds &abft_lds() {
  __shared__ AbftLds L;
  return L;
}

// Checksum update from the MFMA fragments already in registers.  Lane l
// holds A at rows wm*64 + mb*16 + (l & 15) and B at columns
// wn*64 + nb*16 + (l & 15), at k = 16 g + 4 (l >> 4) + q of k-group g, so
//   rows:     c[mb] += sum_q A(row, k) (B e)_k
//   columns:  c[nb] += sum_q (e^T A)_k B(k, col).
// Both waves of a wave row hold the same rows of A (and both of a wave
// column the same columns of B): waves (0, 1) and (1, 0) form the row
// checksums of their wave rows, waves (0, 0) and (1, 1) the column checksums
// of their wave columns.  Entries past the end of k are zero in the staged
// tiles and in the encodings; rows and columns past the matrix give
// checksums that are never verified.
__device__ __forceinline__ bool abft_rows_wave(int wm, int wn) { return wm != wn; }

// The encodings that meet a lane's fragments of k-group g (B e for a row
// wave, e^T A for a column wave), at k = 16 g + 4 (l >> 4) + q, q = 0..3.
__device__ __forceinline__ f4_t abft_read_e(AbftLds &L, int stage, int g, bool rows) {
  const int h = (threadIdx.x & 63) >> 4;
  return *reinterpret_cast<const f4_t *>(&L.e[stage][rows ? 1 : 0][16 * g + 4 * h]);
}

__device__ __forceinline__ void abft_fma(const f4_t (&x)[4], f4_t e, AbftPart &pt) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) pt.c[j] += x[j][q] * e[q];
}

// One MFMA group and, in the ABFT kernels, the wave's checksum FMAs of that
// k-group, issued before the group (measured: the FMAs cost least there; set
// among the MFMAs they slow the group down).  The empty asm takes the
// checksums as operands, so that the compiler cannot sink the FMAs below the
// group.
template <class C, bool ABFT>
__device__ __forceinline__ void s_group(const f4_t (&av)[C::MB], const f4_t (&bv)[C::NB],
                                        f4_t (&acc)[C::NACC], bool rows, f4_t e, AbftPart &pt) {
  static_assert(!ABFT || C::BM == SCfg::BM, "ABFT runs on the 128 x 128 instance");
  if constexpr (ABFT) {
    if (rows)  // uniform over the wave
      abft_fma(av, e, pt);
    else
      abft_fma(bv, e, pt);
    asm volatile("" : "+v"(pt.c[0]), "+v"(pt.c[1]), "+v"(pt.c[2]), "+v"(pt.c[3]));
    __builtin_amdgcn_sched_barrier(0);
  }
  s_mfmas<C>(av, bv, acc);
}

__device__ __forceinline__ void abft_record(const KernelArgs &a, int64_t row, int64_t col, float delta,
                                            int status, int tile, int seg_begin) {
  const int idx = atomicAdd(&a.report->n_records, 1);
  if (idx < SK_ABFT_MAX_RECORDS) {
    sk_abft_record &r = a.report->records[idx];
    r.row = row; r.col = col; r.delta = delta; r.status = status; r.tile = tile; r.seg_begin = seg_begin;
  }
}

// Verification of one segment; acc in the 16x16 block layout of the SGEMM
// kernel (lane l of wave (wm, wn) holds row wm*64 + mb*16 + (l & 15) and
// columns wn*64 + nb*16 + 4*(l >> 4) + e of the tile).
__device__ __forceinline__ void abft_verify(const KernelArgs &a, AbftLds &L, const AbftPart &pt,
                                            f4_t (&acc)[SCfg::NACC], int m0, int n0, int lb, int le) {
  const int t = threadIdx.x, w = wave_id(), lane = t & 63;
  const int wm = w / 2, wn = w % 2;
  const int m_valid = a.m - m0, n_valid = a.n - n0;
  {
    // one partial per lane group: row checksums from the row waves, column
    // checksums from the column waves
    const int h = lane >> 4, li = lane & 15;
    const bool rows = abft_rows_wave(wm, wn);
    const int x0 = rows ? wm * SCfg::WTM + li : wn * SCfg::WTN + li;
#pragma unroll
    for (int j = 0; j < 4; ++j) L.part[rows ? 0 : 1][h][x0 + j * 16] = pt.c[j];
  }
  if (t < 4) L.bad[t] = t == 0 || t == 2 ? 0 : -1;
  // injected faults (testing): applied to the accumulator before verification
  for (int f = 0; f < a.n_faults; ++f) {
    const sk_fault F = a.faults[f];
    if (F.row < m0 || F.row >= m0 + SCfg::BM || F.col < n0 || F.col >= n0 + SCfg::BN) continue;
    if (F.iter < lb || F.iter >= le) continue;
    const int li = (int)(F.row - m0) - wm * SCfg::WTM, lj = (int)(F.col - n0) - wn * SCfg::WTN;
    if (li < 0 || li >= SCfg::WTM || lj < 0 || lj >= SCfg::WTN) continue;
    if ((lane & 15) != (li & 15) || (lane >> 4) != ((lj & 15) >> 2)) continue;
    // every accumulator index stays a compile-time constant (a runtime index
    // would move the whole accumulator array to scratch memory)
#pragma unroll
    for (int b = 0; b < SCfg::NACC; ++b) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (b != (li >> 4) * SCfg::NB + (lj >> 4) || e != (lj & 3)) continue;
        if (F.kind == 0) {
          acc[b][e] += F.value;
        } else {
          acc[b][e] = __uint_as_float(__float_as_uint(acc[b][e]) ^ (1u << (F.bit & 31)));
        }
      }
    }
  }
  // row and column sums of the accumulators (valid elements only)
#pragma unroll
  for (int mb = 0; mb < SCfg::MB; ++mb) {
    float sr = 0.f;
#pragma unroll
    for (int nb = 0; nb < SCfg::NB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = wn * SCfg::WTN + nb * 16 + 4 * (lane >> 4) + e;
        if (j < n_valid) sr += acc[mb * SCfg::NB + nb][e];
      }
    sr += __shfl_xor(sr, 16);
    sr += __shfl_xor(sr, 32);
    if ((lane >> 4) == 0) L.sums[0][wn][wm * SCfg::WTM + mb * 16 + lane] = sr;
  }
#pragma unroll
  for (int nb = 0; nb < SCfg::NB; ++nb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sc = 0.f;
#pragma unroll
      for (int mb = 0; mb < SCfg::MB; ++mb) {
        const int i = wm * SCfg::WTM + mb * 16 + (lane & 15);
        if (i < m_valid) sc += acc[mb * SCfg::NB + nb][e];
      }
      sc += __shfl_xor(sc, 1);
      sc += __shfl_xor(sc, 2);
      sc += __shfl_xor(sc, 4);
      sc += __shfl_xor(sc, 8);
      if ((lane & 15) == 0) L.sums[1][wm][wn * SCfg::WTN + nb * 16 + 4 * (lane >> 4) + e] = sc;
    }
  __syncthreads();
  const int kseg = ((le * SCfg::BK < a.k ? le * SCfg::BK : a.k) - lb * SCfg::BK);
  const float u = 5.9604644775390625e-08f * sqrtf((float)kseg);  // 2^-24 sqrt(k_seg)
  {
    const int x = t & 127;
    const bool is_row = t < 128;
    const bool valid = is_row ? x < m_valid : x < n_valid;
    float ratio = 0.f;  // margin of the checks that pass: |residual| / tau
    if (valid) {
      const int q = is_row ? 0 : 1;
      const float ck = ((L.part[q][0][x] + L.part[q][1][x]) + L.part[q][2][x]) + L.part[q][3][x];
      // bound of sum_k |a_ik| (|B| e)_k (row) or sum_k (e^T|A|)_k |b_kj| (column)
      const float ab = is_row ? a.norm_a[m0 + x] * a.emax_b[n0 / SCfg::BN]
                              : a.emax_a[m0 / SCfg::BM] * a.norm_b[n0 + x];
      const float sm = L.sums[is_row ? 0 : 1][0][x] + L.sums[is_row ? 0 : 1][1][x];
      const float r = sm - ck;
      const float tau = a.abft_tau * u * ab;
      if (!(fabsf(r) <= tau)) {
        atomicAdd(&L.bad[2 * q], 1);
        L.bad[2 * q + 1] = x;
      } else if (tau > 0.f) {
        ratio = fabsf(r) / tau;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ratio = fmaxf(ratio, __shfl_xor(ratio, o));
    // non-negative floats order like their bit patterns
    if ((t & 63) == 0 && ratio > 0.f) atomicMax(reinterpret_cast<int *>(&a.report->max_ratio), __float_as_int(ratio));
    if (t == 0) atomicAdd(&a.report->checked, min(m_valid, SCfg::BM) + min(n_valid, SCfg::BN));
  }
  __syncthreads();
  const int nbr = L.bad[0], nbc = L.bad[2];
  if (nbr == 0 && nbc == 0) return;
  const int tile = (m0 / SCfg::BM) * a.tiles_n + n0 / SCfg::BN;
  if (nbr == 1 && nbc == 1) {
    const int bi = L.bad[1], bj = L.bad[3];
    // sum of the bad row without the bad element, in a fixed order
    float s = 0.f;
    const int li = bi - wm * SCfg::WTM;
    if (li >= 0 && li < SCfg::WTM && (lane & 15) == (li & 15)) {
#pragma unroll
      for (int mb = 0; mb < SCfg::MB; ++mb) {
        if (mb != (li >> 4)) continue;
#pragma unroll
        for (int nb = 0; nb < SCfg::NB; ++nb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = wn * SCfg::WTN + nb * 16 + 4 * (lane >> 4) + e;
            if (j < n_valid && j != bj) s += acc[mb * SCfg::NB + nb][e];
          }
      }
    }
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 8);
    if (lane == 0) L.others[w] = s;
    __syncthreads();
    const int lj = bj - wn * SCfg::WTN;
    if (li >= 0 && li < SCfg::WTM && lj >= 0 && lj < SCfg::WTN && (lane & 15) == (li & 15) &&
        (lane >> 4) == ((lj & 15) >> 2)) {
      float others = 0.f;
#pragma unroll
      for (int v = 0; v < SCfg::NT / 64; ++v) others += L.others[v];
      const float rc = ((L.part[0][0][bi] + L.part[0][1][bi]) + L.part[0][2][bi]) + L.part[0][3][bi];
      const float fixed = rc - others;
      float delta = 0.f;
#pragma unroll
      for (int b = 0; b < SCfg::NACC; ++b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (b != (li >> 4) * SCfg::NB + (lj >> 4) || e != (lj & 3)) continue;
          delta = acc[b][e] - fixed;
          acc[b][e] = fixed;
        }
      }
      atomicAdd(&a.report->detected, 1);
      atomicAdd(&a.report->corrected, 1);
      abft_record(a, (int64_t)m0 + bi, (int64_t)n0 + bj, delta, 1, tile, lb);
    }
  } else if (t == 0) {
    atomicAdd(&a.report->detected, 1);
    atomicAdd(&a.report->uncorrectable, 1);
    abft_record(a, nbr == 1 ? (int64_t)m0 + L.bad[1] : -1, nbc == 1 ? (int64_t)n0 + L.bad[3] : -1, 0.f, 2,
                tile, lb);
  }
  __syncthreads();
}

// MacLoop of the fp32 kernel, same two-stage pipeline as the HGEMM one:
// the fragments of k-group 1 are read while the MFMAs of group 0 run; then
// wait for this wave's loads of the next stage, barrier, issue the loads of
// iteration i+2 into this stage's buffer and read group 0 of the next stage
// while the MFMAs of group 1 run.  ABFT: each group's checksum FMAs run
// just before its MFMAs, from the same fragments.
template <class C, bool AK, bool BKM, bool ABFT>
__device__ __forceinline__ void s_macloop(const KernelArgs &a, int m0, int n0, int lb, int le,
                                          f4_t (&acc)[C::NACC]) {
  const int w = wave_id();
  const int wm = w / 2, wn = w % 2;
#pragma unroll
  for (int i = 0; i < C::NACC; ++i) acc[i] = f4_t{0.f, 0.f, 0.f, 0.f};
  const int n = le - lb;
  if (n <= 0) return;
  AbftPart pt{};
  // ABFT: wave 0 carries the encodings of a k-iteration (lanes 0-31: the
  // tile row's e^T A, lanes 32-63: the tile column's B e) from memory to the
  // stage's LDS slot: loaded with the stage's tiles, stored after the next
  // wait for them, read after the barrier after that.
  const int wv = wave_id();
  const bool enc_lane = ABFT && wv == 0;
  const float *esrc = nullptr;  // this lane's encodings
  float ev = 0.f, ev1 = 0.f;
  if constexpr (ABFT) {
    const int lane = threadIdx.x & 63;
    esrc = (lane < 32 ? a.enc_a + (int64_t)(m0 / C::BM) * a.enc_kb * 32
                      : a.enc_b + (int64_t)(n0 / C::BN) * a.enc_kb * 32) + (lane & 31);
    if (enc_lane) {
      ev = esrc[(int64_t)lb * 32];
      if (n > 1) ev1 = esrc[(int64_t)(lb + 1) * 32];
    }
  }
  SLoader<C, AK> la;
  SLoader<C, BKM> lbd;
  la.init(a.A, a.lda, m0, a.m, a.k, a.a_kext);
  lbd.init(a.B, a.ldb, n0, a.n, a.k, a.b_kext);
  auto load = [&](int stage, int kit) {
    la.load(stage * C::STAGE, kit, a.k);
    lbd.load(stage * C::STAGE + C::A_BYTES, kit, a.k);
  };
  load(0, lb);
  if (n > 1) {
    load(1, lb + 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_le(SLoader<C, AK>::LOADS + SLoader<C, BKM>::LOADS));
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  if constexpr (ABFT) {
    if (enc_lane) {
      AbftLds &L = abft_lds();
      (&L.e[0][0][0])[threadIdx.x] = ev;
      if (n > 1) (&L.e[1][0][0])[threadIdx.x] = ev1;
    }
  }
  __syncthreads();
  f4_t a0[C::MB], b0[C::NB], a1[C::MB], b1[C::NB];
  s_frags<C, AK, BKM>(0, 0, wm, wn, a0, b0);
  int buf = 0;
  const bool rows = abft_rows_wave(wm, wn);
  f4_t e0{}, e1{};  // ABFT: the wave's encodings for the two k-groups of this stage
  for (int i = 0; i < n; ++i) {
    // ABFT: both groups' encodings are read before the barrier (wave 0
    // stores those of iteration i+2 into this slot after it), and before
    // the fragments, so that the first FMAs wait for them alone
    if constexpr (ABFT) {
      e0 = abft_read_e(abft_lds(), buf, 0, rows);
      e1 = abft_read_e(abft_lds(), buf, 1, rows);
    }
    s_frags<C, AK, BKM>(buf, 1, wm, wn, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    s_group<C, ABFT>(a0, b0, acc, rows, e0, pt);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (ABFT) {
      // the encodings of iteration i+1, loaded at iteration i-1 (the
      // prologue stored those of iterations 0 and 1)
      if (enc_lane && i >= 1 && i + 1 < n) (&abft_lds().e[buf ^ 1][0][0])[threadIdx.x] = ev;
    }
    __syncthreads();
    if (i + 2 < n) {
      load(buf, lb + i + 2);
      if constexpr (ABFT) {
        if (enc_lane) ev = esrc[(int64_t)(lb + i + 2) * 32];
      }
    }
    if (i + 1 < n) s_frags<C, AK, BKM>(buf ^ 1, 0, wm, wn, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    s_group<C, ABFT>(a1, b1, acc, rows, e1, pt);
    __builtin_amdgcn_sched_barrier(0);
    buf ^= 1;
  }
  if constexpr (ABFT) abft_verify(a, abft_lds(), pt, acc, m0, n0, lb, le);
}

template <int TILE>
struct SPolicy {
  using C = SCfgT<TILE>;
  static constexpr int BM = C::BM, BN = C::BN, NT = C::NT;
  static constexpr int NACC4 = C::NACC;
  static constexpr int LDS_BYTES = 2 * C::STAGE;
  struct Acc { f4_t v[C::NACC]; };
  static __device__ __forceinline__ f4_t get4(const Acc &c, int i) { return c.v[i]; }
  static __device__ __forceinline__ void add4(Acc &c, int i, f4_t x) { c.v[i] += x; }
};

// 16x16 block layout (SGEMM): lane l of a wave holds, for block (mb, nb),
// row (l & 15) and columns 4*(l >> 4) + {0..3} of the block.
template <int TILE>
__device__ __forceinline__ void s_epilogue(const KernelArgs &a, bool vec_ok, int m0, int n0,
                                           const typename SPolicy<TILE>::Acc &acc) {
  using C = SCfgT<TILE>;
  const int w = wave_id(), lane = threadIdx.x & 63;
  constexpr int WN = C::BN / C::WTN;
  const int r0 = m0 + (w / WN) * C::WTM, c0 = n0 + (w % WN) * C::WTN;
  // a tile wholly inside C: straight-line stores (as in the HGEMM epilogue)
  if (vec_ok && m0 + C::BM <= a.m && n0 + C::BN <= a.n) {
    float *cb = static_cast<float *>(a.C) + (int64_t)(r0 + (lane & 15)) * a.ldc + c0 + 4 * (lane >> 4);
    const int64_t rstep = (int64_t)16 * a.ldc;
    if (a.beta == 0.f) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
          Elem<SK_F32>::st4(cb + mb * rstep, nb * 16, a.alpha * acc.v[mb * C::NB + nb]);
    } else {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          float *q = cb + mb * rstep;
          Elem<SK_F32>::st4(q, nb * 16, a.alpha * acc.v[mb * C::NB + nb] + a.beta * Elem<SK_F32>::ld4(q, nb * 16));
        }
    }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
      store4<SK_F32>(a, vec_ok, r0 + mb * 16 + (lane & 15), c0 + nb * 16 + 4 * (lane >> 4),
                     acc.v[mb * C::NB + nb]);
}

// ======================================================= work iteration

// Runs one segment: MacLoop, then partial store, or fixup + epilogue.
template <class P, class MacLoop, class Epilogue>
__device__ __forceinline__ void run_segment(const KernelArgs &a, const Sched &S, int x, const Segment &g,
                                            MacLoop macloop, Epilogue epilogue) {
  typename P::Acc acc;
  const int tile = (int)g.tile;
  const int tm = sched_div(tile, S.tiles_n), tn = tile - tm * S.tiles_n;
  const int m0 = tm * P::BM, n0 = tn * P::BN;
  macloop(m0, n0, (int)g.lb, (int)g.le, acc);
  // One call site each for the partial store, the partial add and the
  // epilogue (a second inlined copy of them doubles the live accumulators).
  //  page order: a non-owner stores; the owner adds x+1 .. last_peer;
  //  tree (sk_gemm.h, fixup_tree): with r = x - first, at level l a
  //  workgroup with bit l of r set stores, else adds the subtree of r + 2^l.
  const bool tree = S.tree != 0;
  const int first = g.first < 0 ? x : (int)g.first, last = g.last < 0 ? x : (int)g.last;
  const int pieces = last - first + 1, r = x - first;
  bool publish = false;
  for (int step = 0;; ++step) {
    int child;
    if (tree) {
      if ((1 << step) >= pieces) break;
      if (r & (1 << step)) {
        publish = true;
        break;
      }
      child = r + (1 << step) < pieces ? first + r + (1 << step) : -1;
    } else {
      if (!g.started) {
        publish = true;
        break;
      }
      child = x + 1 + step;
      if (child > (int)g.last_peer) break;
    }
    if (child >= 0 && wait_flag(a, child)) add_partial<P>(a, child, acc);
  }
  if (publish)
    store_partial<P>(a, x, acc);
  else
    epilogue(m0, n0, acc);
}

// The schedule, read from the kernel arguments once and held in scalar
// registers: an empty asm statement that may change each field makes it a
// computed value, which the compiler keeps, instead of a load it re-issues
// after every branch of the walk (each such reload waited a full memory
// round trip at kernel start, about a microsecond in all before the first
// tile).
__device__ __forceinline__ int32_t sgpr(int32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ Sched sched_in_sgprs(const Sched &s) {
  Sched r;
  r.ipt = sgpr(s.ipt); r.tiles = sgpr(s.tiles); r.tiles_m = sgpr(s.tiles_m); r.tiles_n = sgpr(s.tiles_n);
  r.sk_tiles = sgpr(s.sk_tiles); r.sk_q = sgpr(s.sk_q); r.sk_r = sgpr(s.sk_r); r.grid = sgpr(s.grid);
  r.phase_div = sgpr(s.phase_div); r.blocks = sgpr(s.blocks); r.block_len = sgpr(s.block_len);
  r.block_cut = sgpr(s.block_cut); r.group_rows = sgpr(s.group_rows); r.tree = sgpr(s.tree);
  return r;
}

// All segments of workgroup blockIdx.x, in the order the schedule gives
// them: its Stream-K range, then its data-parallel tiles.
template <class P, class MacLoop, class Epilogue>
__device__ __forceinline__ void run_workgroup(const KernelArgs &a, MacLoop macloop, Epilogue epilogue) {
  const int x = blockIdx.x;
  const Sched S = sched_in_sgprs(a.sched);
  SegIter I = sched_begin(S, x);
  Segment g;
  while (sched_next(S, I, g)) run_segment<P>(a, S, x, g, macloop, epilogue);
}

template <class P, bool BZ>
__global__ __launch_bounds__(P::NT, P::WPE) void hgemm_kernel(KernelArgs a, int vec_ok) {
  run_workgroup<P>(
      a, [&](int m0, int n0, int lb, int le, typename P::Acc &acc) { h_macloop_la2<P>(a, m0, n0, lb, le, acc); },
      [&](int m0, int n0, const typename P::Acc &acc) { h_epilogue<P, BZ>(a, vec_ok != 0, m0, n0, acc); });
}

template <class P>
__global__ __launch_bounds__(P::NT, 1) void ngemm_kernel(KernelArgs a, int vec_ok) {
  run_workgroup<P>(
      a, [&](int m0, int n0, int lb, int le, typename P::Acc &acc) { n_macloop<P>(a, m0, n0, lb, le, acc); },
      [&](int m0, int n0, const typename P::Acc &acc) { n_epilogue<P>(a, vec_ok != 0, m0, n0, acc); });
}

template <int TILE, bool AK, bool BKM, bool ABFT>
__global__ __launch_bounds__(SCfgT<TILE>::NT, TILE == 128 ? 2 : 4) void sgemm_kernel(KernelArgs a, int vec_ok) {
  using P = SPolicy<TILE>;
  run_workgroup<P>(
      a,
      [&](int m0, int n0, int lb, int le, typename P::Acc &acc) {
        s_macloop<typename P::C, AK, BKM, ABFT>(a, m0, n0, lb, le, acc.v);
      },
      [&](int m0, int n0, const typename P::Acc &acc) { s_epilogue<TILE>(a, vec_ok != 0, m0, n0, acc); });
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

// Repack: dst[r * ldd + l] = src(r, l) for l < k, 0 for k <= l < ldd, rows
// r < rows; src(r, l) is src[r * lds + l] (k-major) or src[l * lds + r]
// (mn-major).  One workgroup per 64 x 64 block, 16 bytes per lane on both
// sides where the operands allow it (the destination always does; the
// source is read in pieces of src_align bytes, 16, 8, 4 or the element
// size: the largest power of two dividing both its base address and its
// row pitch): a k-major source is copied row by row; an mn-major one is
// transposed through LDS -- loaded along r into tile rows of l (rows of 64
// elements plus 8 bytes, so that the element reads of the store side fall
// at most two to a bank), and read back along l.
template <typename U>
__global__ __launch_bounds__(256) void pack_kernel(const U *src, int64_t lds, int src_kmajor, int src_align,
                                                   int64_t rows, int64_t k, U *dst, int64_t ldd) {
  constexpr int EPV = 16 / sizeof(U);         // elements per 16-byte vector
  constexpr int VPR = 64 / EPV;              // vectors per 64-element row
  constexpr int RPP = 256 / VPR;             // rows per pass of the workgroup
  constexpr int PITCH = 64 + 8 / sizeof(U);  // elements per LDS tile row
  static_assert((PITCH * sizeof(U)) % 8 == 0, "8-byte aligned tile rows");
  union Vec {
    u4_t v;
    u2_t h[2];
    uint32_t w[4];
    U e[EPV];
  };
  // one whole 16-byte vector of the source at p (every element in range),
  // in pieces of src_align bytes
  auto load_vec = [src_align](const U *p, Vec &x) {
    if (src_align >= 16) {
      x.v = *reinterpret_cast<const u4_t *>(p);
    } else if (src_align == 8) {
      x.h[0] = reinterpret_cast<const u2_t *>(p)[0];
      x.h[1] = reinterpret_cast<const u2_t *>(p)[1];
    } else if (src_align == 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) x.w[q] = reinterpret_cast<const uint32_t *>(p)[q];
    } else {
#pragma unroll
      for (int e = 0; e < EPV; ++e) x.e[e] = p[e];
    }
  };
  const int64_t r0 = (int64_t)blockIdx.y * 64, l0 = (int64_t)blockIdx.x * 64;
  const int t = threadIdx.x, vi = t % VPR, ri = t / VPR;
  const int64_t l = l0 + vi * EPV;  // this lane's first element along l (k-major copy and store side)
  if (src_kmajor) {
    for (int p = 0; p < 64; p += RPP) {
      const int64_t r = r0 + p + ri;
      if (r >= rows || l >= ldd) continue;
      Vec x;
      if (l + EPV <= k) {
        load_vec(src + r * lds + l, x);
      } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e) x.e[e] = l + e < k ? src[r * lds + l + e] : U(0);
      }
      if (l + EPV <= ldd) {
        *reinterpret_cast<u4_t *>(dst + r * ldd + l) = x.v;
      } else {
        for (int e = 0; e < EPV && l + e < ldd; ++e) dst[r * ldd + l + e] = x.e[e];
      }
    }
    return;
  }
  __shared__ __align__(16) U tile[64 * PITCH];  // tile[li][ri]: element (r0 + ri, l0 + li)
  for (int p = 0; p < 64; p += RPP) {
    const int li = p + ri;
    const int64_t ll = l0 + li, r = r0 + vi * EPV;
    Vec x;
    if (ll < k && r + EPV <= rows) {
      load_vec(src + ll * lds + r, x);
    } else {
#pragma unroll
      for (int e = 0; e < EPV; ++e) x.e[e] = ll < k && r + e < rows ? src[ll * lds + r + e] : U(0);
    }
    u2_t *d = reinterpret_cast<u2_t *>(tile + li * PITCH + vi * EPV);
    d[0] = x.h[0];
    d[1] = x.h[1];
  }
  __syncthreads();
  for (int p = 0; p < 64; p += RPP) {
    const int rr = p + ri;
    const int64_t r = r0 + rr;
    if (r >= rows || l >= ldd) continue;
    Vec x;
#pragma unroll
    for (int e = 0; e < EPV; ++e) x.e[e] = tile[(vi * EPV + e) * PITCH + rr];
    if (l + EPV <= ldd) {
      *reinterpret_cast<u4_t *>(dst + r * ldd + l) = x.v;
    } else {
      for (int e = 0; e < EPV && l + e < ldd; ++e) dst[r * ldd + l + e] = x.e[e];
    }
  }
}

// ABFT preparation (both operands in one launch).  Workgroup (operand,
// tile, group) walks the group's chunks of 64 values of k in order; the
// next chunk's loads are in flight while the current one is reduced.  Per
// chunk the tile's 128 rows are staged in LDS (a wave reads 64 consecutive
// elements of the operand in either storage order), four threads per k sum
// 32 rows each in row order and the four sums are added in order (the
// encoding e^T X of the tile per k, rows past the matrix left out, k past
// the end zero), and likewise for the absolute values.  Over the group, each
// row's sum of absolute values (chunks in order, k in order) goes to
// rowabs[group][row] and the largest column sum of absolute values to
// tmax[tile][group].  The last workgroup of a tile to finish (a counter per
// tile) adds each row's group sums in order into norm[row] and takes the
// largest tmax of the tile into emax[tile].
template <bool KMAJOR>
__device__ __forceinline__ void prep_load(const float *X, int64_t ld, int64_t r0, int64_t rv, int64_t k0, int64_t k,
                                          f4_t (&x)[8]) {
  const int t = threadIdx.x;
  // 16-byte loads where all four elements are inside the operand (rows of
  // a k-major operand and k-lines of an mn-major one start 16-byte aligned:
  // the leading dimension is a multiple of four and the base is aligned),
  // single elements at the edges
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    x[q] = f4_t{0.f, 0.f, 0.f, 0.f};
    if (KMAJOR) {
      const int kc = t & 15, r = (t >> 4) + 16 * q;  // k = k0 + 4 kc .. + 3
      const int64_t kk0 = k0 + 4 * kc;
      if (r < rv) {
        const float *src = X + (r0 + r) * ld + kk0;
        if (kk0 + 3 < k) {
          x[q] = *reinterpret_cast<const f4_t *>(src);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kk0 + e < k) x[q][e] = src[e];
        }
      }
    } else {
      const int r = 4 * (t & 31), kk = (t >> 5) + 8 * q;  // rows r .. r + 3
      if (k0 + kk < k) {
        const float *src = X + (k0 + kk) * ld + r0 + r;
        if (r + 3 < rv) {
          x[q] = *reinterpret_cast<const f4_t *>(src);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (r + e < rv) x[q][e] = src[e];
        }
      }
    }
  }
}

template <bool KMAJOR>
__device__ __forceinline__ void prep_stage(float (&T)[64][129], const f4_t (&x)[8]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    if (KMAJOR) {
      const int kc = t & 15, r = (t >> 4) + 16 * q;
#pragma unroll
      for (int e = 0; e < 4; ++e) T[4 * kc + e][r] = x[q][e];
    } else {
      const int r = 4 * (t & 31), kk = (t >> 5) + 8 * q;
#pragma unroll
      for (int e = 0; e < 4; ++e) T[kk][r + e] = x[q][e];
    }
  }
}

template <bool KMAJOR>
__device__ __forceinline__ void prep_walk(const AbftPrepArgs &p, const AbftPrepOperand &o, int64_t tile,
                                          int64_t c_begin, int64_t c_end, float (&T)[64][129],
                                          float (&P)[2][4][64], float &rowsum, float &tmx) {
  const int t = threadIdx.x;
  const int64_t r0 = tile * 128, rows = o.rows, k = p.k, kb = p.kb;
  const int64_t rv = rows - r0 < 128 ? rows - r0 : 128;  // valid rows of the tile
  f4_t x[8];
  prep_load<KMAJOR>(o.X, o.ld, r0, rv, c_begin * 64, k, x);
  for (int64_t c = c_begin; c < c_end; ++c) {
    __syncthreads();  // the previous chunk's readers of T and P are done
    prep_stage<KMAJOR>(T, x);
    if (c + 1 < c_end) prep_load<KMAJOR>(o.X, o.ld, r0, rv, (c + 1) * 64, k, x);
    __syncthreads();
    {
      const int kk = t & 63, g = t >> 6;
      float sm = 0.f, sa = 0.f;
#pragma unroll 8
      for (int r = 32 * g; r < 32 * g + 32; ++r) {
        const float v = T[kk][r];
        sm += v;
        sa += fabsf(v);
      }
      P[0][g][kk] = sm;
      P[1][g][kk] = sa;
    }
    if (t < 128) {
#pragma unroll 8
      for (int kk = 0; kk < 64; ++kk) rowsum += fabsf(T[kk][t]);
    }
    __syncthreads();
    if (t < 64) {
      const int64_t l = c * 64 + t;
      const float sm = ((P[0][0][t] + P[0][1][t]) + P[0][2][t]) + P[0][3][t];
      float sa = ((P[1][0][t] + P[1][1][t]) + P[1][2][t]) + P[1][3][t];
      if (l < kb * 32) o.enc[(tile * kb + l / 32) * 32 + (l % 32)] = sm;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sa = fmaxf(sa, __shfl_xor(sa, off));
      tmx = fmaxf(tmx, sa);
    }
  }
}

__global__ __launch_bounds__(256, 4) void abft_prep_kernel(AbftPrepArgs p) {
  __shared__ float T[64][129];
  __shared__ float P[2][4][64];
  __shared__ int last;
  const int t = threadIdx.x;
  const int64_t groups = p.groups, gsize = p.group_chunks;
  const int64_t blocks_a = p.op[0].tiles * groups;
  const int which = blockIdx.x < blocks_a ? 0 : 1;
  const AbftPrepOperand &o = p.op[which];
  const int64_t b = blockIdx.x - (which ? blocks_a : 0);
  const int64_t tile = b / groups, grp = b % groups;
  const int64_t c_begin = grp * gsize, c_end = c_begin + gsize < p.chunks ? c_begin + gsize : p.chunks;
  const int64_t r0 = tile * 128, rows = o.rows;
  const int64_t rv = rows - r0 < 128 ? rows - r0 : 128;
  if (blockIdx.x == 0 && p.report != nullptr) {
    int32_t *w = reinterpret_cast<int32_t *>(p.report);
    for (int i = t; i < (int)(sizeof(sk_abft_report) / 4); i += 256) w[i] = 0;
  }
  float rowsum = 0.f, tmx = 0.f;
  if (o.kmajor)
    prep_walk<true>(p, o, tile, c_begin, c_end, T, P, rowsum, tmx);
  else
    prep_walk<false>(p, o, tile, c_begin, c_end, T, P, rowsum, tmx);
  // The last workgroup of the tile reads what the others wrote to rowabs
  // and tmax.  As in the Stream-K fixup, no release or acquire (each would
  // write back or invalidate a whole L2): those arrays are written and read
  // with agent-coherent relaxed atomics (sc1 accesses), and the count
  // follows this workgroup's completed stores (wait, barrier).
  if (t < rv) __hip_atomic_store(&o.rowabs[grp * rows + r0 + t], rowsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t == 0) __hip_atomic_store(&o.tmax[tile * groups + grp], tmx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
  __syncthreads();
  uint32_t *ctr = p.counters + (which ? p.op[0].tiles : 0) + tile;
  if (t == 0) {
    const uint32_t done = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = done + 1 == (uint32_t)groups;
  }
  __syncthreads();
  if (!last) return;
  if (t < rv) {
    float s = 0.f;
    for (int64_t g = 0; g < groups; ++g)
      s += __hip_atomic_load(&o.rowabs[g * rows + r0 + t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    o.norm[r0 + t] = s;
  }
  if (t < 64) {
    float mx = 0.f;
    for (int64_t g = t; g < groups; g += 64)
      mx = fmaxf(mx, __hip_atomic_load(&o.tmax[tile * groups + g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (t == 0) {
      o.emax[tile] = mx;
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
    }
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

// Entry point of the fp32 kernel for the tile instance (0: 128 x 128, 1:
// 64 x 64, no ABFT), the operands' storage orders and the mode.
static const void *sgemm_entry(int inst, bool ak, bool bk, bool abft) {
  using namespace dev;
  if (inst == 1) {
    if (ak && bk) return reinterpret_cast<const void *>(&sgemm_kernel<64, true, true, false>);
    if (ak) return reinterpret_cast<const void *>(&sgemm_kernel<64, true, false, false>);
    if (bk) return reinterpret_cast<const void *>(&sgemm_kernel<64, false, true, false>);
    return reinterpret_cast<const void *>(&sgemm_kernel<64, false, false, false>);
  }
  if (abft) {
    if (ak && bk) return reinterpret_cast<const void *>(&sgemm_kernel<128, true, true, true>);
    if (ak) return reinterpret_cast<const void *>(&sgemm_kernel<128, true, false, true>);
    if (bk) return reinterpret_cast<const void *>(&sgemm_kernel<128, false, true, true>);
    return reinterpret_cast<const void *>(&sgemm_kernel<128, false, false, true>);
  }
  if (ak && bk) return reinterpret_cast<const void *>(&sgemm_kernel<128, true, true, false>);
  if (ak) return reinterpret_cast<const void *>(&sgemm_kernel<128, true, false, false>);
  if (bk) return reinterpret_cast<const void *>(&sgemm_kernel<128, false, true, false>);
  return reinterpret_cast<const void *>(&sgemm_kernel<128, false, false, false>);
}

// Entry point of an fp16/bf16 tile instance.
template <int DT>
static const void *ngemm_entry(int inst) {
  using namespace dev;
  switch (inst) {
    case 2: return reinterpret_cast<const void *>(&ngemm_kernel<NPolicy<DT, 2>>);
    case 3: return reinterpret_cast<const void *>(&ngemm_kernel<NPolicy<DT, 4>>);
    case 4: return reinterpret_cast<const void *>(&ngemm_kernel<NPolicy<DT, 6>>);
    default: return reinterpret_cast<const void *>(&ngemm_kernel<NPolicy<DT, 8>>);
  }
}

template <int DT, int TILE, bool BMN, bool AMN>
static const void *hgemm_entry_bz(bool beta_zero) {
  using namespace dev;
  using P = HPolicy<DT, TILE, (TILE == 256 ? 8 : 4), BMN, AMN>;
  return beta_zero ? reinterpret_cast<const void *>(&hgemm_kernel<P, true>)
                   : reinterpret_cast<const void *>(&hgemm_kernel<P, false>);
}

template <int DT, int TILE>
static const void *hgemm_entry_b(bool beta_zero, bool b_mn, bool a_mn) {
  if (a_mn)
    return b_mn ? hgemm_entry_bz<DT, TILE, true, true>(beta_zero) : hgemm_entry_bz<DT, TILE, false, true>(beta_zero);
  return b_mn ? hgemm_entry_bz<DT, TILE, true, false>(beta_zero) : hgemm_entry_bz<DT, TILE, false, false>(beta_zero);
}

// b_mn / a_mn: B read n-contiguous / A read m-contiguous (instances 0 and 1)
static const void *hgemm_entry(int dtype, int inst, bool beta_zero, bool b_mn, bool a_mn) {
  if (inst >= 2) return dtype == SK_F16 ? ngemm_entry<SK_F16>(inst) : ngemm_entry<SK_BF16>(inst);
  if (inst == 1)
    return dtype == SK_F16 ? hgemm_entry_b<SK_F16, 128>(beta_zero, b_mn, a_mn)
                           : hgemm_entry_b<SK_BF16, 128>(beta_zero, b_mn, a_mn);
  return dtype == SK_F16 ? hgemm_entry_b<SK_F16, 256>(beta_zero, b_mn, a_mn)
                         : hgemm_entry_b<SK_BF16, 256>(beta_zero, b_mn, a_mn);
}

int launch_gemm(const Plan &p, const KernelArgs &a, hipStream_t stream) {
  dim3 grid(p.grid), block(p.cfg.threads);
  const int vec_ok = c_vec_ok(a, p.dtype) ? 1 : 0;
  const size_t lds = p.cfg.lds_bytes;
  // the narrow instance reads k-contiguous operands only
  if (p.dtype != SK_F32 && (!a.a_kmajor || !a.b_kmajor) && p.cfg.inst >= 2) return (int)hipErrorInvalidValue;
  const void *f = p.dtype != SK_F32 ? hgemm_entry(p.dtype, p.cfg.inst, a.beta == 0.f, !a.b_kmajor, !a.a_kmajor)
                                    : sgemm_entry(p.cfg.inst, a.a_kmajor != 0, a.b_kmajor != 0, a.abft != 0);
  void *params[] = {const_cast<KernelArgs *>(&a), const_cast<int *>(&vec_ok)};
  return (int)hipLaunchKernel(f, grid, block, params, lds, stream);
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
  // the kernel writes 16-byte vectors into dst: 16-byte aligned rows of it
  const int es = dtype == SK_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(dst) % 16 != 0 || (ldd * es) % 16 != 0) return (int)hipErrorInvalidValue;
  // the largest of 16, 8, 4 bytes dividing the source's base and row pitch,
  // else the element size
  int src_align = 16;
  while (src_align > es && (reinterpret_cast<uintptr_t>(src) % src_align != 0 || (lds * es) % src_align != 0))
    src_align /= 2;
  if (dtype == SK_F32)
    hipLaunchKernelGGL(dev::pack_kernel<uint32_t>, grid, block, 0, stream,
                       static_cast<const uint32_t *>(src), lds, src_kmajor ? 1 : 0, src_align, rows, k,
                       static_cast<uint32_t *>(dst), ldd);
  else
    hipLaunchKernelGGL(dev::pack_kernel<uint16_t>, grid, block, 0, stream,
                       static_cast<const uint16_t *>(src), lds, src_kmajor ? 1 : 0, src_align, rows, k,
                       static_cast<uint16_t *>(dst), ldd);
  return (int)hipGetLastError();
}

int launch_zero_report(sk_abft_report *report, hipStream_t stream) {
  const int64_t words = (int64_t)(sizeof(sk_abft_report) / 4);
  hipLaunchKernelGGL(dev::zero_words_kernel, dim3(1), dim3(256), 0, stream,
                     reinterpret_cast<int32_t *>(report), words);
  return (int)hipGetLastError();
}

int launch_abft_prep(const AbftPrepArgs &args, hipStream_t stream) {
  const int64_t blocks = (args.op[0].tiles + args.op[1].tiles) * args.groups;
  if (args.group_chunks <= 0 || args.groups != (args.chunks + args.group_chunks - 1) / args.group_chunks)
    return (int)hipErrorInvalidValue;
  if (blocks <= 0 || blocks > INT32_MAX) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(dev::abft_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, args);
  return (int)hipGetLastError();
}

int kernel_occupancy(int dtype, bool abft, int inst, int *blocks_per_cu) {
  const TileCfg c = tile_cfg(dtype, inst);
  hipError_t e = hipSuccess;
  int nb = 0;
  if (dtype == SK_F32) {
    // the four storage-order instances of the mode: the slot count is the
    // smallest occupancy among them
    nb = 1 << 20;
    for (int i = 0; i < 4 && e == hipSuccess; ++i) {
      const void *f = sgemm_entry(inst, i & 1, (i >> 1) & 1, abft);
      e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, c.lds_bytes);
      int o = 0;
      if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, f, c.threads, c.lds_bytes);
      if (o < nb) nb = o;
    }
  } else {
    // both beta forms and both orders of A and of B: the smaller occupancy
    nb = 1 << 20;
    for (int v = 0; v < 8 && e == hipSuccess; ++v) {
      const void *f = hgemm_entry(dtype, inst, (v & 1) != 0, inst < 2 && (v & 2) != 0, inst < 2 && (v & 4) != 0);
      e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, c.lds_bytes);
      int o = 0;
      if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, f, c.threads, c.lds_bytes);
      if (o < nb) nb = o;
    }
  }
  *blocks_per_cu = nb;
  return (int)e;
}

}  // namespace sk
