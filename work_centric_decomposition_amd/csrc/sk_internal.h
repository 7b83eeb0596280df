// sk_internal.h -- definitions shared by the library's host code (planner,
// C ABI) and its HIP kernels.  Not part of the public interface.
#pragma once

#include <stdint.h>

#include "../../include/sk_gemm.h"

namespace sk {

// Tile shape and launch shape of each kernel instance.
//   HGEMM (fp16/bf16): 256 x 256 x 64 tiles, 512 threads (8 wave64s laid out
//   2 x 4, two per SIMD, each owning a 128 x 64 block of C), two LDS stages
//   of 64 KiB, one workgroup per CU.
//   SGEMM (fp32): 128 x 128 x 32 tiles, 256 threads (4 wave64s, 2 x 2, each
//   64 x 64), two LDS stages of 32 KiB, two workgroups per CU.
struct TileCfg {
  int bm, bn, bk;
  int threads;
  int occupancy;     // workgroups per CU
  int lds_bytes;     // dynamic LDS per workgroup
  // default grid-size model constants, in units of one MAC iteration
  float a, b, c, d;
};

// k-depth of an HGEMM tile iteration and number of LDS stages (a build-time
// choice; the default is two stages of 64).
#ifndef SK_HGEMM_BK
#define SK_HGEMM_BK 64
#endif
#ifndef SK_HGEMM_STAGES
#define SK_HGEMM_STAGES 2
#endif
// waves per HGEMM workgroup: 8 (two per SIMD, 128 x 64 wave tiles) or 4 (one
// per SIMD, 128 x 128 wave tiles)
#ifndef SK_HGEMM_WAVES
#define SK_HGEMM_WAVES 8
#endif

inline TileCfg tile_cfg(int dtype) {
  // fp32: a 64 KiB partial costs about one and a half 32-deep iterations
  if (dtype == SK_F32) return TileCfg{128, 128, 32, 256, 2, 2 * 2 * 128 * 32 * 4, 2.f, 1.5f, 1.f, 1.5f};
  // model constants in units of one iteration, fitted to the fp16 shape
  // sweep on MI355X: a 256 x 256 fp32 partial (256 KiB) costs about five
  // 64-deep iterations to write and four to read and add when every
  // workgroup exchanges one at the same time
  const float it = SK_HGEMM_BK / 64.f;
  return TileCfg{256, 256, SK_HGEMM_BK, 64 * SK_HGEMM_WAVES, 1, SK_HGEMM_STAGES * 2 * 256 * SK_HGEMM_BK * 2,
                 4.f / it, 5.f / it, 1.f, 4.f / it};
}

// Resolved work decomposition (integers only).
struct Plan {
  int64_t m, n, k;
  int dtype, layout;
  TileCfg cfg;
  int slots;            // p
  int grid;             // g
  int schedule;         // resolved sk_schedule
  int64_t tiles_m, tiles_n, tiles, ipt, total;
  int64_t sk_tiles;     // Stream-K region: tiles [0, sk_tiles)
  int64_t sk_q, sk_r;   // even split of sk_tiles*ipt over g: first sk_r get sk_q+1
  int64_t dp_tiles;     // tiles [sk_tiles, tiles), round-robin over g
  int w, r;             // full waves and leftover tiles
  int max_peers;        // filled by plan_max_peers (inspection only)
  bool pack_a, pack_b;  // operand repacked to k-contiguous before the GEMM
};

// Fills `plan` (except max_peers); returns SK_OK or an sk_status.  slots > 0.
int make_plan(const sk_gemm_desc &d, const sk_options &o, int slots, Plan &plan);
// Most partials any owner adds under `plan` (O(tiles); for inspection).
int plan_max_peers(const Plan &plan);

// First Stream-K iteration of workgroup x (x == grid gives the region's end).
inline int64_t sk_first_iter(int64_t q, int64_t r, int64_t x) { return x * q + (x < r ? x : r); }
// Workgroup whose Stream-K range holds iteration `it`.
inline int64_t sk_owner_of(int64_t q, int64_t r, int64_t it) {
  int64_t big = r * (q + 1);
  return it < big ? it / (q + 1) : r + (it - big) / q;
}

// Does the kernel read this operand directly (true), or from a repacked
// k-contiguous copy (false)?  `kmajor` = operand contiguous along k.
bool operand_direct(int dtype, bool kmajor, const void *ptr, int64_t ld, int64_t k);

// Arguments of the GEMM kernels (passed by value).
struct KernelArgs {
  const void *A;       // A operand (maybe a repacked copy)
  const void *B;
  void *C;
  int64_t lda, ldb, ldc;
  int32_t m, n, k;
  int32_t a_kmajor, b_kmajor;  // operand contiguous along k
  // k extent of a k-major operand's rows that may be read (k itself, or the
  // zero-padded row length of a repacked copy); bounds the buffer range so
  // that the hardware range check never cuts a valid element off
  int32_t a_kext, b_kext;
  float alpha, beta;
  int32_t tiles_m, tiles_n, tiles, ipt;
  int32_t grid, sk_tiles;
  int64_t sk_q, sk_r;
  float *partials;     // grid slots of BM*BN floats
  uint32_t *flags;     // grid flags
  uint32_t epoch;
  int32_t *status;     // device error word (bit 0: fixup time-out)
  int64_t spin_limit;  // time-out in ticks of the 100 MHz real-time counter
  // ABFT (fp32 only)
  int32_t abft;
  int32_t n_faults;
  const sk_fault *faults;
  sk_abft_report *report;
  float abft_tau;
};

// Kernel launchers (sk_kernels.hip).  Return a hipError_t value.
int launch_gemm(const Plan &plan, const KernelArgs &args, hipStream_t stream);
int launch_scale(int dtype, int64_t m, int64_t n, float beta, void *C, int64_t ldc,
                 hipStream_t stream);
// Copies a rows x k operand (rows = m for A, n for B) into dst[rows][ldd],
// k-contiguous, zero-filling columns k..ldd-1.  src element (r, l) is
// src[r*lds + l] when src_kmajor, else src[l*lds + r].
int launch_pack(int dtype, const void *src, int64_t lds, bool src_kmajor, int64_t rows,
                int64_t k, void *dst, int64_t ldd, hipStream_t stream);
int launch_zero_report(sk_abft_report *report, hipStream_t stream);
// Occupancy query for the GEMM kernel of `dtype` (fp32: with or without ABFT).
int kernel_occupancy(int dtype, bool abft, int *blocks_per_cu);

}  // namespace sk
