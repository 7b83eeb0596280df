// sk_internal.h -- definitions shared by the library's host code (planner,
// C ABI) and its HIP kernels.  Not part of the public interface.
#pragma once

#include <stdint.h>

#include <algorithm>

#include "../../include/sk_gemm.h"

namespace sk {

// Tile shape and launch shape of each kernel instance.
//   HGEMM (fp16/bf16): 256 x 256 x 64 tiles, 512 threads (8 wave64s laid out
//   2 x 4, two per SIMD, each owning a 128 x 64 block of C), two LDS stages
//   of 64 KiB, one workgroup per CU.
//   SGEMM (fp32): 128 x 128 x 32 tiles, 256 threads (4 wave64s, 2 x 2, each
//   64 x 64), two LDS stages of 32 KiB, two workgroups per CU; and 64 x 64 x
//   32 tiles (32 x 32 per wave, stages of 16 KiB, four workgroups per CU).
struct TileCfg {
  int bm, bn, bk;
  int threads;
  int occupancy;     // workgroups per CU
  int lds_bytes;     // dynamic LDS per workgroup
  // default grid-size model constants, in units of one MAC iteration
  float a, b, c, d;
  int inst;          // tile instance: fp16/bf16 0: 256 x 256, 1: 128 x 128,
                     // 2-5: narrow-m, 64/128/192/256 x 256; fp32 0: 128 x 128,
                     // 1: 64 x 64
  // the tile-instance choice, microseconds (least-squares fit, relative
  // error, to the fp16 shape sweep timed on each instance): fixed cost of a
  // launch (start, first loads, epilogue), one level of partial exchange,
  // and one iteration of the busiest workgroup, which depends on how busy
  // the chip is: with one workgroup per CU, iter_a + iter_b * grid / slots
  // (a partly idle chip runs at a higher clock); with two, iter_a while
  // every workgroup has a CU to itself and iter_b once two share one
  float fixed_us, level_us, iter_a_us, iter_b_us;
  // the grid-size model's iteration cost when every one of the
  // `occupancy` workgroup slots of each CU is busy, in units of c (a
  // workgroup alone on its CU: 1), interpolated linearly in between
  float c_shared = 1.f;
};

// Tile instances.  fp32: instance 0, 128 x 128 x 32, 4 waves, two
// workgroups per CU; instance 1, 64 x 64 x 32, 4 waves, four per CU, for
// shapes with few 128 x 128 tiles.  fp16/bf16: instance 0, 256 x 256 x 64 with 8 waves and one workgroup per
// CU; instance 1, 128 x 128 x 64 with 4 waves and two per CU, for shapes
// with few large tiles.  Model constants in units of one MAC iteration of
// the instance.
inline TileCfg tile_cfg(int dtype, int inst = 0) {
  // narrow-m fp16/bf16 (m up to 256): BM = 64 (inst - 1) rows by 256
  // columns, 8 waves, one workgroup per CU, four A stages of BM x 64 in LDS;
  // a BM x 256 fp32 partial against one iteration's 32 KiB of B
  if (dtype != SK_F32 && inst >= 2 && inst <= 5) {
    const int bm = 64 * (inst - 1);
    return TileCfg{bm, 256, 64, 512, 1, 4 * bm * 128, 4.f, 4.f * bm / 256, 1.f, 4.f * bm / 256, inst,
                   13.8f, 8.45f, 0.745f, 1.153f};
  }
  // fp32 constants measured on MI355X (1024-4096 cubes and one-wave
  // data-parallel and split grids, fp32 row-major): 64 x 64 x 32, 4 waves,
  // four workgroups per CU -- 0.68 us per iteration alone on a CU, 2.08 with
  // four per CU (3.06 times), 2 us per exchange of a 16 KiB partial (three
  // iterations), 5.5 us fixed
  if (dtype == SK_F32 && inst == 1)
    return TileCfg{64, 64, 32, 256, 4, 2 * 2 * 64 * 32 * 4, 8.f, 1.5f, 1.f, 1.5f, 1, 5.5f, 2.f, 0.68f, 2.08f, 3.06f};
  // 128 x 128 x 32, two workgroups per CU -- 2.08 us per iteration alone,
  // 3.79 with two per CU (1.82 times), 5 us per exchange of a 64 KiB
  // partial (two and a half iterations), 12 us fixed
  if (dtype == SK_F32) return TileCfg{128, 128, 32, 256, 2, 2 * 2 * 128 * 32 * 4, 6.f, 1.2f, 1.f, 1.2f, 0, 12.f, 5.f, 2.08f, 3.79f, 1.82f};
  // 128 x 128 fp16: a 64 KiB partial against a quarter of the large tile's
  // iteration work
  if (inst == 1) return TileCfg{128, 128, 64, 256, 2, 2 * 2 * 128 * 64 * 2, 4.f, 5.f, 1.f, 4.f, 1, 9.16f, 3.39f, 0.413f, 1.2f};
  // model constants fitted to the fp16 shape sweep on MI355X: a 256 x 256
  // fp32 partial (256 KiB) costs about five 64-deep iterations to write and
  // four to read and add when every workgroup exchanges one at the same time
  return TileCfg{256, 256, 64, 512, 1, 2 * 2 * 256 * 64 * 2, 4.f, 5.f, 1.f, 4.f, 0, 13.8f, 8.45f, 0.745f, 1.153f};
}

// How the kernels walk the work (shared by the kernels and the host's
// segment listing, so both enumerate exactly the same segments).
//
// Tiles are visited in "region order" u = 0 .. tiles-1: the Stream-K region
// is u < sk_tiles, the data-parallel tiles follow.  With group_rows == 0,
// region order is the linear m -> n order and data-parallel tile j of
// workgroup x is u = sk_tiles + x + j * grid (the page's layout).
//
// With group_rows = G > 0 (the XCD-aware schedule), u is mapped to tiles in
// bands of G tile rows, column by column within a band, and
//  * the data-parallel tiles go in waves of `grid`; a wave's R tiles are cut
//    into 8 runs of consecutive u (lengths R / 8 or R / 8 + 1) and run c goes to the
//    workgroups the dispatcher places on XCD c (x mod 8 = c, in order of
//    x / 8): each XCD works on a compact block of tiles sharing A rows and B
//    columns, and a partial last wave still spreads over all eight XCDs;
//  * the Stream-K region is split in quanta of ipt / D iterations
//    (D = phase_div, a multiple of 8): workgroup x covers
//    [floor(x s ipt / D), floor((x+1) s ipt / D)) of the region's
//    iterations, cut at sk_tiles * ipt.  Workgroups with equal x mod D then
//    work at the same k offset at the same time, and the region's tile index
//    L is mapped so that those workgroups also work on neighbouring tiles:
//    L = j s + v (v < s) is tile u = prefix(v) + j, where block v holds the
//    block_len (or block_len - 1 for v >= block_cut) tiles L = v, v + s, ....
// All fields and every value the helpers below form (products included)
// are below 2^31: the planner only hands such plans to the kernels
// (sched_fits), so the device walks the schedule in 32-bit arithmetic; a
// 64-bit division would expand to a long dependent instruction chain at
// every segment.
struct Sched {
  int32_t ipt, tiles, tiles_m, tiles_n;
  int32_t sk_tiles;
  int32_t sk_q, sk_r;   // even split (group_rows == 0): the first sk_r get sk_q + 1
  int32_t grid;
  int32_t phase_div;    // D (XCD-aware schedule with a Stream-K region), else 0
  int32_t blocks;       // s: quanta per workgroup
  int32_t block_len;    // J = ceil(sk_tiles / s)
  int32_t block_cut;    // sk_tiles - (J - 1) * s
  int32_t group_rows;   // G, 0 for the page's linear order
  int32_t tree;         // 1: the partials of a split tile are combined in a binary tree
};

#define SK_HD __host__ __device__ __forceinline__

SK_HD int32_t sched_min(int32_t a, int32_t b) { return a < b ? a : b; }

// Quotient of non-negative a and positive b.
SK_HD int32_t sched_div(int32_t a, int32_t b) { return (int32_t)((uint32_t)a / (uint32_t)b); }

// Tile (linear m -> n index) of region-order position u.
SK_HD int32_t sched_tile_of_u(const Sched &S, int32_t u) {
  if (S.group_rows <= 0) return u;
  const int32_t band = S.group_rows * S.tiles_n;
  const int32_t b = sched_div(u, band), rem = u - b * band;
  const int32_t rows = sched_min(S.group_rows, S.tiles_m - b * S.group_rows);
  const int32_t col = sched_div(rem, rows);
  return (b * S.group_rows + rem - col * rows) * S.tiles_n + col;
}

// Tile of Stream-K region position L.
SK_HD int32_t sched_sk_tile(const Sched &S, int32_t L) {
  if (S.phase_div <= 0) return sched_tile_of_u(S, L);
  const int32_t j = sched_div(L, S.blocks), v = L - j * S.blocks;
  const int32_t over = v - S.block_cut;
  return sched_tile_of_u(S, v * S.block_len - (over > 0 ? over : 0) + j);
}

// First Stream-K iteration of workgroup x (x == grid gives the region's end).
SK_HD int32_t sched_first_iter(const Sched &S, int32_t x) {
  if (S.phase_div > 0) return sched_min(sched_div(x * S.blocks * S.ipt, S.phase_div), S.sk_tiles * S.ipt);
  return x * S.sk_q + (x < S.sk_r ? x : S.sk_r);
}

// Workgroup whose Stream-K range holds iteration `it`.
SK_HD int32_t sched_owner_of(const Sched &S, int32_t it) {
  if (S.phase_div > 0) return sched_div((it + 1) * S.phase_div - 1, S.blocks * S.ipt);
  const int32_t big = S.sk_r * (S.sk_q + 1);
  return it < big ? sched_div(it, S.sk_q + 1) : S.sk_r + sched_div(it - big, S.sk_q);
}

// Segments of workgroup x in execution order: its Stream-K range (Algorithm
// 5: a workgroup that holds a tile's k = 0 iteration but not its last one
// adds the partials of workgroups x+1 .. last_peer), then its data-parallel
// tiles.  The iterator keeps four integers of state, so that a kernel that
// runs a whole MAC loop per segment keeps little alive across it (the
// kernels call next() from a single site).
struct SegIter {
  int32_t it, end;  // remaining Stream-K range
  int32_t d;        // next data-parallel index (XCD-aware order: wave)
  int32_t x;        // the workgroup
};
// first / last: the workgroups holding the tile's first and last iteration,
// -1 where that is x itself.
struct Segment {
  int32_t tile, lb, le, last_peer, first, last;
  bool started, ended;
};

SK_HD SegIter sched_begin(const Sched &S, int32_t x) {
  SegIter I;
  I.it = S.sk_tiles > 0 ? sched_first_iter(S, x) : 0;
  I.end = S.sk_tiles > 0 ? sched_first_iter(S, x + 1) : 0;
  I.d = 0;  // XCD-aware order: data-parallel wave index; else the next index
  if (!(S.group_rows > 0 && S.grid % 8 == 0)) I.d = x;
  I.x = x;
  return I;
}

// Data-parallel tile u (region order) of wave `wave` for workgroup x in the
// XCD-aware order, or -1: the wave's R tiles are cut into 8 runs of
// consecutive tiles whose lengths differ by at most one, run c going to the
// workgroups of XCD c.
SK_HD int32_t sched_dp_xcd(const Sched &S, int32_t wave, int32_t x) {
  const int32_t dp = S.tiles - S.sk_tiles;
  const int32_t base = wave * S.grid;
  if (base >= dp) return -1;
  const int32_t R = sched_min(S.grid, dp - base);
  const int32_t q = R >> 3, e = R & 7;
  const int32_t c = x & 7, pos = x >> 3;
  if (pos >= q + (c < e)) return -1;
  return S.sk_tiles + base + c * q + sched_min(c, e) + pos;
}

SK_HD bool sched_next(const Sched &S, SegIter &I, Segment &g) {
  if (I.it < I.end) {
    const int32_t L = sched_div(I.it, S.ipt), ts = L * S.ipt, te = ts + S.ipt;
    g.lb = I.it - ts;
    g.le = (I.end < te ? I.end : te) - ts;
    g.started = g.lb == 0;
    g.ended = I.end >= te;
    g.first = g.started ? -1 : sched_owner_of(S, ts);
    g.last = g.ended ? -1 : sched_owner_of(S, te - 1);
    g.last_peer = (g.started && !g.ended) ? g.last : -1;
    g.tile = sched_sk_tile(S, L);
    I.it = te;
    return true;
  }
  int32_t u = -1;
  if (S.group_rows > 0 && S.grid % 8 == 0) {
    // full waves give every workgroup a tile; only the last wave can leave
    // one without, and nothing follows it
    const int32_t waves = sched_div(S.tiles - S.sk_tiles + S.grid - 1, S.grid);
    while (u < 0 && I.d < waves) u = sched_dp_xcd(S, I.d++, I.x);
  } else if (I.d < S.tiles - S.sk_tiles) {
    u = S.sk_tiles + I.d;
    I.d += S.grid;
  }
  if (u >= 0) {
    g.tile = sched_tile_of_u(S, u);
    g.lb = 0;
    g.le = S.ipt;
    g.started = g.ended = true;
    g.last_peer = g.first = g.last = -1;
    return true;
  }
  return false;
}

// Calls f(tile, lb, le, started, ended, last_peer) for each segment of
// workgroup x (host-side listing).
template <class F>
SK_HD void sched_segments(const Sched &S, int32_t x, F &&f) {
  SegIter I = sched_begin(S, x);
  Segment g;
  while (sched_next(S, I, g)) f(g.tile, g.lb, g.le, g.started, g.ended, g.last_peer);
}

// Fills the fields of S that follow from the others (block_len, block_cut).
inline void sched_derive(Sched &S) {
  if (S.phase_div > 0 && S.blocks > 0) {
    S.block_len = (S.sk_tiles + S.blocks - 1) / S.blocks;
    S.block_cut = S.sk_tiles - (S.block_len - 1) * S.blocks;
  }
}

// Do all of a plan's schedule values, and the products the helpers form
// from them (tile positions up to tiles + grid, x s ipt up to x = grid,
// (it + 1) D, sk_r (sk_q + 1)), stay below 2^31?
inline bool sched_fits(int64_t tiles, int64_t tiles_m, int64_t tiles_n, int64_t ipt, int64_t grid,
                       int64_t sk_tiles, int64_t phase_div, int64_t blocks) {
  const int64_t lim = (int64_t)1 << 31;
  if (tiles_m >= lim || tiles_n >= lim || ipt >= lim) return false;
  const int64_t D = phase_div > 0 ? phase_div : 1;
  const int64_t big = std::max({tiles + grid, (sk_tiles * ipt + 1) * D, (grid + 1) * blocks * ipt,
                                sk_tiles * ipt + grid, (int64_t)8 * tiles_n});
  return big < lim;
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
  int64_t sk_tiles;     // Stream-K region: tiles [0, sk_tiles) of region order
  int64_t sk_q, sk_r;   // even split of sk_tiles*ipt over g: first sk_r get sk_q+1
  int64_t dp_tiles;     // the remaining tiles, dealt over g
  int w, r;             // full waves and leftover tiles
  int phase_div, blocks, group_rows;  // XCD-aware schedule (see Sched)
  int max_peers;        // filled by plan_max_peers (inspection only)
  bool pack_a, pack_b;  // operand repacked to k-contiguous before the GEMM
  Sched sched() const {
    Sched S{};
    S.ipt = (int32_t)ipt; S.tiles = (int32_t)tiles; S.tiles_m = (int32_t)tiles_m; S.tiles_n = (int32_t)tiles_n;
    S.sk_tiles = (int32_t)sk_tiles; S.sk_q = (int32_t)sk_q; S.sk_r = (int32_t)sk_r; S.grid = grid;
    S.phase_div = phase_div; S.blocks = blocks; S.group_rows = group_rows;
    S.tree = phase_div > 0 ? 1 : 0;
    sched_derive(S);
    return S;
  }
};

// Matrix-vector path (SK_SCHED_GEMV_SPLIT), in one of three forms:
//  kGemvDot: out[r * ldo] = alpha * (M row r) . v + beta * out[r * ldo] for
//    r < R, M rows of K elements (k-contiguous, stride ldm), v contiguous;
//    each row split in S chunks of `chunk` elements;
//  kGemvAxpy: out[j * ldo] = alpha * sum_r v[r * incv] M[r, j] +
//    beta * out[j * ldo] for j < R, M rows of R elements (contiguous along
//    the output, stride ldm), r < K; the output is cut in blocks of one
//    wave's width and the K rows in S chunks of `chunk` rows;
//  kGemvMulti: V (2 .. 16 for fp32, 2 .. 8 for fp16/bf16) vectors, rows of v
//    with stride ldv, against the R k-contiguous rows of M:
//    out[i * ld_v + r * ld_r] = alpha * (v row i) . (M row r) + beta * (the
//    same) for i < V, r < R; tasks are blocks of 64 (fp32) or 16 rows times
//    S chunks of `chunk` k.
// `grid` workgroups of 256 threads.
enum { kGemvDot = 0, kGemvAxpy = 1, kGemvMulti = 2 };
struct GemvPlan {
  const void *M, *v;
  void *out;
  int64_t ldm, ldo, incv, R, K, chunk, S;
  int64_t ldv, ld_v, ld_r;  // kGemvMulti
  int V;                    // kGemvMulti
  int form;
  int grid;
};
// Fills `g` and returns true if the call is a matrix-vector product the
// path takes: m == 1 or n == 1 (dot form: the matrix operand k-contiguous
// with 16-byte aligned base and rows, the vector contiguous and 16-byte
// aligned; axpy form, when the matrix operand is contiguous along the
// output instead: 16-byte aligned base and rows, any vector stride), or
// 2 <= m or n <= 16 (fp16/bf16: 8), neither 1, with both operands
// k-contiguous and 16-byte aligned (multi form); cus: compute units.
bool gemv_plan(const sk_gemm_desc &d, int cus, GemvPlan &g);
int launch_gemv(int dtype, const GemvPlan &g, float *part, float alpha, float beta, hipStream_t stream);

// Fills `plan` (except max_peers); returns SK_OK or an sk_status.  slots:
// resident workgroups of the large (or fp32) and of the small-tile instance.
// The narrow-m instance for m rows (m <= 256): the smallest BM that holds m.
inline int narrow_inst(int64_t m) { return m <= 64 ? 2 : m <= 128 ? 3 : m <= 192 ? 4 : 5; }
// slots: resident workgroups of the large, small and narrow-m instances
int make_plan(const sk_gemm_desc &d, const sk_options &o, const int slots[3], Plan &plan);
// The runtime model's predicted time of a plan, in microseconds.
double plan_cost_us(const Plan &plan);
// Most partials any owner adds under `plan` (O(tiles); for inspection).
int plan_max_peers(const Plan &plan);

// Does the kernel read this operand directly (true), or from a repacked
// k-contiguous copy (false)?  `kmajor` = operand contiguous along k; `mn` =
// its extent along m (A) or n (B); `mn_ok` = the instance has a 16-bit
// m- or n-contiguous read for it (the 256 and 128 HGEMM instances).
bool operand_direct(int dtype, bool kmajor, const void *ptr, int64_t ld, int64_t k, int64_t mn, bool mn_ok);

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
  Sched sched;
  float *partials;     // grid slots of BM*BN floats
  uint32_t *flags;     // grid flags
  uint32_t epoch;
  int32_t *status;     // error word (bit 0: fixup time-out): mapped host memory, or device memory
  int64_t spin_limit;  // time-out in ticks of the 100 MHz real-time counter
  int32_t no_signal;   // testing: producers store partials without signalling them
  // ABFT (fp32 only)
  int32_t abft;
  int32_t n_faults;
  const sk_fault *faults;
  sk_abft_report *report;
  float abft_tau;
  // ABFT encodings (abft_prep_kernel): per 128-row tile of A and 128-column
  // tile of B and per k-iteration of 32, the 32 sums
  const float *enc_a, *enc_b;
  int32_t enc_kb;      // k-iterations per tile in the encoding arrays
  // detection-threshold inputs: per row of A and column of B the sum of |x|
  // over all of k; per tile the largest column (row) sum of |x| over k
  const float *norm_a, *norm_b, *emax_a, *emax_b;
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
// ABFT preparation of an fp32 GEMM, in one launch over both operands.  For
// operand X of `rows` rows (m for A, n for B) and k columns, element (r, l)
// at X[r*ld + l] when kmajor, else X[l*ld + r]:
//   enc[(tile*kb + l/32)*32 + l%32]  the sum of the 128-row tile's rows at
//                                    k = l < 32*kb (rows past `rows` left
//                                    out, l >= k zero);
//   norm[r]    sum over k of |X(r, k)|;
//   emax[tile] max over k of the tile's sum of |X(r, k)| over its rows;
// k is cut into chunks of 64 (chunks = ceil(32*kb / 64)) and the chunks
// into `groups` groups of group_chunks, one workgroup per (tile, group);
// scratch arrays rowabs (groups * rows) and tmax (tiles * groups).  The last
// workgroup of a tile to finish reduces the tile's norms and emax (counters:
// one per tile of A, then of B, zero before the call and left zero after
// it).  The first workgroup zeroes the report (if not null).
struct AbftPrepOperand {
  const float *X;
  int64_t ld;
  int32_t kmajor;
  int64_t rows, tiles;
  float *enc, *rowabs, *tmax, *norm, *emax;
};
struct AbftPrepArgs {
  AbftPrepOperand op[2];  // A, B
  int64_t k, kb, chunks, group_chunks, groups;
  uint32_t *counters;     // tiles of A + tiles of B
  sk_abft_report *report;
};
int launch_abft_prep(const AbftPrepArgs &args, hipStream_t stream);
// Occupancy query for the GEMM kernel of `dtype` (fp32: with or without ABFT).
int kernel_occupancy(int dtype, bool abft, int inst, int *blocks_per_cu);

}  // namespace sk
