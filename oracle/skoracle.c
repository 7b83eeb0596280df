/*
 * skoracle.c -- CPU oracle for the Stream-K GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the GPU library and must never be reached
 * from the product path.
 *
 * What it computes, and where each part is defined:
 *
 *  - or_gemm: C_out = alpha*A*B + beta*C_in (GEMM definition in the Stream-K
 *    page, section 3 "background") evaluated with the sequential cache-blocked
 *    six-loop structure of that page's Algorithm 1 (section 3.1): output tiles
 *    of BLK_M x BLK_N are zeroed, then the MAC loop walks k in steps of BLK_K,
 *    k ascending.  Inputs are decoded exactly to fp64, accumulation is fp64,
 *    alpha/beta are applied in fp64, and the result is rounded once to the
 *    output type with IEEE round-to-nearest-even.  C_in is not read when
 *    beta == 0.  The componentwise bound D = |alpha| |A||B| + |beta| |C_in|
 *    is produced in the same pass (used as the error denominator).
 *
 *  - or_sk_plan / or_sk_execute: the work decompositions of the Stream-K page:
 *    data-parallel (Algorithm 2), fixed-split (Algorithm 4), basic Stream-K
 *    (Algorithm 5) and the two hybrids of section 5.2 ("DP + one-tile SK" and
 *    "two-tile SK + DP"), executed by simulated workgroups on the CPU with
 *    partials and flags in host arrays and a seeded interleaving in which a
 *    wait is a yield until the flag is set.
 *
 *  - or_abft_check: one verification domain of threadblock-level ABFT from the
 *    fault-tolerant GEMM page (section on thread-level ABFT, Fig. 3; and the
 *    threadblock-level scheme, Figs. 5-7): row and column checksums of the
 *    block, verify, locate at the intersection of the mismatching row and
 *    column, correct from the row checksum.
 *
 *  - or_freivalds: randomised product check (Freivalds' algorithm), a textbook
 *    identity, used for shapes too large for or_gemm.
 *
 * Readings of the pages that this file relies on are listed next to the code
 * that takes them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Oracle's own codes (kept numerically equal to the public ABI's so that the
 * tests can pass one value to both; no header is shared). */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_A_ROW_B_ROW = 0, OR_A_ROW_B_COL = 1, OR_A_COL_B_ROW = 2, OR_A_COL_B_COL = 3 };

/* ------------------------------------------------------------------------ */
/* Exact decode of the storage formats to fp64 (IEEE 754 binary16, bfloat16 */
/* = the top half of binary32, binary32).                                   */
/* ------------------------------------------------------------------------ */

double or_decode_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(f | 1024), e - 25); /* (1024 + f) * 2^(e-15-10) */
  return s ? -v : v;
}

double or_decode_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static inline double dec(int dt, const void *p, int64_t idx) {
  if (dt == OR_F32) return (double)((const float *)p)[idx];
  if (dt == OR_F16) return or_decode_f16(((const uint16_t *)p)[idx]);
  return or_decode_bf16(((const uint16_t *)p)[idx]);
}

/* ------------------------------------------------------------------------ */
/* Round-to-nearest-even from fp64 straight to the target format (one       */
/* rounding; no detour through fp32).  nearbyint() uses the default         */
/* rounding mode, which is to-nearest, ties-to-even.                        */
/* ------------------------------------------------------------------------ */

uint16_t or_round_f16(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return 0x7E00;
  double a = fabs(x);
  if (isinf(a)) return sign | 0x7C00;
  if (a < ldexp(1.0, -14)) { /* subnormal range, quantum 2^-24 */
    double r = nearbyint(ldexp(a, 24));
    return sign | (uint16_t)r; /* r == 1024 is the smallest normal */
  }
  int e;
  (void)frexp(a, &e);           /* a in [2^(e-1), 2^e) */
  int E = e - 1;                /* unbiased exponent   */
  double r = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
  if (r == 2048.0) { r = 1024.0; E += 1; }
  if (E > 15) return sign | 0x7C00;
  return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)r - 1024);
}

uint16_t or_round_bf16(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return 0x7FC0;
  double a = fabs(x);
  if (isinf(a)) return sign | 0x7F80;
  if (a < ldexp(1.0, -126)) { /* subnormal range, quantum 2^-133 */
    double r = nearbyint(ldexp(a, 133));
    return sign | (uint16_t)r;
  }
  int e;
  (void)frexp(a, &e);
  int E = e - 1;
  double r = nearbyint(ldexp(a, 7 - E)); /* in [128, 256] */
  if (r == 256.0) { r = 128.0; E += 1; }
  if (E > 127) return sign | 0x7F80;
  return sign | (uint16_t)((E + 127) << 7) | (uint16_t)((int)r - 128);
}

static void store_rounded(int dt, void *out, int64_t idx, double v) {
  if (dt == OR_F32)
    ((float *)out)[idx] = (float)v; /* C conversion: round to nearest even */
  else if (dt == OR_F16)
    ((uint16_t *)out)[idx] = or_round_f16(v);
  else
    ((uint16_t *)out)[idx] = or_round_bf16(v);
}

/* Element addressing for the four storage orders.  A is m x k, B is k x n;
 * "row" means the second index is contiguous. */
static inline int a_row_major(int layout) { return layout == OR_A_ROW_B_ROW || layout == OR_A_ROW_B_COL; }
static inline int b_row_major(int layout) { return layout == OR_A_ROW_B_ROW || layout == OR_A_COL_B_ROW; }
static inline int64_t a_idx(int layout, int64_t i, int64_t l, int64_t lda) {
  return a_row_major(layout) ? i * lda + l : l * lda + i;
}
static inline int64_t b_idx(int layout, int64_t l, int64_t j, int64_t ldb) {
  return b_row_major(layout) ? l * ldb + j : j * ldb + l;
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
  return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

int or_num_threads(void) { return set_threads(0); }

/* ------------------------------------------------------------------------ */
/* Six-loop blocked GEMM (Algorithm 1), fp64.                               */
/* ------------------------------------------------------------------------ */
/*
 * out64, bound : m x n, row stride n (may be NULL)
 * out_round    : m x n in the storage type, row stride n (may be NULL)
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int or_gemm(int64_t m, int64_t n, int64_t k, double alpha, const void *A, int64_t lda,
            const void *B, int64_t ldb, double beta, const void *Cin, int64_t ldc, int dtype,
            int layout, int64_t blk_m, int64_t blk_n, int64_t blk_k, double *out64, double *bound,
            void *out_round, int nthreads) {
  if (m < 0 || n < 0 || k < 0 || blk_m <= 0 || blk_n <= 0 || blk_k <= 0) return -1;
  if (m == 0 || n == 0) return 0;
  /* Decode once: Ad is m x k (row i contiguous in l), Bd is n x k (column j
   * of B contiguous in l).  This is a storage choice; the arithmetic below is
   * exactly Algorithm 1's. */
  double *Ad = (double *)malloc(sizeof(double) * (size_t)(m * (k ? k : 1)));
  double *Bd = (double *)malloc(sizeof(double) * (size_t)(n * (k ? k : 1)));
  if (!Ad || !Bd) { free(Ad); free(Bd); return -1; }
  for (int64_t i = 0; i < m; ++i)
    for (int64_t l = 0; l < k; ++l) Ad[i * k + l] = dec(dtype, A, a_idx(layout, i, l, lda));
  for (int64_t j = 0; j < n; ++j)
    for (int64_t l = 0; l < k; ++l) Bd[j * k + l] = dec(dtype, B, b_idx(layout, l, j, ldb));

  const int64_t tiles_m = (m + blk_m - 1) / blk_m, tiles_n = (n + blk_n - 1) / blk_n;
  const int64_t ntiles = tiles_m * tiles_n;
  int fail = 0;
  int nt = set_threads(nthreads);
#pragma omp parallel num_threads(nt)
  {
    double *acc = (double *)malloc(sizeof(double) * (size_t)(blk_m * blk_n));
    double *acc_abs = (double *)malloc(sizeof(double) * (size_t)(blk_m * blk_n));
    if (!acc || !acc_abs) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < ntiles; ++t) {
      if (!acc || !acc_abs) continue;
      /* tile-processing outer loops (mm, nn) */
      const int64_t mm = (t / tiles_n) * blk_m, nn = (t % tiles_n) * blk_n;
      const int64_t me = mm + blk_m < m ? mm + blk_m : m;
      const int64_t ne = nn + blk_n < n ? nn + blk_n : n;
      /* zero-initialise the output tile */
      for (int64_t x = 0; x < blk_m * blk_n; ++x) { acc[x] = 0.0; acc_abs[x] = 0.0; }
      /* MAC iterations for this tile, k ascending */
      for (int64_t kk = 0; kk < k; kk += blk_k) {
        const int64_t ke = kk + blk_k < k ? kk + blk_k : k;
        for (int64_t i = mm; i < me; ++i)
          for (int64_t j = nn; j < ne; ++j) {
            double s = acc[(i - mm) * blk_n + (j - nn)];
            double sa = acc_abs[(i - mm) * blk_n + (j - nn)];
            const double *ar = Ad + i * k, *bc = Bd + j * k;
            for (int64_t l = kk; l < ke; ++l) {
              s += ar[l] * bc[l];
              sa += fabs(ar[l]) * fabs(bc[l]);
            }
            acc[(i - mm) * blk_n + (j - nn)] = s;
            acc_abs[(i - mm) * blk_n + (j - nn)] = sa;
          }
      }
      /* scale and store */
      for (int64_t i = mm; i < me; ++i)
        for (int64_t j = nn; j < ne; ++j) {
          double ab = acc[(i - mm) * blk_n + (j - nn)];
          double v = alpha * ab, d = fabs(alpha) * acc_abs[(i - mm) * blk_n + (j - nn)];
          if (beta != 0.0) {
            double c = dec(dtype, Cin, i * ldc + j);
            v += beta * c;
            d += fabs(beta) * fabs(c);
          }
          if (out64) out64[i * n + j] = v;
          if (bound) bound[i * n + j] = d;
          if (out_round) store_rounded(dtype, out_round, i * n + j, v);
        }
    }
    free(acc);
    free(acc_abs);
  }
  free(Ad);
  free(Bd);
  return fail ? -1 : 0;
}

/* Selected entries of the same product, one plain dot product each, k
 * ascending (for sizes where the full oracle is too slow). */
int or_gemm_entries(int64_t m, int64_t n, int64_t k, double alpha, const void *A, int64_t lda,
                    const void *B, int64_t ldb, double beta, const void *Cin, int64_t ldc,
                    int dtype, int layout, int64_t n_e, const int64_t *rows, const int64_t *cols,
                    double *out64, double *bound, int nthreads) {
  int bad = 0;
  int nt = set_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 16)
  for (int64_t e = 0; e < n_e; ++e) {
    int64_t i = rows[e], j = cols[e];
    if (i < 0 || i >= m || j < 0 || j >= n) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    double s = 0.0, sa = 0.0;
    for (int64_t l = 0; l < k; ++l) {
      double a = dec(dtype, A, a_idx(layout, i, l, lda));
      double b = dec(dtype, B, b_idx(layout, l, j, ldb));
      s += a * b;
      sa += fabs(a) * fabs(b);
    }
    double v = alpha * s, d = fabs(alpha) * sa;
    if (beta != 0.0) {
      double c = dec(dtype, Cin, i * ldc + j);
      v += beta * c;
      d += fabs(beta) * fabs(c);
    }
    out64[e] = v;
    if (bound) bound[e] = d;
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Work decompositions of the Stream-K page, as segment lists per CTA.      */
/* ------------------------------------------------------------------------ */
/*
 * Modes:
 *   OR_DP         Algorithm 2: one CTA per output tile (g = t).
 *   OR_FIXED      Algorithm 4: s CTAs per tile; CTA (x, y) does iterations
 *                 [y*ceil(ipt/s), min(ipt, (y+1)*ceil(ipt/s))); y != 0 stores
 *                 a partial, y == 0 sums peers 1..s-1 (reading: the printed
 *                 loop bound "1 to s" covers the s-1 peers).  CTA id = x*s + y.
 *   OR_SK         Algorithm 5 over all tiles with a grid of g CTAs.  Each
 *                 CTA gets a contiguous range of the m -> n -> k iteration
 *                 space; the ranges differ in length by at most one
 *                 iteration: with q = floor(total/g) and rr = total mod g,
 *                 CTA x covers [x*q + min(x, rr), (x+1)*q + min(x+1, rr)).
 *                 Reading: the printed pseudo-code gives every CTA
 *                 ceil(total/g) iterations (leaving trailing CTAs short or
 *                 empty when g does not divide total), while the prose says
 *                 the split is even to within one iteration; the two agree
 *                 whenever g divides total (every worked example on the
 *                 page), and the prose is taken otherwise.  A CTA with an
 *                 empty range (g > total) does nothing.
 *   OR_HYBRID1    section 5.2 "DP + one-tile SK" on p CTAs: the r = t mod p
 *                 leftover tiles (the first r tiles) are split by Algorithm 5
 *                 over the p CTAs; the remaining w*p tiles run data-parallel.
 *   OR_HYBRID2    section 5.2 "two-tile SK + DP" on p CTAs: one full DP wave
 *                 is given back, so the first r + p tiles are split by
 *                 Algorithm 5 over the p CTAs (each gets between one and two
 *                 tiles of iterations) and the remaining (w-1)*p tiles run
 *                 data-parallel.  Requires w >= 1 and r > 0 (reading: the
 *                 mechanism "give back one wave" needs one full wave).
 *   OR_DP_PERSISTENT  p CTAs, CTA x takes tiles x, x+p, x+2p, ...
 * In the hybrids each CTA runs its Stream-K segments first and its DP tiles
 * after (reading: the page does not fix the order; results do not depend on
 * it).  DP tiles in the hybrids are dealt round-robin: CTA x takes
 * sk_tiles + x, sk_tiles + x + p, ...
 *
 * A segment record is 7 int64: cta, tile, local_begin, local_end, started,
 * ended, last_peer (the highest CTA id whose partial the owner must add; -1
 * when the segment needs no peers).  Records are listed CTA by CTA, each CTA's
 * segments in execution order.
 */
enum { OR_DP = 0, OR_FIXED = 1, OR_SK = 2, OR_HYBRID1 = 3, OR_HYBRID2 = 4, OR_DP_PERSISTENT = 5 };

typedef struct {
  int64_t cta, tile, lb, le, started, ended, last_peer;
} or_seg;

typedef struct {
  int64_t t, ipt, total;
  int64_t ncta;      /* CTAs launched */
  int64_t sk_tiles;  /* tiles handled by the Stream-K region (from tile 0) */
  int64_t sk_g;      /* CTAs sharing the Stream-K region */
  int64_t q, rr;     /* Stream-K region: floor(iters/g) and iters mod g */
  int64_t s, ips;    /* fixed-split factor and iterations per split */
  int64_t dp_first;  /* first data-parallel tile */
  int mode;
} or_decomp;

static int decompose(int64_t m, int64_t n, int64_t k, int64_t bm, int64_t bn, int64_t bk, int mode,
                     int64_t param, or_decomp *d) {
  if (m <= 0 || n <= 0 || k <= 0 || bm <= 0 || bn <= 0 || bk <= 0) return -1;
  memset(d, 0, sizeof(*d));
  d->mode = mode;
  d->t = ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
  d->ipt = (k + bk - 1) / bk;
  d->total = d->t * d->ipt;
  switch (mode) {
  case OR_DP:
    d->ncta = d->t; d->dp_first = 0; break;
  case OR_FIXED:
    if (param < 1) return -1;
    d->s = param; d->ips = (d->ipt + param - 1) / param; d->ncta = d->t * param; break;
  case OR_SK:
    if (param < 1) return -1;
    d->ncta = param; d->sk_tiles = d->t; d->sk_g = param;
    d->q = d->total / param; d->rr = d->total % param; d->dp_first = d->t; break;
  case OR_HYBRID1:
  case OR_HYBRID2: {
    if (param < 1) return -1;
    int64_t p = param, w = d->t / p, r = d->t % p;
    d->ncta = p;
    if (mode == OR_HYBRID1) d->sk_tiles = r;
    else {
      if (w < 1 || r == 0) return -2; /* not defined for this shape */
      d->sk_tiles = r + p;
    }
    d->sk_g = p;
    d->q = d->sk_tiles * d->ipt / p;
    d->rr = d->sk_tiles * d->ipt % p;
    d->dp_first = d->sk_tiles;
    break;
  }
  case OR_DP_PERSISTENT:
    if (param < 1) return -1;
    d->ncta = param; d->dp_first = 0; break;
  default:
    return -1;
  }
  return 0;
}

/* First Stream-K iteration of CTA x (x may be sk_g: the region's end). */
static int64_t cta_first_iter(const or_decomp *d, int64_t x) {
  return x * d->q + (x < d->rr ? x : d->rr);
}

/* The CTA whose Stream-K range holds iteration `it`. */
static int64_t cta_of_iter(const or_decomp *d, int64_t it) {
  int64_t big = d->rr * (d->q + 1); /* iterations held by the longer ranges */
  if (it < big) return it / (d->q + 1);
  return d->rr + (it - big) / d->q;
}

/* Segments of CTA x; returns the count written (<= cap) or -1. */
static int64_t cta_segments(const or_decomp *d, int64_t x, or_seg *out, int64_t cap) {
  int64_t c = 0;
#define PUSH(T, LB, LE, ST, EN, LP)                                                 \
  do {                                                                              \
    if (c >= cap) return -1;                                                        \
    out[c].cta = x; out[c].tile = (T); out[c].lb = (LB); out[c].le = (LE);          \
    out[c].started = (ST); out[c].ended = (EN); out[c].last_peer = (LP); ++c;       \
  } while (0)
  if (d->mode == OR_DP) {
    PUSH(x, 0, d->ipt, 1, 1, -1);
    return c;
  }
  if (d->mode == OR_FIXED) {
    int64_t tile = x / d->s, y = x % d->s;
    int64_t lb = y * d->ips, le = lb + d->ips < d->ipt ? lb + d->ips : d->ipt;
    if (lb >= le) { /* an empty split still takes part in the handshake */
      lb = le = d->ipt;
    }
    /* started/ended as in Algorithm 5: the segment holds iteration 0 / the
     * tile's last iteration */
    if (y != 0) PUSH(tile, lb, le, 0, le == d->ipt, -1);
    else PUSH(tile, lb, le, 1, le == d->ipt, d->s == 1 ? -1 : tile * d->s + d->s - 1);
    return c;
  }
  /* Stream-K region.  CTA x holds the contiguous iteration range
   * [first(x), first(x+1)) of the even split of the region's iterations
   * (Stream-K page, Algorithm 5).  Its segments are the intersections of
   * that range with the tiles it meets, in tile order: a segment holding a
   * tile's first iteration has started the tile, one holding its last
   * iteration has ended it, and a tile started but not ended here is
   * finished by the CTA whose range holds the tile's last iteration. */
  if (d->sk_tiles > 0 && x < d->sk_g) {
    const int64_t r_lo = cta_first_iter(d, x), r_hi = cta_first_iter(d, x + 1);
    if (r_lo < r_hi) {
      for (int64_t tile = r_lo / d->ipt; tile <= (r_hi - 1) / d->ipt; ++tile) {
        const int64_t t_lo = tile * d->ipt, t_hi = t_lo + d->ipt;
        const int64_t lo = r_lo > t_lo ? r_lo : t_lo, hi = r_hi < t_hi ? r_hi : t_hi;
        const int64_t started = lo == t_lo, ended = hi == t_hi;
        PUSH(tile, lo - t_lo, hi - t_lo, started, ended, started && !ended ? cta_of_iter(d, t_hi - 1) : -1);
      }
    }
  }
  /* data-parallel region */
  if (d->mode == OR_SK) return c;
  for (int64_t tile = d->dp_first + x; tile < d->t; tile += d->ncta) PUSH(tile, 0, d->ipt, 1, 1, -1);
  return c;
#undef PUSH
}

/* Plan as records (7 int64 each).  Returns the number of records, -1 on bad
 * arguments, -2 if the mode is undefined for the shape, -3 if cap is too
 * small. */
int64_t or_sk_plan(int64_t m, int64_t n, int64_t k, int64_t bm, int64_t bn, int64_t bk, int mode,
                   int64_t param, int64_t *rec, int64_t cap, int64_t *ncta_out) {
  or_decomp d;
  int rc = decompose(m, n, k, bm, bn, bk, mode, param, &d);
  if (rc) return rc;
  if (ncta_out) *ncta_out = d.ncta;
  int64_t per = d.t + 4; /* a CTA never has more segments than this */
  or_seg *tmp = (or_seg *)malloc(sizeof(or_seg) * (size_t)per);
  if (!tmp) return -1;
  int64_t c = 0;
  for (int64_t x = 0; x < d.ncta; ++x) {
    int64_t ns = cta_segments(&d, x, tmp, per);
    if (ns < 0) { free(tmp); return -1; }
    for (int64_t i = 0; i < ns; ++i) {
      if (c >= cap) { free(tmp); return -3; }
      int64_t *r = rec + 7 * c;
      r[0] = tmp[i].cta; r[1] = tmp[i].tile; r[2] = tmp[i].lb; r[3] = tmp[i].le;
      r[4] = tmp[i].started; r[5] = tmp[i].ended; r[6] = tmp[i].last_peer;
      ++c;
    }
  }
  free(tmp);
  return c;
}

/* ------------------------------------------------------------------------ */
/* Simulated execution of a decomposition.                                  */
/* ------------------------------------------------------------------------ */

static uint64_t xs_next(uint64_t *s) { /* xorshift64*, for the interleaving only */
  uint64_t x = *s;
  x ^= x >> 12; x ^= x << 25; x ^= x >> 27;
  *s = x;
  return x * 0x2545F4914F6CDD1DULL;
}

typedef struct {
  int64_t nseg, cur;   /* segment cursor */
  int phase;           /* 0: compute next segment, 1: collecting peers */
  int64_t next_peer;   /* next peer to wait for (phase 1) */
  or_seg *segs;
  double *accum;       /* BLK_M x BLK_N */
} or_cta;

/* MacLoop (Algorithm 3): zero the accumulator, then iterations [lb, le) of
 * tile `tile`, k ascending.  Tile coordinates follow the m -> n -> k
 * linearisation (reading: the printed "tile_idx / ceil(m/BLK_M)" and
 * "tile_idx % ceil(m/BLK_M)" use the m tile count for both; with the stated
 * m -> n -> k order the divisor is the n tile count). */
static void mac_loop(const double *Ad, const double *Bd, int64_t m, int64_t n, int64_t k,
                     int64_t bm, int64_t bn, int64_t bk, int64_t tiles_n, int64_t tile, int64_t lb,
                     int64_t le, double *accum) {
  int64_t mm = (tile / tiles_n) * bm, nn = (tile % tiles_n) * bn;
  for (int64_t x = 0; x < bm * bn; ++x) accum[x] = 0.0;
  for (int64_t it = lb; it < le; ++it) {
    int64_t kk = it * bk, ke = kk + bk < k ? kk + bk : k;
    for (int64_t i = mm; i < mm + bm && i < m; ++i)
      for (int64_t j = nn; j < nn + bn && j < n; ++j) {
        double s = accum[(i - mm) * bn + (j - nn)];
        for (int64_t l = kk; l < ke; ++l) s += Ad[i * k + l] * Bd[j * k + l];
        accum[(i - mm) * bn + (j - nn)] = s;
      }
  }
}

/*
 * Runs the decomposition with simulated CTAs.  `policy`: 0 = seeded random
 * choice of the next CTA to step, 1 = always the lowest runnable CTA id,
 * 2 = always the highest.  A CTA that waits on a flag that is not set yields.
 * Returns 0 on success, -1 on bad arguments, -2 undefined mode, -4 deadlock.
 * *n_yields receives the number of waits that had to yield.
 */
int or_sk_execute(int64_t m, int64_t n, int64_t k, double alpha, const void *A, int64_t lda,
                  const void *B, int64_t ldb, double beta, const void *Cin, int64_t ldc,
                  int dtype, int layout, int64_t bm, int64_t bn, int64_t bk, int mode,
                  int64_t param, uint64_t seed, int policy, double *out64, int64_t *n_yields) {
  or_decomp d;
  int rc = decompose(m, n, k, bm, bn, bk, mode, param, &d);
  if (rc) return rc;
  const int64_t tiles_n = (n + bn - 1) / bn;
  double *Ad = (double *)malloc(sizeof(double) * (size_t)(m * k));
  double *Bd = (double *)malloc(sizeof(double) * (size_t)(n * k));
  or_cta *ctas = (or_cta *)calloc((size_t)d.ncta, sizeof(or_cta));
  double *partials = (double *)malloc(sizeof(double) * (size_t)(d.ncta * bm * bn));
  int *flags = (int *)calloc((size_t)d.ncta, sizeof(int));
  int64_t per = d.t + 4;
  int ok = Ad && Bd && ctas && partials && flags;
  for (int64_t x = 0; ok && x < d.ncta; ++x) {
    ctas[x].segs = (or_seg *)malloc(sizeof(or_seg) * (size_t)per);
    ctas[x].accum = (double *)malloc(sizeof(double) * (size_t)(bm * bn));
    if (!ctas[x].segs || !ctas[x].accum) { ok = 0; break; }
    ctas[x].nseg = cta_segments(&d, x, ctas[x].segs, per);
    if (ctas[x].nseg < 0) ok = 0;
  }
  int result = ok ? 0 : -1;
  if (ok) {
    for (int64_t i = 0; i < m; ++i)
      for (int64_t l = 0; l < k; ++l) Ad[i * k + l] = dec(dtype, A, a_idx(layout, i, l, lda));
    for (int64_t j = 0; j < n; ++j)
      for (int64_t l = 0; l < k; ++l) Bd[j * k + l] = dec(dtype, B, b_idx(layout, l, j, ldb));
    uint64_t rng = seed * 0x9E3779B97F4A7C15ULL + 0x632BE59BD9B4E019ULL;
    if (!rng) rng = 1;
    int64_t yields = 0, remaining = 0;
    for (int64_t x = 0; x < d.ncta; ++x) remaining += ctas[x].nseg > 0;
    int64_t *runnable = (int64_t *)malloc(sizeof(int64_t) * (size_t)d.ncta);
    while (remaining > 0 && runnable) {
      /* CTAs that can make progress now */
      int64_t nr = 0;
      for (int64_t x = 0; x < d.ncta; ++x) {
        or_cta *c = &ctas[x];
        if (c->cur >= c->nseg) continue;
        if (c->phase == 1 && !flags[c->next_peer]) continue;
        runnable[nr++] = x;
      }
      if (nr == 0) { result = -4; break; }
      /* count the waiting CTAs that are passed over (they yielded) */
      for (int64_t x = 0; x < d.ncta; ++x)
        if (ctas[x].cur < ctas[x].nseg && ctas[x].phase == 1 && !flags[ctas[x].next_peer]) ++yields;
      int64_t pick = policy == 1 ? runnable[0]
                   : policy == 2 ? runnable[nr - 1]
                                 : runnable[xs_next(&rng) % (uint64_t)nr];
      or_cta *c = &ctas[pick];
      or_seg *s = &c->segs[c->cur];
      if (c->phase == 0) {
        mac_loop(Ad, Bd, m, n, k, bm, bn, bk, tiles_n, s->tile, s->lb, s->le, c->accum);
        if (!s->started) {
          /* StorePartials(partials[x]); Signal(flags[x]) */
          memcpy(partials + pick * bm * bn, c->accum, sizeof(double) * (size_t)(bm * bn));
          flags[pick] = 1;
          c->cur++;
          if (c->cur >= c->nseg) --remaining;
          continue;
        }
        if (s->last_peer >= 0) { /* owner that did not end the tile */
          c->phase = 1;
          c->next_peer = pick + 1;
          continue;
        }
      } else {
        /* Wait(flags[peer]) satisfied: accum += LoadPartials(partials[peer]) */
        const double *pp = partials + c->next_peer * bm * bn;
        for (int64_t x = 0; x < bm * bn; ++x) c->accum[x] += pp[x];
        if (c->next_peer < s->last_peer) { c->next_peer++; continue; }
        c->phase = 0;
      }
      /* StoreTile */
      int64_t mm = (s->tile / tiles_n) * bm, nn = (s->tile % tiles_n) * bn;
      for (int64_t i = mm; i < mm + bm && i < m; ++i)
        for (int64_t j = nn; j < nn + bn && j < n; ++j) {
          double v = alpha * c->accum[(i - mm) * bn + (j - nn)];
          if (beta != 0.0) v += beta * dec(dtype, Cin, i * ldc + j);
          out64[i * n + j] = v;
        }
      c->cur++;
      if (c->cur >= c->nseg) --remaining;
    }
    free(runnable);
    if (n_yields) *n_yields = yields;
  }
  if (ctas)
    for (int64_t x = 0; x < d.ncta; ++x) { free(ctas[x].segs); free(ctas[x].accum); }
  free(ctas); free(Ad); free(Bd); free(partials); free(flags);
  return result;
}

/* ------------------------------------------------------------------------ */
/* ABFT: one verification domain (fault-tolerant GEMM page, thread-level    */
/* scheme of Fig. 3 lifted to a block; threadblock-level scheme, Figs. 5-7).*/
/* ------------------------------------------------------------------------ */
/*
 * The block C_blk (rows x cols, row stride cols) was computed as
 * A_blk (rows x kk, row stride kk) times B_blk (kk x cols, row stride cols),
 * possibly with a fault.  Checksums from the encodings e^T A and B e:
 *     rc_i = sum_l A_il (B e)_l        (row checksum,  C e   = A (B e))
 *     cc_j = sum_l (e^T A)_l B_lj      (column checksum, e^T C = (e^T A) B)
 * and absolute versions ra, ca with |A|, |B| for the detection threshold
 * tau = c_tau * 2^-24 * sqrt(kk) * ra_i (rows), likewise with ca_j (columns)
 * (reading: the pages give no threshold; the rounding error of an fp32 dot
 * product of length kk grows like sqrt(kk) * 2^-24 * sum |a||b|).
 * Verify: row residual dr_i = sum_j C_ij - rc_i, column residual dc_j likewise;
 * a row/column mismatches when |residual| > tau or the residual is not finite.
 * Locate: the intersection of the single mismatching row and column.
 * Correct: C_ij <- rc_i - sum_{l != j} C_il (recomputed from the row checksum:
 * the page derives the size of the fix from the checksums' discrepancy,
 * "Anatomy of High-Performance GEMM with Online Fault Tolerance on GPUs",
 * Fig. 3; recomputing instead of subtracting the discrepancy stays correct
 * when the fault made C_ij huge, Inf or NaN).
 * Returns 0 clean, 1 corrected (fills *fi, *fj, *fdelta = faulty - corrected),
 * 2 mismatch that cannot be located to one element, -1 bad arguments.
 */
int or_abft_check(int64_t rows, int64_t cols, int64_t kk, const double *A_blk, const double *B_blk,
                  float *C_blk, double c_tau, int64_t *fi, int64_t *fj, double *fdelta) {
  if (rows <= 0 || cols <= 0 || kk < 0) return -1;
  double *be = (double *)calloc((size_t)(kk ? kk : 1), sizeof(double));
  double *bea = (double *)calloc((size_t)(kk ? kk : 1), sizeof(double));
  double *ea = (double *)calloc((size_t)(kk ? kk : 1), sizeof(double));
  double *eaa = (double *)calloc((size_t)(kk ? kk : 1), sizeof(double));
  if (!be || !bea || !ea || !eaa) { free(be); free(bea); free(ea); free(eaa); return -1; }
  for (int64_t l = 0; l < kk; ++l) {
    for (int64_t j = 0; j < cols; ++j) { be[l] += B_blk[l * cols + j]; bea[l] += fabs(B_blk[l * cols + j]); }
    for (int64_t i = 0; i < rows; ++i) { ea[l] += A_blk[i * kk + l]; eaa[l] += fabs(A_blk[i * kk + l]); }
  }
  const double u = ldexp(1.0, -24) * sqrt((double)(kk > 0 ? kk : 1));
  int64_t bad_r = -1, bad_c = -1, n_bad_r = 0, n_bad_c = 0;
  for (int64_t i = 0; i < rows; ++i) {
    double rc = 0, ra = 0, s = 0;
    for (int64_t l = 0; l < kk; ++l) { rc += A_blk[i * kk + l] * be[l]; ra += fabs(A_blk[i * kk + l]) * bea[l]; }
    for (int64_t j = 0; j < cols; ++j) s += (double)C_blk[i * cols + j];
    double r = s - rc;
    if (!(fabs(r) <= c_tau * u * ra)) { ++n_bad_r; bad_r = i; }
  }
  for (int64_t j = 0; j < cols; ++j) {
    double cc = 0, ca = 0, s = 0;
    for (int64_t l = 0; l < kk; ++l) { cc += ea[l] * B_blk[l * cols + j]; ca += eaa[l] * fabs(B_blk[l * cols + j]); }
    for (int64_t i = 0; i < rows; ++i) s += (double)C_blk[i * cols + j];
    double r = s - cc;
    if (!(fabs(r) <= c_tau * u * ca)) { ++n_bad_c; bad_c = j; }
  }
  int ret;
  if (n_bad_r == 0 && n_bad_c == 0) ret = 0;
  else if (n_bad_r == 1 && n_bad_c == 1) {
    double rc = 0;
    for (int64_t l = 0; l < kk; ++l) rc += A_blk[bad_r * kk + l] * be[l];
    double others = 0;
    for (int64_t j = 0; j < cols; ++j)
      if (j != bad_c) others += (double)C_blk[bad_r * cols + j];
    float fixed = (float)(rc - others);
    if (fi) *fi = bad_r;
    if (fj) *fj = bad_c;
    if (fdelta) *fdelta = (double)C_blk[bad_r * cols + bad_c] - (double)fixed;
    C_blk[bad_r * cols + bad_c] = fixed;
    ret = 1;
  } else ret = 2;
  free(be); free(bea); free(ea); free(eaa);
  return ret;
}

/* ------------------------------------------------------------------------ */
/* Freivalds check.                                                         */
/* ------------------------------------------------------------------------ */
/*
 * For nvec vectors x (n entries each, passed in by the caller, rows of X with
 * stride n): computes y = A (B x) and the bound |alpha| |A| (|B| |x|) +
 * |beta| |C_in| |x| in fp64, and returns in *worst the largest
 * |C_out x - (alpha y + beta C_in x)|_i / bound_i over rows i and vectors
 * (0/0 counts as 0, nonzero/0 as +inf).  C_out has the storage type, row
 * stride ldo.
 */
int or_freivalds(int64_t m, int64_t n, int64_t k, double alpha, const void *A, int64_t lda,
                 const void *B, int64_t ldb, double beta, const void *Cin, int64_t ldc,
                 const void *Cout, int64_t ldo, int dtype, int layout, int64_t nvec,
                 const double *X, double *worst, int nthreads) {
  double *y = (double *)malloc(sizeof(double) * (size_t)(k ? k : 1));
  double *ya = (double *)malloc(sizeof(double) * (size_t)(k ? k : 1));
  if (!y || !ya) { free(y); free(ya); return -1; }
  double w = 0.0;
  int nt = set_threads(nthreads);
  for (int64_t v = 0; v < nvec; ++v) {
    const double *x = X + v * n;
#pragma omp parallel for num_threads(nt)
    for (int64_t l = 0; l < k; ++l) {
      double s = 0, sa = 0;
      for (int64_t j = 0; j < n; ++j) {
        double b = dec(dtype, B, b_idx(layout, l, j, ldb));
        s += b * x[j];
        sa += fabs(b) * fabs(x[j]);
      }
      y[l] = s; ya[l] = sa;
    }
#pragma omp parallel for num_threads(nt) reduction(max : w)
    for (int64_t i = 0; i < m; ++i) {
      double z = 0, za = 0, cx = 0, cix = 0, cia = 0;
      for (int64_t l = 0; l < k; ++l) {
        double a = dec(dtype, A, a_idx(layout, i, l, lda));
        z += a * y[l];
        za += fabs(a) * ya[l];
      }
      for (int64_t j = 0; j < n; ++j) {
        cx += dec(dtype, Cout, i * ldo + j) * x[j];
        if (beta != 0.0) {
          double c = dec(dtype, Cin, i * ldc + j);
          cix += c * x[j];
          cia += fabs(c) * fabs(x[j]);
        }
      }
      double num = fabs(cx - (alpha * z + beta * cix));
      double den = fabs(alpha) * za + fabs(beta) * cia;
      double r = num == 0.0 ? 0.0 : (den == 0.0 ? INFINITY : num / den);
      if (isnan(r)) r = INFINITY;
      if (r > w) w = r;
    }
  }
  *worst = w;
  free(y); free(ya);
  return 0;
}
