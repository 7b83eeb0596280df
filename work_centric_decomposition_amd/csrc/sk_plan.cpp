// sk_plan.cpp -- the work decomposition (host side, integers only).
//
// Stream-K page ("Stream-K: Work-centric Parallel Decomposition for Dense
// Matrix-Matrix Multiplication on the GPU"):
//  * section 3.2 / Algorithm 2: data-parallel, one tile per workgroup;
//  * section 4 / Algorithm 5: the total MAC-loop iterations t * ipt are laid
//    out in m -> n -> k order and split evenly over g workgroups; a tile is
//    written by the workgroup holding its k = 0 iteration after it adds the
//    partial sums of the other workgroups that covered the tile;
//  * section 5.2: "data-parallel + one-tile Stream-K" (only the r = t mod p
//    leftover tiles are split) and "two-tile Stream-K + data-parallel" (one
//    full data-parallel wave is given back so every Stream-K workgroup gets
//    between one and two tiles of iterations; each owner then receives from
//    exactly one peer);
//  * section 5.1 / appendix A.1: the grid size is picked by a runtime model
//    with a fixed cost a, a partial-output cost b, a per-iteration cost c and
//    a per-peer cost d.  The page's equation did not survive; the form used
//    here is the plainest one built from those four definitions:
//        T(g) = a + b * [some tile is split] + c * ceil(total / g)
//                 + d * (most peers any owner adds),
//    minimised over g in [t, min(p, total)], ties to the smaller g.
//
// Readings (the page leaves these open):
//  * the split is even to within one iteration (the prose), i.e. workgroup x
//    covers [x*q + min(x, r), (x+1)*q + min(x+1, r)) with q = floor(I/g),
//    r = I mod g; the printed pseudo-code's ceil(I/g) per workgroup gives the
//    same ranges whenever g divides I;
//  * the Stream-K region is the first tiles in linear order; each workgroup
//    runs its Stream-K segments first and then its data-parallel tiles,
//    which are dealt round-robin (tile sk_tiles + x + j*g);
//
// XCD-aware schedule (this library's design for MI355X, not the page's): on
// a chip whose 256 CUs sit in 8 XCDs with one L2 each, a workgroup reads
// 2 * 256 * 64 * 2 bytes per 64-deep fp16 iteration, so the 256 workgroups
// together ask for about 10 TB/s and the L2s must serve most of it.  Under
// the page's even split every workgroup starts at a different k offset and
// the L2 hit rate falls from about 0.6-0.7 (data-parallel) to under 0.2
// (measured with TCC_HIT / TCC_MISS), which makes the Stream-K region slower
// per iteration than data-parallel.  The XCD-aware schedule (see Sched)
// quantises the split to ipt / D so that the workgroups of one XCD run in
// lock-step on a compact block of tiles.  Its planning:
//  * the Stream-K region is all tiles when w < hybrid_min_waves (w == 0
//    included), else one full wave plus the r leftover tiles (two-tile
//    hybrid); r == 0 with w >= 1 leaves no region (XCD-ordered DP);
//  * with a wave or more, D is 8, 16 or 32, whichever gives the shortest
//    per-workgroup work s * ipt / D (s = ceil(D * sk_tiles / p)), each
//    doubling of D charged 3 % since it halves the workgroups in lock-step;
//  * below a wave, D (a multiple of 8 up to p) and s are chosen by the
//    runtime model with g = D * ceil(t / s), the same 3 % charge per doubling
//    of D beyond 16, and AUTO also asks for at least 15 % fewer iterations
//    per workgroup than the single data-parallel wave (kSmallGain);
//  * AUTO keeps the region only when the model predicts it beats the
//    XCD-ordered data-parallel form.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "sk_internal.h"

namespace sk {

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Iteration cost of a grid of g workgroups relative to a workgroup alone on
// its CU: the instance's c_shared once every slot of a CU is busy, linear in
// the workgroups per CU in between (the dispatcher spreads a grid over the
// CUs before it doubles up).
static double share(const TileCfg &c, int slots, int64_t g) {
  if (c.occupancy <= 1) return 1.0;
  const int64_t cus = std::max<int64_t>(1, slots / c.occupancy);
  const int64_t j = std::min<int64_t>(c.occupancy, cdiv(g, cus));
  return 1.0 + (c.c_shared - 1.0) * (double)(j - 1) / (c.occupancy - 1);
}

bool operand_direct(int dtype, bool kmajor, const void *ptr, int64_t ld, int64_t k, int64_t mn, bool mn_ok) {
  const int64_t es = dtype == SK_F32 ? 4 : 2;
  const int64_t vec = 16 / es;  // elements per 128-bit load
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return false;
  if (ld % vec != 0) return false;
  if (kmajor && k % vec != 0) return false;  // a 128-bit chunk never straddles k
  if (dtype != SK_F32 && !kmajor) {
    // HGEMM reads an m-contiguous A or n-contiguous B in place on the 256
    // and 128 instances: whole 128-bit chunks along m or n, and byte offsets
    // over all of k that fit a 31-bit buffer offset
    if (!mn_ok || mn % vec != 0) return false;
    if ((k + 64) * ld * es + 1024 >= 0x7FFFFFFF) return false;
  }
  return true;
}

// Largest number of workgroups covering one tile, minus one, for the basic
// split of `tiles` tiles of `ipt` iterations over g workgroups; also reports
// whether any tile is split.
static int split_peers(int64_t tiles, int64_t ipt, int64_t g, bool *any_split) {
  const int64_t I = tiles * ipt, q = I / g, r = I % g;
  auto sk_owner_of = [](int64_t q, int64_t r, int64_t it) {
    const int64_t big = r * (q + 1);
    return it < big ? it / (q + 1) : r + (it - big) / q;
  };
  int peers = 0;
  bool split = false;
  for (int64_t t = 0; t < tiles; ++t) {
    int64_t first = sk_owner_of(q, r, t * ipt), last = sk_owner_of(q, r, (t + 1) * ipt - 1);
    int64_t p = last - first;
    if (p > 0) split = true;
    if (p > peers) peers = (int)p;
  }
  if (any_split) *any_split = split;
  return peers;
}

// Grid size of basic Stream-K from the runtime model (evaluated in O(1) per
// candidate, so planning stays cheap next to a small kernel): a tile is
// split unless every workgroup boundary falls on a tile boundary, and a tile
// of ipt iterations meets at most ceil((ipt - 1) / q) + 1 workgroups whose
// ranges hold at least q iterations.
static int64_t model_grid(const TileCfg &cfg, int64_t t, int64_t ipt, int slots, float a, float b, float c,
                          float d) {
  const int64_t total = t * ipt;
  int64_t hi = std::min<int64_t>(slots, total);
  if (hi <= t) return t;
  double best = 1e300;
  int64_t best_g = t;
  for (int64_t g = t; g <= hi; ++g) {
    const int64_t q = total / g, r = total % g;
    const bool split = !(r == 0 && q % ipt == 0);
    const int64_t peers = split ? std::max<int64_t>(1, cdiv(ipt - 1, q)) : 0;
    const double T = a + (split ? b : 0.0) + c * (double)cdiv(total, g) * share(cfg, slots, g) + d * (double)peers;
    if (T < best - 1e-9) { best = T; best_g = g; }
  }
  return best_g;
}

// Below one wave, the smallest iteration gain of the split over the single
// data-parallel wave that AUTO accepts.
static constexpr double kSmallGain = 1.15;

// Charge for the phase classes that share one XCD's L2 (D / 8 of them).
static double phase_charge(int64_t D) {
  double f = 1.0;
  for (int64_t d = 16; d < D; d *= 2) f *= 1.03;
  return f;
}

// XCD-aware schedule over a Stream-K region of sk_tiles tiles with the whole
// grid (a wave or more): D in {8, 16, 32} and s = ceil(D * sk_tiles / p).
static void aligned_wave(int64_t sk_tiles, int64_t ipt, int slots, int *D_out, int *s_out) {
  double best = 1e300;
  for (int64_t D = 8; D <= 32 && D <= slots; D *= 2) {
    if (slots % D) continue;
    const int64_t s = cdiv(D * sk_tiles, slots);
    const double T = (double)cdiv(s * ipt, D) * (D > 8 ? 1.03 * phase_charge(D) : 1.0);
    if (T < best - 1e-9) { best = T; *D_out = (int)D; *s_out = (int)s; }
  }
}

// XCD-aware schedule below one wave: D (multiple of 8 dividing p) and s by
// the runtime model with g = D * ceil(t / s) workgroups.
static double aligned_small(const TileCfg &cfg, int64_t t, int64_t ipt, int slots, float a, float b, float c,
                            float d, int *D_out, int *s_out) {
  double best = 1e300;
  for (int64_t D = 8; D <= slots; D *= 2) {
    if (slots % D) continue;
    for (int64_t s = 1; s <= D; ++s) {
      const int64_t J = cdiv(t, s);
      if (D * J > slots) continue;
      const bool split = s % D != 0 || (s * ipt) % D != 0;
      const int64_t work = cdiv(s * ipt, D);
      // the partials of a tile meet in a binary tree: on its critical path
      // each of the ceil(log2(pieces)) levels stores a partial (b) and adds
      // it (d) one after the other.  Workgroup x of a class covers
      // [floor(x s ipt / D), floor((x + 1) s ipt / D)); the widest of its s
      // tiles sets the depth.
      int64_t pieces = 1;
      for (int64_t j = 0; split && j < s; ++j) {
        const int64_t f = ((j * ipt + 1) * D - 1) / (s * ipt), l = (((j + 1) * ipt) * D - 1) / (s * ipt);
        pieces = std::max(pieces, l - f + 1);
      }
      int64_t levels = 0;
      while (((int64_t)1 << levels) < pieces) ++levels;
      const double T = (a + c * (double)work * share(cfg, slots, D * J) + (b + d) * (double)levels) * phase_charge(D);
      if (T < best - 1e-9) { best = T; *D_out = (int)D; *s_out = (int)s; }
    }
  }
  return best;
}

struct DecisionKey {
  int dtype, inst;
  int64_t tiles_m, tiles_n, ipt;
  int slots, schedule, forced_grid, min_waves;
  float ma, mb, mc, md;
  bool operator==(const DecisionKey &o) const {
    return dtype == o.dtype && inst == o.inst && tiles_m == o.tiles_m && tiles_n == o.tiles_n && ipt == o.ipt && slots == o.slots &&
           schedule == o.schedule && forced_grid == o.forced_grid && min_waves == o.min_waves && ma == o.ma &&
           mb == o.mb && mc == o.mc && md == o.md;
  }
};
struct Decision {
  DecisionKey key;
  int schedule, grid, phase_div, blocks, group_rows;
  int64_t sk_tiles, sk_q, sk_r;
  bool valid;
};
static std::mutex g_decision_mu;
static Decision g_decisions[64];
static unsigned g_decision_next = 0;

static bool lookup_decision(const DecisionKey &k, Plan &P) {
  std::lock_guard<std::mutex> lock(g_decision_mu);
  for (const Decision &e : g_decisions) {
    if (!e.valid || !(e.key == k)) continue;
    P.schedule = e.schedule; P.grid = e.grid; P.phase_div = e.phase_div; P.blocks = e.blocks;
    P.group_rows = e.group_rows; P.sk_tiles = e.sk_tiles; P.sk_q = e.sk_q; P.sk_r = e.sk_r;
    P.dp_tiles = P.tiles - P.sk_tiles;
    return true;
  }
  return false;
}

static void store_decision(const DecisionKey &k, const Plan &P) {
  std::lock_guard<std::mutex> lock(g_decision_mu);
  Decision &e = g_decisions[g_decision_next++ % 64];
  e = Decision{k, P.schedule, P.grid, P.phase_div, P.blocks, P.group_rows, P.sk_tiles, P.sk_q, P.sk_r, true};
}

// The plan of one tile instance (arguments already validated).
static int plan_inst(const sk_gemm_desc &d, const sk_options &o, int inst, int slots, Plan &P) {
  std::memset(&P, 0, sizeof(P));
  P.m = d.m; P.n = d.n; P.k = d.k;
  P.dtype = d.dtype; P.layout = d.layout;
  P.cfg = tile_cfg(d.dtype, inst);
  P.slots = slots;
  const TileCfg &c = P.cfg;
  P.tiles_m = cdiv(d.m, c.bm);
  P.tiles_n = cdiv(d.n, c.bn);
  P.tiles = P.tiles_m * P.tiles_n;
  P.ipt = cdiv(d.k, c.bk);
  P.total = P.tiles * P.ipt;
  P.w = (int)(P.tiles / slots);
  P.r = (int)(P.tiles % slots);
  const bool a_kmajor = d.layout == SK_A_ROW_B_ROW || d.layout == SK_A_ROW_B_COL;
  const bool b_kmajor = d.layout == SK_A_ROW_B_COL || d.layout == SK_A_COL_B_COL;
  P.pack_a = !operand_direct(d.dtype, a_kmajor, d.A, d.lda, d.k, d.m, inst < 2);
  P.pack_b = !operand_direct(d.dtype, b_kmajor, d.B, d.ldb, d.k, d.n, inst < 2);
  if (P.tiles == 0 || P.ipt == 0) {  // nothing to decompose (quick-return paths)
    P.schedule = SK_SCHED_DP;
    return SK_OK;
  }
  const float ma = o.model_a > 0 ? o.model_a : c.a;
  const float mb = o.model_b > 0 ? o.model_b : c.b;
  const float mc = o.model_c > 0 ? o.model_c : c.c;
  const float md = o.model_d > 0 ? o.model_d : c.d;
  const int min_waves = o.hybrid_min_waves > 0 ? o.hybrid_min_waves : 1;

  // The schedule depends only on these integers and the options; a small
  // cache keeps its search (a few microseconds below a wave) off the launch
  // path of repeated shapes.
  const DecisionKey key{d.dtype, inst, P.tiles_m, P.tiles_n, P.ipt, slots, o.schedule, o.forced_grid, min_waves,
                        ma, mb, mc, md};
  if (lookup_decision(key, P)) return SK_OK;

  int sched = o.schedule;
  int64_t grid = 0, sk_tiles = 0;
  if (o.forced_grid > 0) {
    sched = SK_SCHED_SK_BASIC;
    grid = o.forced_grid;
    sk_tiles = P.tiles;
  } else {
    if (sched == SK_SCHED_AUTO) sched = SK_SCHED_XCD_ALIGNED;
    // the page's two-tile hybrid needs hybrid_min_waves full waves (reading
    // of its "w >= 2" against the mechanism, which works from one wave);
    // with fewer it is basic Stream-K over all tiles, with no leftover tiles
    // data-parallel
    if (sched == SK_SCHED_SK_HYBRID2 && (P.w < min_waves || P.r == 0))
      sched = P.r == 0 ? SK_SCHED_DP : SK_SCHED_SK_BASIC;
    switch (sched) {
      case SK_SCHED_DP:
        grid = std::min<int64_t>(P.tiles, slots);
        sk_tiles = 0;
        break;
      case SK_SCHED_SK_BASIC:
        grid = P.tiles >= slots ? slots : model_grid(c, P.tiles, P.ipt, slots, ma, mb, mc, md);
        sk_tiles = P.tiles;
        break;
      case SK_SCHED_SK_HYBRID2:
        grid = slots;
        sk_tiles = P.r + slots;
        break;
      case SK_SCHED_SK_HYBRID1:
        grid = slots;
        sk_tiles = P.r;
        break;
      case SK_SCHED_XCD_ALIGNED: {
        P.group_rows = 8;
        int D = 0, s = 0;
        if (P.w == 0) {
          const double t_al = aligned_small(c, P.tiles, P.ipt, slots, ma, mb, mc, md, &D, &s);
          // the data-parallel form: one tile per workgroup.  Below a wave it
          // leaves p - t CUs idle and the busy ones then run at a higher
          // clock, so the split must also promise at least 15 % fewer
          // iterations per workgroup (measured on the fp16 shape sweep:
          // splits promising 10 % ran 7 % slower than the single wave)
          const double dp_iter = (double)P.ipt * share(c, slots, P.tiles);
          const double t_dp = ma + mc * dp_iter;
          const double work = (double)cdiv((int64_t)s * P.ipt, D) * share(c, slots, (int64_t)D * cdiv(P.tiles, s));
          if (o.schedule == SK_SCHED_AUTO && (t_dp <= t_al || dp_iter < kSmallGain * work)) D = 0;
        } else if (P.r > 0) {
          sk_tiles = P.w >= min_waves ? P.r + slots : P.tiles;
          aligned_wave(sk_tiles, P.ipt, slots, &D, &s);
          const double t_al = (double)cdiv((int64_t)s * P.ipt, D) +
                              (double)((P.tiles - sk_tiles) / slots) * P.ipt + (mb + md) / mc;
          const double t_dp = (double)(P.w + 1) * P.ipt;
          if (o.schedule == SK_SCHED_AUTO && t_dp <= t_al) D = 0;
        }
        if (D > 0) {
          if (P.w == 0) sk_tiles = P.tiles;
          P.phase_div = D;
          P.blocks = s;
          grid = P.w == 0 ? (int64_t)D * cdiv(P.tiles, s) : slots;
        } else {
          sk_tiles = 0;
          grid = std::min<int64_t>(P.tiles, slots);
        }
        break;
      }
    }
  }
  if (grid > INT32_MAX / 2) return SK_ERR_UNSUPPORTED;
  P.schedule = sched;
  P.grid = (int)grid;
  P.sk_tiles = sk_tiles;
  P.dp_tiles = P.tiles - sk_tiles;
  if (sk_tiles > 0 && P.phase_div > 0) {
    P.sk_q = (int64_t)P.blocks * P.ipt / P.phase_div;
    P.sk_r = (int64_t)P.blocks * P.ipt % P.phase_div;
  } else if (sk_tiles > 0) {
    const int64_t I = sk_tiles * P.ipt;
    P.sk_q = I / grid;
    P.sk_r = I % grid;
  }
  if (!sched_fits(P.tiles, P.tiles_m, P.tiles_n, P.ipt, P.grid, P.sk_tiles, P.phase_div, P.blocks)) {
    // the kernels walk schedules in 32-bit arithmetic; beyond it (k in the
    // millions with the XCD-aware quanta) AUTO takes the page's hybrid,
    // whose Stream-K region is smaller, else the data-parallel order
    if (o.schedule != SK_SCHED_AUTO) return SK_ERR_UNSUPPORTED;
    sk_options o2 = o;
    o2.schedule = SK_SCHED_SK_HYBRID2;
    int rc = plan_inst(d, o2, inst, slots, P);
    if (rc == SK_ERR_UNSUPPORTED) {
      o2.schedule = SK_SCHED_DP;
      rc = plan_inst(d, o2, inst, slots, P);
    }
    if (rc != SK_OK) return rc;
  }
  store_decision(key, P);
  return SK_OK;
}

// Predicted time of a plan in microseconds, by the runtime model: the fixed
// cost, the workgroup with the most iterations (its Stream-K range plus its
// data-parallel tiles), and the exchanges on the critical path of the most
// divided tile (s - 1 partials added in a row by the page's owner, or
// ceil(log2 s) store/add levels in the tree); constants per tile instance.
double plan_cost_us(const Plan &P) {
  const TileCfg &c = P.cfg;
  if (P.tiles == 0 || P.ipt == 0) return 0.0;
  double work = (double)cdiv(P.dp_tiles, std::max(P.grid, 1)) * (double)P.ipt;
  int64_t pieces = 1;
  if (P.sk_tiles > 0) {
    work += P.phase_div > 0 ? (double)cdiv((int64_t)P.blocks * P.ipt, P.phase_div)
                            : (double)(P.sk_q + (P.sk_r > 0 ? 1 : 0));
    const Sched S = P.sched();
    for (int32_t L = 0; L < S.sk_tiles; ++L) {
      const int32_t ts = L * S.ipt;
      pieces = std::max<int64_t>(pieces, sched_owner_of(S, ts + S.ipt - 1) - sched_owner_of(S, ts) + 1);
    }
  }
  double levels = 0.0;
  if (pieces > 1) {
    if (P.phase_div > 0) {
      int l = 0;
      while (((int64_t)1 << l) < pieces) ++l;
      levels = l;
    } else {
      levels = (double)(pieces - 1);
    }
  }
  double iter = c.iter_a_us + c.iter_b_us * (double)P.grid / P.slots;
  if (c.occupancy > 1) {  // iter_a with a CU to itself, iter_b with every slot busy
    const int64_t cus = std::max<int64_t>(1, P.slots / c.occupancy);
    const int64_t j = std::min<int64_t>(c.occupancy, cdiv(P.grid, cus));
    iter = c.iter_a_us + (c.iter_b_us - c.iter_a_us) * (double)(j - 1) / (c.occupancy - 1);
  }
  return c.fixed_us + iter * work + c.level_us * levels;
}

struct InstKey {
  int dtype;
  int64_t tm, tn, ipt;  // 128-row and 128-column tile counts, k-iterations
  int slots0, slots1, schedule, forced_grid, min_waves;
  float ma, mb, mc, md;
  bool operator==(const InstKey &o) const {
    return dtype == o.dtype && tm == o.tm && tn == o.tn && ipt == o.ipt && slots0 == o.slots0 &&
           slots1 == o.slots1 && schedule == o.schedule && forced_grid == o.forced_grid &&
           min_waves == o.min_waves && ma == o.ma && mb == o.mb && mc == o.mc && md == o.md;
  }
};
static std::mutex g_inst_mu;
static std::pair<InstKey, int> g_inst[64];
static bool g_inst_valid[64];
static unsigned g_inst_next = 0;

// A grid above the resident slot count runs only if workgroups are
// dispatched in index order (per XCD) as slots free up.  Owners wait only on
// higher-numbered peers whose partial is their first segment, so the
// smallest resident workgroup can block only on a peer at least slots - 8
// workgroups after it (eight XCDs, each dispatching its share in order);
// plans whose owners reach that far could wait on a workgroup that cannot
// be dispatched before they finish, and are refused.
static int forced_grid_ok(int rc, const Plan &P) {
  if (rc != SK_OK || P.grid <= P.slots) return rc;
  return plan_max_peers(P) < P.slots - 8 ? SK_OK : SK_ERR_UNSUPPORTED;
}

int make_plan(const sk_gemm_desc &d, const sk_options &o, const int slots[3], Plan &P) {
  std::memset(&P, 0, sizeof(P));
  if (d.m < 0 || d.n < 0 || d.k < 0) return SK_ERR_INVALID_ARG;
  if (d.dtype != SK_F32 && d.dtype != SK_F16 && d.dtype != SK_BF16) return SK_ERR_INVALID_ARG;
  if (d.layout < SK_A_ROW_B_ROW || d.layout > SK_A_COL_B_COL) return SK_ERR_INVALID_ARG;
  if (o.schedule < SK_SCHED_AUTO || o.schedule > SK_SCHED_GEMV_SPLIT) return SK_ERR_INVALID_ARG;
  if (o.schedule == SK_SCHED_GEMV_SPLIT) return SK_ERR_UNSUPPORTED;  // not a matrix-vector call
  if (o.tile < SK_TILE_AUTO || o.tile > SK_TILE_NARROW) return SK_ERR_INVALID_ARG;
  if (o.forced_grid < 0 || slots[0] <= 0 || slots[1] <= 0 || slots[2] <= 0) return SK_ERR_INVALID_ARG;
  // 32-bit indices inside the kernels
  if (d.m > INT32_MAX / 2 || d.n > INT32_MAX / 2 || d.k > INT32_MAX / 2) return SK_ERR_UNSUPPORTED;
  // a forced grid is a count of large-tile workgroups unless a tile is given
  // fp32: no narrow-m instance, and ABFT runs on the 128 x 128 tile only
  const bool f32 = d.dtype == SK_F32;
  if (f32 && (o.tile == SK_TILE_NARROW || (o.abft && o.tile == SK_TILE_SMALL))) return SK_ERR_UNSUPPORTED;
  if ((f32 && o.abft) || o.tile == SK_TILE_LARGE || (o.tile == SK_TILE_AUTO && o.forced_grid > 0))
    return forced_grid_ok(plan_inst(d, o, 0, slots[0], P), P);
  if (o.tile == SK_TILE_SMALL) return forced_grid_ok(plan_inst(d, o, 1, slots[1], P), P);
  if (o.tile == SK_TILE_NARROW) {
    if (d.m > 256) return SK_ERR_UNSUPPORTED;
    return forced_grid_ok(plan_inst(d, o, narrow_inst(d.m), slots[2], P), P);
  }
  // AUTO: whichever instance the model predicts faster (cached per shape
  // class); measured on the fp16 shape sweep, the small tile wins on most
  // shapes below one wave of large tiles and on short-k shapes up to about
  // two waves, the large one on long-k and large shapes (fp32 likewise)
  int rc = plan_inst(d, o, 0, slots[0], P);
  if (rc != SK_OK || P.tiles == 0 || P.ipt == 0) return rc;
  const InstKey key{d.dtype, cdiv(d.m, 128), cdiv(d.n, 128), P.ipt, slots[0], slots[1], o.schedule,
                    o.forced_grid, o.hybrid_min_waves, o.model_a, o.model_b, o.model_c, o.model_d};
  int inst = -1;
  {
    std::lock_guard<std::mutex> lock(g_inst_mu);
    for (int i = 0; i < 64; ++i)
      if (g_inst_valid[i] && g_inst[i].first == key) inst = g_inst[i].second;
  }
  if (inst == 0) return SK_OK;
  Plan Q;
  rc = plan_inst(d, o, 1, slots[1], Q);
  if (rc != SK_OK) return SK_OK;  // the large-tile plan stands
  if (inst < 0) {
    inst = plan_cost_us(Q) < plan_cost_us(P) ? 1 : 0;
    std::lock_guard<std::mutex> lock(g_inst_mu);
    const unsigned i = g_inst_next++ % 64;
    g_inst[i] = {key, inst};
    g_inst_valid[i] = true;
  }
  if (inst == 1) P = Q;
  return SK_OK;
}

bool gemv_plan(const sk_gemm_desc &d, int cus, GemvPlan &g) {
  if (d.k <= 0 || d.m <= 0 || d.n <= 0 || cus <= 0) return false;
  const int64_t es = d.dtype == SK_F32 ? 4 : 2, vec = 16 / es;
  const bool ak = d.layout == SK_A_ROW_B_ROW || d.layout == SK_A_ROW_B_COL;
  const bool bk = d.layout == SK_A_ROW_B_COL || d.layout == SK_A_COL_B_COL;
  g.form = kGemvDot;
  g.incv = 1;
  g.V = 1;
  g.ldv = g.ld_v = g.ld_r = 0;
  if (d.k <= 0) return false;
  // 2 .. 16 vectors against k-contiguous rows (neither m nor n 1): the
  // multi form
  // (fp16 and bf16: up to 8; beyond that the tiled kernels are as fast)
  const int64_t vmax = d.dtype == SK_F32 ? 16 : 8;
  const bool few_m = d.m >= 2 && d.m <= vmax, few_n = d.n >= 2 && d.n <= vmax;
  if ((few_m || few_n) && d.m >= 2 && d.n >= 2 && ak && bk) {
    g.form = kGemvMulti;
    if (few_m) {  // rows of A against the rows of column-major B
      g.V = (int)d.m; g.v = d.A; g.ldv = d.lda; g.M = d.B; g.ldm = d.ldb; g.R = d.n;
      g.ld_v = d.ldc; g.ld_r = 1;
    } else {  // columns of B against the rows of row-major A
      g.V = (int)d.n; g.v = d.B; g.ldv = d.ldb; g.M = d.A; g.ldm = d.lda; g.R = d.m;
      g.ld_v = 1; g.ld_r = d.ldc;
    }
    g.out = d.C; g.ldo = 0; g.K = d.k;
    if (reinterpret_cast<uintptr_t>(g.M) % 16 || reinterpret_cast<uintptr_t>(g.v) % 16) return false;
    if ((g.ldm * es) % 16 || (g.ldv * es) % 16) return false;
    // k slabs of one load per lane (64 bytes of every row per wave load);
    // chunks of at least eight slabs; tasks of 64 rows (fp32) or 16, about 8
    // (fp32) or 16 of them per CU
    const int64_t slab = 64 / es;
    const int64_t rows = d.dtype == SK_F32 ? 64 : 16;
    const int64_t blocks = cdiv(g.R, rows);
    const int64_t want = cdiv((int64_t)(d.dtype == SK_F32 ? 8 : 16) * cus, blocks);
    int64_t S = std::max<int64_t>(1, std::min<int64_t>(want, g.K / (8 * slab)));
    g.chunk = cdiv(cdiv(g.K, S), slab) * slab;
    g.S = cdiv(g.K, g.chunk);
    g.grid = (int)std::min<int64_t>(cdiv(blocks * g.S, 4), (int64_t)8 * cus);
    return true;
  }
  if (d.m != 1 && d.n != 1) return false;
  if (d.n == 1 && ak && (bk || d.ldb == 1 || d.k == 1)) {  // rows of A against the column B
    g.M = d.A; g.ldm = d.lda; g.v = d.B; g.R = d.m; g.out = d.C; g.ldo = d.ldc;
  } else if (d.m == 1 && bk && (ak || d.lda == 1 || d.k == 1)) {  // the row A against columns of B
    g.M = d.B; g.ldm = d.ldb; g.v = d.A; g.R = d.n; g.out = d.C; g.ldo = 1;
  } else if (d.m == 1 && !bk) {  // C row = sum_k A[0, k] B[k, :], B rows contiguous along n
    g.form = kGemvAxpy;
    g.M = d.B; g.ldm = d.ldb; g.v = d.A; g.incv = ak ? 1 : d.lda; g.R = d.n; g.out = d.C; g.ldo = 1;
  } else if (d.n == 1 && !ak) {  // C column = sum_k A[:, k] B[k, 0], A columns contiguous along m
    g.form = kGemvAxpy;
    g.M = d.A; g.ldm = d.lda; g.v = d.B; g.incv = bk ? 1 : d.ldb; g.R = d.m; g.out = d.C; g.ldo = d.ldc;
  } else {
    return false;
  }
  g.K = d.k;
  if (reinterpret_cast<uintptr_t>(g.M) % 16) return false;
  if (g.form == kGemvDot) {
    if (reinterpret_cast<uintptr_t>(g.v) % 16) return false;
    if (g.R > 1 && (g.ldm * es) % 16) return false;
    // enough chunks to keep every CU busy (about 32 per CU), none shorter
    // than eight 1 KiB passes of a wave (the kernel keeps eight in flight)
    const int64_t piece = 64 * vec;
    const int64_t want = cdiv((int64_t)32 * cus, g.R);
    int64_t S = std::max<int64_t>(1, std::min<int64_t>(want, g.K / (8 * piece)));
    g.chunk = cdiv(cdiv(g.K, S), vec) * vec;
    g.S = cdiv(g.K, g.chunk);
    g.grid = (int)std::min<int64_t>(cdiv(g.R * g.S, 4), (int64_t)8 * cus);
    return true;
  }
  if (g.K > 1 && (g.ldm * es) % 16) return false;
  // output blocks of one wave's width (64 lanes x 16 bytes); chunks of at
  // least 64 rows, enough (block, chunk) tasks for about 8 per CU: each
  // task streams a whole chunk, and more chunks only add partial sums to
  // write and add up
  const int64_t blocks = cdiv(g.R, 64 * vec);
  const int64_t want = cdiv((int64_t)8 * cus, blocks);
  const int64_t S = std::max<int64_t>(1, std::min<int64_t>(want, g.K / 64));
  g.chunk = cdiv(g.K, S);
  g.S = cdiv(g.K, g.chunk);
  g.grid = (int)std::min<int64_t>(cdiv(blocks * g.S, 4), (int64_t)8 * cus);
  return true;
}

int plan_max_peers(const Plan &P) {
  if (P.sk_tiles <= 0) return 0;
  if (P.phase_div <= 0) return split_peers(P.sk_tiles, P.ipt, P.grid, nullptr);
  const Sched S = P.sched();
  int32_t peers = 0;
  for (int32_t x = 0; x < P.grid; ++x)
    sched_segments(S, x, [&](int32_t, int32_t, int32_t, bool, bool, int32_t lp) {
      if (lp >= 0 && lp - x > peers) peers = lp - x;
    });
  return (int)peers;
}

}  // namespace sk

using namespace sk;

extern "C" int64_t sk_plan_segments(const sk_plan *plan, int64_t x, sk_segment *out, int64_t cap) {
  if (!plan || x < 0 || cap < 0 || (cap > 0 && !out)) return SK_ERR_INVALID_ARG;
  if (plan->schedule == SK_SCHED_GEMV_SPLIT) return 0;
  if (x >= plan->grid) return 0;
  if (plan->iters_per_tile <= 0 || plan->tiles <= 0) return 0;
  if (plan->phase_div > 0 && plan->sk_blocks <= 0) return SK_ERR_INVALID_ARG;
  if (!sched_fits(plan->tiles, plan->tiles_m, plan->tiles_n, plan->iters_per_tile, plan->grid, plan->sk_tiles,
                  plan->phase_div, plan->sk_blocks))
    return SK_ERR_INVALID_ARG;
  Sched S{};
  S.ipt = (int32_t)plan->iters_per_tile; S.tiles = (int32_t)plan->tiles;
  S.tiles_m = (int32_t)plan->tiles_m; S.tiles_n = (int32_t)plan->tiles_n;
  S.sk_tiles = (int32_t)plan->sk_tiles; S.sk_q = (int32_t)plan->sk_iters_q; S.sk_r = (int32_t)plan->sk_iters_r;
  S.grid = plan->grid; S.phase_div = plan->phase_div; S.blocks = plan->sk_blocks;
  S.group_rows = plan->group_rows;
  S.tree = plan->fixup_tree ? 1 : 0;
  sched_derive(S);
  int64_t n = 0;
  sched_segments(S, (int32_t)x, [&](int32_t tile, int32_t lb, int32_t le, bool st, bool en, int32_t lp) {
    if (n < cap) out[n] = sk_segment{tile, lb, le, st ? 1 : 0, en ? 1 : 0, lp};
    ++n;
  });
  return n;
}
