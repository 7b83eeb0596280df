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
//  * AUTO: r == 0 is plain data-parallel; w == 0 is basic Stream-K with the
//    model's grid size; w >= hybrid_min_waves (default 1) and r > 0 is the
//    two-tile hybrid when the model predicts it beats data-parallel (the
//    iterations it saves exceed the cost of one partial and one peer), else
//    data-parallel.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "sk_internal.h"

namespace sk {

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool operand_direct(int dtype, bool kmajor, const void *ptr, int64_t ld, int64_t k) {
  const int64_t es = dtype == SK_F32 ? 4 : 2;
  const int64_t vec = 16 / es;  // elements per 128-bit load
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return false;
  if (ld % vec != 0) return false;
  if (dtype != SK_F32 && !kmajor) return false;  // HGEMM reads k-contiguous tiles only
  if (kmajor && k % vec != 0) return false;       // a 128-bit chunk never straddles k
  return true;
}

// Largest number of workgroups covering one tile, minus one, for the basic
// split of `tiles` tiles of `ipt` iterations over g workgroups; also reports
// whether any tile is split.
static int split_peers(int64_t tiles, int64_t ipt, int64_t g, bool *any_split) {
  const int64_t I = tiles * ipt, q = I / g, r = I % g;
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
static int64_t model_grid(int64_t t, int64_t ipt, int slots, float a, float b, float c, float d) {
  const int64_t total = t * ipt;
  int64_t hi = std::min<int64_t>(slots, total);
  if (hi <= t) return t;
  double best = 1e300;
  int64_t best_g = t;
  for (int64_t g = t; g <= hi; ++g) {
    const int64_t q = total / g, r = total % g;
    const bool split = !(r == 0 && q % ipt == 0);
    const int64_t peers = split ? std::max<int64_t>(1, cdiv(ipt - 1, q)) : 0;
    const double T = a + (split ? b : 0.0) + c * (double)cdiv(total, g) + d * (double)peers;
    if (T < best - 1e-9) { best = T; best_g = g; }
  }
  return best_g;
}

int make_plan(const sk_gemm_desc &d, const sk_options &o, int slots, Plan &P) {
  std::memset(&P, 0, sizeof(P));
  if (d.m < 0 || d.n < 0 || d.k < 0) return SK_ERR_INVALID_ARG;
  if (d.dtype != SK_F32 && d.dtype != SK_F16 && d.dtype != SK_BF16) return SK_ERR_INVALID_ARG;
  if (d.layout < SK_A_ROW_B_ROW || d.layout > SK_A_COL_B_COL) return SK_ERR_INVALID_ARG;
  if (o.schedule < SK_SCHED_AUTO || o.schedule > SK_SCHED_SK_HYBRID1) return SK_ERR_INVALID_ARG;
  if (o.forced_grid < 0 || slots <= 0) return SK_ERR_INVALID_ARG;
  // 32-bit indices inside the kernels
  if (d.m > INT32_MAX / 2 || d.n > INT32_MAX / 2 || d.k > INT32_MAX / 2) return SK_ERR_UNSUPPORTED;
  P.m = d.m; P.n = d.n; P.k = d.k;
  P.dtype = d.dtype; P.layout = d.layout;
  P.cfg = tile_cfg(d.dtype);
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
  P.pack_a = !operand_direct(d.dtype, a_kmajor, d.A, d.lda, d.k);
  P.pack_b = !operand_direct(d.dtype, b_kmajor, d.B, d.ldb, d.k);
  if (P.tiles == 0 || P.ipt == 0) {  // nothing to decompose (quick-return paths)
    P.schedule = SK_SCHED_DP;
    return SK_OK;
  }
  const float ma = o.model_a > 0 ? o.model_a : c.a;
  const float mb = o.model_b > 0 ? o.model_b : c.b;
  const float mc = o.model_c > 0 ? o.model_c : c.c;
  const float md = o.model_d > 0 ? o.model_d : c.d;
  const int min_waves = o.hybrid_min_waves > 0 ? o.hybrid_min_waves : 1;

  int sched = o.schedule;
  int64_t grid = 0, sk_tiles = 0;
  if (o.forced_grid > 0) {
    sched = SK_SCHED_SK_BASIC;
    grid = o.forced_grid;
    sk_tiles = P.tiles;
  } else {
    if (sched == SK_SCHED_AUTO) {
      if (P.r == 0) {
        sched = SK_SCHED_DP;
      } else if (P.w >= min_waves) {
        // the same model decides whether giving back a wave pays for the
        // fixup: DP runs ceil(t/p) full tiles, the two-tile hybrid
        // ceil((r+p)*ipt/p) Stream-K iterations plus w-1 tiles, one partial
        // and one peer per workgroup
        const double t_dp = (double)(P.w + 1) * P.ipt;
        const double t_h2 = (double)cdiv((P.r + slots) * P.ipt, slots) + (double)(P.w - 1) * P.ipt +
                            (mb + md) / mc;
        sched = t_h2 < t_dp ? SK_SCHED_SK_HYBRID2 : SK_SCHED_DP;
      } else {
        sched = SK_SCHED_SK_BASIC;
      }
    }
    if (sched == SK_SCHED_SK_HYBRID2 && (P.w < 1 || P.r == 0))
      sched = P.r == 0 ? SK_SCHED_DP : SK_SCHED_SK_BASIC;
    switch (sched) {
      case SK_SCHED_DP:
        grid = std::min<int64_t>(P.tiles, slots);
        sk_tiles = 0;
        break;
      case SK_SCHED_SK_BASIC:
        grid = P.tiles >= slots ? slots : model_grid(P.tiles, P.ipt, slots, ma, mb, mc, md);
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
    }
  }
  if (grid > INT32_MAX / 2) return SK_ERR_UNSUPPORTED;
  P.schedule = sched;
  P.grid = (int)grid;
  P.sk_tiles = sk_tiles;
  P.dp_tiles = P.tiles - sk_tiles;
  if (sk_tiles > 0) {
    const int64_t I = sk_tiles * P.ipt;
    P.sk_q = I / grid;
    P.sk_r = I % grid;
  }
  return SK_OK;
}

int plan_max_peers(const Plan &P) {
  return P.sk_tiles > 0 ? split_peers(P.sk_tiles, P.ipt, P.grid, nullptr) : 0;
}

}  // namespace sk

using namespace sk;

extern "C" int64_t sk_plan_segments(const sk_plan *plan, int64_t x, sk_segment *out, int64_t cap) {
  if (!plan || x < 0 || cap < 0 || (cap > 0 && !out)) return SK_ERR_INVALID_ARG;
  if (x >= plan->grid) return 0;
  int64_t n = 0;
  auto push = [&](int64_t tile, int64_t lb, int64_t le, int st, int en, int64_t lp) {
    if (n < cap) out[n] = sk_segment{tile, lb, le, st, en, lp};
    ++n;
  };
  const int64_t ipt = plan->iters_per_tile, q = plan->sk_iters_q, r = plan->sk_iters_r;
  if (plan->sk_tiles > 0) {
    int64_t it = sk_first_iter(q, r, x), end = sk_first_iter(q, r, x + 1);
    while (it < end) {
      int64_t tile = it / ipt, ts = tile * ipt, te = ts + ipt;
      int64_t lb = it - ts, le = std::min(end, te) - ts;
      int st = it == ts, en = end >= te;
      int64_t lp = (st && !en) ? sk_owner_of(q, r, te - 1) : -1;
      push(tile, lb, le, st, en, lp);
      it = te;
    }
  }
  for (int64_t t = plan->sk_tiles + x; t < plan->tiles; t += plan->grid) push(t, 0, ipt, 1, 1, -1);
  return n;
}
