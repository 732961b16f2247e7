// host_emu.cpp -- the device algorithm's steps run serially on the host.
//
// Test entry points only (host_emu.h), built into their own library
// (libbef_emu.so, g++); libbef.so does not contain them.  They take HOST
// planes and follow the kernels' decisions and decomposition with the
// integer steps of ordsum.h and its shared shape constants:
//  - the general walk: exact per-row sums, a per-row plan from the exact
//    prefix (with the test flags' wrong or missing plans), row pairs from
//    segments of kPairSeg samples, each kPairLanes lane runs joined by a
//    balanced ordered tree, segments joined in row order; the plane walked
//    kWalkChunk rows at a time as stretches of rows with one plan (up to
//    kWalkMaxSeg stretches, else row by row), a stretch's pair a
//    kWalkThreads-leaf composition; a row that leaves its plan taken as
//    at most three groups of its kWalkThreads runs (apply_groups), else
//    its runs one by one under the binade S is in and the next, else its
//    terms with the one-term step;
//  - the fast path: the plan as five threshold edges (seven for planes
//    whose sum lies in the binade of 2^55), exact and closed-form
//    stretches, stretches in the binade of 2^55 as joined pairs (of rows
//    as k_pairs forms them, or of a row's lane runs), the rows and terms at
//    an edge one by one, and noise stretches as composed row pairs.
// The pages' own host test checks their twins' steps the same way, under
// correct plans and under plans broken on purpose (ADR-1497, Decision).
#include <errno.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "../../include/bef.h"
#include "host_emu.h"
#include "load_shape.h"
#include "ordsum.h"

using namespace bef;

namespace {

struct Plane {
  const void* p;
  int w, h;
  ptrdiff_t stride;
  int bpc;
  uint32_t x(int i, int j) const {
    const ptrdiff_t k = (ptrdiff_t)i * stride + j;
    return bpc == 8 ? ((const uint8_t*)p)[k] : ((const uint16_t*)p)[k];
  }
};

// Balanced ordered tree over a power-of-two number of leaves: leaf l takes
// leaf l + off for off = 1, 2, 4, ... (the shape of the kernels' shuffle
// and DPP trees, and of a block's tree over its waves).
template <class P, class Then>
P tree(std::vector<P> v, P id, Then then) {
  size_t n = 1;
  while (n < v.size()) n <<= 1;
  v.resize(n, id);
  for (size_t off = 1; off < n; off <<= 1)
    for (size_t l = 0; l + off < n; l += 2 * off) v[l] = then(v[l], v[l + off]);
  return v[0];
}
Pair64 tree64(const std::vector<Pair64>& v, int sh) {
  return tree(v, pair64_id(), [&](Pair64 a, Pair64 b) { return then64(a, b, sh); });
}
Pair32 tree32(const std::vector<Pair32>& v, int sh) {
  return tree(v, pair32_id(), [&](Pair32 a, Pair32 b) { return then32(a, b, sh); });
}

// A composite of items [a, b) the way a walk block forms it: thread t of
// kWalkThreads folds items [a + t*c, a + t*c + c) in order (c = ceil((b -
// a) / kWalkThreads)), then the threads' composites go through a balanced
// tree (64 lanes a wave, then the waves).
template <class PairOf>
Pair64 block_compose(int a, int b, int sh, PairOf pair_of) {
  const int c = (b - a + kWalkThreads - 1) / kWalkThreads;
  std::vector<Pair64> leaves(kWalkThreads, pair64_id());
  for (int t = 0; t < kWalkThreads; ++t) {
    Pair64 acc = pair64_id();
    for (int k = a + t * c; k < a + (t + 1) * c && k < b; ++k) acc = then64(acc, pair_of(k), sh);
    leaves[t] = acc;
  }
  return tree64(leaves, sh);
}

// Row i's pair under binade e as k_pairs forms it: segments of kPairSeg
// samples, each split into kPairLanes runs of ceil(n / kPairLanes) terms
// (each added from both starts with the double add) joined by a balanced
// tree, the segments joined in row order, widened with the row's exact sum.
Pair64 kpairs_row_pair(const Plane& pl, int i, int e, uint64_t Ri) {
  const int sh = e - 52, w = pl.w;
  Pair32 acc = pair32_id();
  for (int s0 = 0; s0 < w; s0 += kPairSeg) {
    const int n = std::min(kPairSeg, w - s0), L = (n + kPairLanes - 1) / kPairLanes;
    std::vector<Pair32> lanes(kPairLanes);
    for (int l = 0; l < kPairLanes; ++l) {
      const int j0 = std::min(l * L, n), j1 = std::min(j0 + L, n);
      lanes[l] = run_pair([&](int j) { return (double)fsq_units(pl.x(i, s0 + j0 + j)); }, j1 - j0, e);
    }
    acc = then32(acc, tree32(lanes, sh), sh);
  }
  return widen_pair(acc, Ri);
}

struct Emu {
  Plane pl;
  unsigned dbg;
  std::vector<uint64_t> R, C;
  std::vector<int> plan;
  std::vector<Pair64> pair;

  uint32_t T(int i, int j) const { return fsq_units(pl.x(i, j)); }

  // Row pair under binade e: the closed form in the binades of 2^53 and
  // 2^54; otherwise the row pair kernel's: segments of kPairSeg samples,
  // each split into kPairLanes runs of ceil(n / kPairLanes) terms (each
  // added from both starts with the double add) joined by a balanced tree,
  // the segments joined in row order, widened with the row's exact sum.
  Pair64 row_pair(int i, int e) const {
    if (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM)) return closed_pair(R[i], C[i], e);
    return kpairs_row_pair(pl, i, e, R[i]);
  }

  uint64_t terms(uint64_t s, int i, int j0, int j1) const {
    for (int j = j0; j < j1; ++j) s = rne53_add(s, T(i, j));
    return s;
  }

  // Items [0, n) with plans, exact sums and odd counts, from s: stretches
  // of equal plan (at most kWalkMaxSeg of them, else item by item), a
  // stretch exact, or one pair inside its binade (closed form, or the
  // items' pairs composed as a block does), else item by item.
  template <class PlanOf, class EOf, class COf, class PairOf, class Step>
  uint64_t walk_items(uint64_t s, int n, PlanOf plan_at, EOf e_at, COf c_at, PairOf pair_at,
                      Step step) const {
    std::vector<int> starts;
    for (int k = 0; k < n; ++k)
      if (k == 0 || plan_at(k) != plan_at(k - 1)) starts.push_back(k);
    if ((int)starts.size() > kWalkMaxSeg) {
      for (int k = 0; k < n; ++k) s = step(s, k);
      return s;
    }
    starts.push_back(n);
    for (size_t g = 0; g + 1 < starts.size(); ++g) {
      const int a = starts[g], b = starts[g + 1], e = plan_at(a);
      uint64_t E = 0, Cn = 0;
      for (int k = a; k < b; ++k) E += e_at(k), Cn += c_at(k);
      bool done = false;
      if (e == kPlanExact) {
        done = try_exact(&s, E);
      } else if (e >= 53 && !(dbg & BEF_DBG_NO_STRETCH)) {
        const Pair64 p = (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM))
                             ? closed_pair(E, Cn, e)
                             : block_compose(a, b, e - 52, [&](int k) { return pair_at(k, e); });
        done = try_apply(&s, p, e);
      }
      if (!done)
        for (int k = a; k < b; ++k) s = step(s, k);
    }
    return s;
  }

  // A row that leaves its plan, by groups of runs: kWalkThreads runs of
  // ceil(w / kWalkThreads) terms, each given a group from its plan (exact
  // sum, exact prefix from S, the row's margin); the runs of groups in a
  // binade from 2^55 up give pairs joined as the walk block joins them (a
  // balanced tree per wave, then the waves in order); apply_groups does
  // the rest.  False when the runs do not form the groups in order.
  bool row_groups(uint64_t* sp, int i) const {
    const int w = pl.w;
    const uint64_t s0 = *sp;
    const bool low = s0 < kTwo53;
    const int eA = low ? 53 : binade(s0), eB = eA + 1, e2 = low ? eA : eB;
    const int L = (w + kWalkThreads - 1) / kWalkThreads, nr = (w + L - 1) / L;
    std::vector<uint64_t> E(kWalkThreads), c(kWalkThreads), Q(kWalkThreads), QC(kWalkThreads);
    std::vector<int> g(kWalkThreads, 3);
    uint64_t tot = 0, totc = 0;
    for (int t = 0; t < kWalkThreads; ++t) {
      const int j0 = std::min(t * L, w), j1 = std::min(j0 + L, w);
      E[t] = c[t] = 0;
      for (int j = j0; j < j1; ++j) E[t] += T(i, j), c[t] += T(i, j) & 1u;
      Q[t] = tot;
      QC[t] = totc;
      tot += E[t];
      totc += c[t];
    }
    for (int t = 0; t < nr; ++t) {
      const int p = plan_of(s0 + Q[t], E[t], (uint64_t)w << (eB - 53));
      g[t] = p == kPlanCross ? 1 : (p == (low ? kPlanExact : eA)) ? 0 : p == e2 ? 2 : 3;
    }
    GroupStart G[4] = {{0, 0, -1}, {0, 0, -1}, {0, 0, -1}, {tot, totc, nr}};
    for (int t = 0; t < nr; ++t) {
      const int gp = t > 0 ? g[t - 1] : -1;
      if (g[t] == 3 || gp > g[t]) return false;
      if (gp != g[t]) G[g[t]] = GroupStart{Q[t], QC[t], t};
    }
    const bool tree0 = !low && eA >= 55, tree2 = e2 >= 55;
    Pair64 c0 = pair64_id(), c2 = pair64_id();
    if (tree0 || tree2) {
      std::vector<Pair64> l0(kWalkThreads, pair64_id()), l2(kWalkThreads, pair64_id());
      for (int t = 0; t < kWalkThreads; ++t) {
        if (!((g[t] == 0 && tree0) || (g[t] == 2 && tree2))) continue;
        const int e = g[t] == 0 ? eA : e2, j0 = std::min(t * L, w), j1 = std::min(j0 + L, w);
        const Pair64 pr =
            widen_pair(run_pair([&](int j) { return (double)T(i, j0 + j); }, j1 - j0, e), E[t]);
        (g[t] == 0 ? l0 : l2)[t] = pr;
      }
      for (int wv = 0; wv < kWalkThreads / 64; ++wv) {
        const std::vector<Pair64> w0(l0.begin() + 64 * wv, l0.begin() + 64 * wv + 64);
        const std::vector<Pair64> w2(l2.begin() + 64 * wv, l2.begin() + 64 * wv + 64);
        // a wave composes only the groups it has a tree for
        const Pair64 q0 = tree0 ? tree64(w0, eA - 52) : pair64_id();
        const Pair64 q2 = tree2 ? tree64(w2, e2 - 52) : pair64_id();
        c0 = wv == 0 ? q0 : then64(c0, q0, eA - 52);
        c2 = wv == 0 ? q2 : then64(c2, q2, e2 - 52);
      }
    }
    return apply_groups(
        sp, G, low, eA,
        [&](uint64_t s, int ra, int rb) { return terms(s, i, ra * L, std::min(rb * L, w)); },
        [&](int k, int e, uint64_t Eg, uint64_t Cg) {
          return e <= 54 ? closed_pair(Eg, Cg, e) : (k == 0 ? c0 : c2);
        });
  }

  // A row that leaves its plan: its terms one by one (test flag), else its
  // groups of runs, else its kWalkThreads runs planned from their own exact
  // prefix with pairs under the binade S is in (eA) and the next (eB),
  // walked as stretches; a run that fits neither goes term by term.
  uint64_t fallback_row(uint64_t s, int i) const {
    const int w = pl.w;
    if (dbg & BEF_DBG_TERMS_ONLY) return terms(s, i, 0, w);
    if (!(dbg & (BEF_DBG_NO_STRETCH | BEF_DBG_NO_CLOSED_FORM))) {
      uint64_t s2 = s;
      if (row_groups(&s2, i)) return s2;
    }
    const int eA = s < kTwo53 ? 53 : binade(s), eB = eA + 1;
    const int L = (w + kWalkThreads - 1) / kWalkThreads;
    std::vector<uint64_t> E(kWalkThreads), c(kWalkThreads);
    std::vector<Pair64> pA(kWalkThreads), pB(kWalkThreads);
    std::vector<int> rp(kWalkThreads), j0(kWalkThreads), j1(kWalkThreads);
    uint64_t q = s;
    const uint64_t Mr = (uint64_t)w << (eB - 53);
    for (int t = 0; t < kWalkThreads; ++t) {
      j0[t] = std::min(t * L, w);
      j1[t] = std::min(j0[t] + L, w);
      E[t] = c[t] = 0;
      for (int j = j0[t]; j < j1[t]; ++j) E[t] += T(i, j), c[t] += T(i, j) & 1u;
      for (int qq = 0; qq < 2; ++qq) {
        const int e = qq ? eB : eA;
        const Pair64 p =
            (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM))
                ? closed_pair(E[t], c[t], e)
                : widen_pair(run_pair([&](int j) { return (double)T(i, j0[t] + j); }, j1[t] - j0[t],
                                      e),
                             E[t]);
        (qq ? pB : pA)[t] = p;
      }
      rp[t] = plan_of(q, E[t], Mr);
      q += E[t];
    }
    return walk_items(
        s, kWalkThreads, [&](int t) { return rp[t]; }, [&](int t) { return E[t]; },
        [&](int t) { return c[t]; }, [&](int t, int e) { return e == eA ? pA[t] : pB[t]; },
        [&](uint64_t s2, int t) {
          if (try_exact(&s2, E[t])) return s2;
          if (try_apply(&s2, pA[t], eA)) return s2;
          if (try_apply(&s2, pB[t], eB)) return s2;
          return terms(s2, i, j0[t], j1[t]);
        });
  }

  void run(uint64_t out[3]) {
    const int h = pl.h, w = pl.w;
    R.assign(h, 0);
    C.assign(h, 0);
    plan.assign(h, kPlanExact);
    pair.assign(h, pair64_id());
    std::vector<uint64_t> P(h, 0);
    uint64_t s1 = 0, tot = 0;
    for (int i = 0; i < h; ++i) {
      for (int j = 0; j < w; ++j) {
        s1 += pl.x(i, j);
        R[i] += T(i, j);
        C[i] += T(i, j) & 1u;
      }
      P[i] = tot;
      tot += R[i];
    }
    out[0] = s1;
    out[1] = tot;
    if (tot <= kTwo53 && !(dbg & BEF_DBG_FORCE_ROUND)) {
      out[2] = tot;
      return;
    }
    const uint64_t M = tot > kTwo53 ? (uint64_t)w * h << (binade(tot) - 53) : 0;
    for (int i = 0; i < h; ++i) {
      int e = plan_of(P[i], R[i], M);
      if (e >= 53 && (dbg & BEF_DBG_PLAN_NONE)) e = kPlanCross;
      if (e >= 53 && (dbg & BEF_DBG_PLAN_WRONG)) e = (i & 1) ? (e > 53 ? e - 1 : e + 2) : e + 1;
      plan[i] = e;
      if (e >= 55 || (e >= 53 && (dbg & BEF_DBG_NO_CLOSED_FORM))) pair[i] = row_pair(i, e);
    }
    // the walk block takes the plane kWalkChunk rows at a time
    uint64_t s = 0;
    for (int a = 0; a < h; a += kWalkChunk) {
      const int n = std::min(kWalkChunk, h - a);
      s = walk_items(
          s, n, [&](int k) { return plan[a + k]; }, [&](int k) { return R[a + k]; },
          [&](int k) { return C[a + k]; },
          [&](int k, int e) {
            return (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM)) ? closed_pair(R[a + k], C[a + k], e)
                                                                : pair[a + k];
          },
          [&](uint64_t s2, int k) {
            const int i = a + k, e = plan[i];
            if (try_exact(&s2, R[i])) return s2;
            if (e >= 53 &&
                try_apply(&s2,
                          (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM)) ? closed_pair(R[i], C[i], e)
                                                                       : pair[i],
                          e))
              return s2;
            return fallback_row(s2, i);
          });
    }
    out[2] = s;
  }
};

// ---------------------------------------------------------------------------
// The fast path's decisions, serially: each edge of the plan is the first
// item meeting its condition (edge_conds), then the segments in order --
// exact adds, closed-form pairs, and the items across an edge one by one.
// The device finds the same first items with lane chunks and a second
// scan; the decisions and every arithmetic step are these.

template <int NE = kEdges>
struct Edges {
  int x[NE + 1];
  uint64_t P[NE + 1], PC[NE + 1];
};

template <int NE = kEdges, class EAt, class CAt>
Edges<NE> first_items(int n, uint64_t base, uint64_t M, EAt e_at, CAt c_at) {
  Edges<NE> r;
  uint64_t q = base, qc = 0;
  unsigned seen = 0;
  for (int j = 0; j <= NE; ++j) r.x[j] = n;
  for (int k = 0; k < n; ++k) {
    const uint64_t e = e_at(k);
    const unsigned now = edge_conds<NE>(q, q + e, M), fresh = now & ~seen;
    for (int j = 0; j < NE; ++j)
      if ((fresh >> j) & 1u) r.x[j] = k, r.P[j] = q, r.PC[j] = qc;
    seen |= now;
    q += e;
    qc += c_at(k);
  }
  for (int j = 0; j <= NE; ++j)
    if (r.x[j] == n) r.P[j] = q, r.PC[j] = qc;
  return r;
}

struct Fast {
  Plane pl;
  std::vector<uint64_t> R, C;

  uint32_t T(int i, int j) const { return fsq_units(pl.x(i, j)); }

  // A row across an edge: its terms' edges from the actual S with margin
  // w * u/2, closed forms, and the terms at an edge by the one-term step;
  // with seven edges, the row's part inside the binade of 2^55 as the pair
  // of the lanes' runs of the staged row (lane l: 8-sample chunks [l*cpl,
  // l*cpl + cpl)) joined by a balanced tree.
  template <int NE>
  bool cross_row(uint64_t* sp, int i) const {
    const uint64_t s0 = *sp;
    const int eB = (s0 < kTwo53 ? 53 : binade(s0)) + 1;
    const uint64_t Mr = (uint64_t)pl.w << (eB - 53);
    const Edges<NE> ed = first_items<NE>(
        pl.w, s0, Mr, [&](int k) { return (uint64_t)T(i, k); },
        [&](int k) { return (uint64_t)(T(i, k) & 1u); });
    uint64_t s = s0, Pa = s0, PCa = 0;
    int a = 0;
    for (int g = 0; g <= NE; ++g) {
      const int b = ed.x[g];
      if (b < a) return false;
      if (b > a) {
        if (g == 1 || g == 3 || (NE == kEdges56 && g == 5)) {
          for (int k = a; k < b; ++k) s = rne53_add(s, T(i, k));
        } else if (NE == kEdges56 && g == 6) {
          const int L = 8 * ((((pl.w + 7) >> 3) + 63) >> 6);
          std::vector<Pair64> lanes(64, pair64_id());
          for (int l = 0; l < 64; ++l) {
            const int j0 = std::max(std::min(l * L, pl.w), a);
            const int j1 = std::min(std::min(l * L + L, pl.w), b);
            if (j1 <= j0) continue;
            uint64_t E = 0;
            for (int k = j0; k < j1; ++k) E += T(i, k);
            lanes[l] = widen_pair(run_pair([&](int j) { return (double)T(i, j0 + j); }, j1 - j0, 55), E);
          }
          if (!try_apply(&s, tree64(lanes, 3), 55)) return false;
        } else if (!fast_apply<NE>(&s, g, ed.P[g] - Pa, ed.PC[g] - PCa)) {
          return false;
        }
      }
      a = b;
      Pa = ed.P[g];
      PCa = ed.PC[g];
    }
    *sp = s;
    return true;
  }

  // The walk with NE edges; the stretch inside the binade of 2^55 composes
  // the rows' pairs as k_pairs forms them, lane l joining rows [a + l*rs,
  // ...) in order, then a balanced tree over the lanes.
  template <int NE>
  void walk(uint64_t out[3]) const {
    const int h = pl.h, w = pl.w;
    const uint64_t M = (NE == kEdges56 ? 4ull : 2ull) * (uint64_t)w * (uint64_t)h;
    const Edges<NE> ed = first_items<NE>(
        h, 0, M, [&](int k) { return R[k]; }, [&](int k) { return C[k]; });
    out[0] = 0;
    out[2] = ed.P[NE];
    if (ed.P[NE] >= (NE == kEdges56 ? (1ull << 56) : (1ull << 55))) return;
    uint64_t s = 0, Pa = 0, PCa = 0;
    int a = 0;
    for (int g = 0; g <= NE; ++g) {
      const int b = ed.x[g];
      if (b < a) return;
      if (b > a) {
        if (g == 1 || g == 3 || (NE == kEdges56 && g == 5)) {
          for (int i = a; i < b; ++i) {
            if (try_exact(&s, R[i])) continue;
            if (s >= kTwo53) {
              const int e = binade(s);
              if (e <= 54 && try_apply(&s, closed_pair(R[i], C[i], e), e)) continue;
            }
            if (!cross_row<NE>(&s, i)) return;
          }
        } else if (NE == kEdges56 && g == 6) {
          const int rs = (b - a + 63) >> 6;
          std::vector<Pair64> lanes(64, pair64_id());
          for (int l = 0; l < 64; ++l)
            for (int i = std::min(a + l * rs, b); i < std::min(a + l * rs + rs, b); ++i)
              lanes[l] = then64(lanes[l], kpairs_row_pair(pl, i, 55, R[i]), 3);
          if (!try_apply(&s, tree64(lanes, 3), 55)) return;
        } else if (!fast_apply<NE>(&s, g, ed.P[g] - Pa, ed.PC[g] - PCa)) {
          return;
        }
      }
      a = b;
      Pa = ed.P[g];
      PCa = ed.PC[g];
    }
    out[0] = 1;
    out[1] = s;
  }

  // out = {handled, S_cpu, S_exact}: five edges below 2^55, seven for a
  // plane whose exact sum lies in [2^55, 2^56), as the device chooses from
  // the plan kernel's plane sum.
  void run(uint64_t out[3]) {
    const int h = pl.h, w = pl.w;
    R.assign(h, 0);
    C.assign(h, 0);
    uint64_t total = 0;
    for (int i = 0; i < h; ++i) {
      for (int j = 0; j < w; ++j) {
        R[i] += T(i, j);
        C[i] += T(i, j) & 1u;
      }
      total += R[i];
    }
    if (total >= (1ull << 55)) walk<kEdges56>(out);
    else walk<kEdges>(out);
  }
};

// The fast PSNR noise: rows' exact sums, the same edges with margin 2 per
// row, exact rows as integers, rows at an edge by the one-term step, and
// each stretch inside one binade as the composed pair of its rows (any
// grouping: composition is associative).  out = {handled, bits of the
// double in units, exact sum}.
void fast_noise(const Plane& r, const Plane& d, uint64_t out[3]) {
  const int h = r.h;
  std::vector<uint64_t> RN(h, 0);
  for (int i = 0; i < h; ++i)
    for (int j = 0; j < r.w; ++j) {
      const int32_t a = (int32_t)r.x(i, j) - (int32_t)d.x(i, j);
      RN[i] += fsq_units((uint32_t)(a < 0 ? -a : a));
    }
  const Edges ed = first_items(
      h, 0, 2ull * (uint64_t)h, [&](int k) { return RN[k]; }, [&](int) { return (uint64_t)0; });
  out[0] = 0;
  out[2] = ed.P[kEdges];
  if (ed.P[kEdges] >= (1ull << 55)) return;
  uint64_t s = 0, Pa = 0;
  int a = 0;
  for (int g = 0; g <= kEdges; ++g) {
    const int b = ed.x[g];
    if (b < a) return;
    if (b > a) {
      const int ep = fast_plan(g);
      if (ep == kPlanExact) {
        if (!try_exact(&s, ed.P[g] - Pa)) return;
      } else if (ep == kPlanCross) {
        for (int i = a; i < b; ++i) s = rne53_add(s, RN[i]);
      } else if (ep == 53 || ep == 54) {
        const int sh = ep - 52;
        Pair64 acc = pair64_id();
        for (int i = a; i < b; ++i) acc = then64(acc, noise_row_pair(RN[i], sh), sh);
        if (!try_apply(&s, acc, ep)) return;
      } else {
        return;
      }
    }
    a = b;
    Pa = ed.P[g];
  }
  const double v = (double)s;
  uint64_t bits;
  __builtin_memcpy(&bits, &v, 8);
  out[0] = 1;
  out[1] = bits;
}

bool bad(const void* a, int w, int h, ptrdiff_t stride, int bpc) {
  return !a || w <= 0 || h <= 0 || w > 32768 || h > 32768 || stride < w || bpc < 8 || bpc > 16;
}

}  // namespace

extern "C" int bef_host_plane_units(const void* plane, int w, int h, ptrdiff_t stride, int bpc,
                                    unsigned dbg_flags, uint64_t out[3]) {
  if (bad(plane, w, h, stride, bpc) || !out) return -EINVAL;
  Emu em{Plane{plane, w, h, stride, bpc}, dbg_flags, {}, {}, {}, {}};
  em.run(out);
  return 0;
}

extern "C" int bef_host_noise_units(const void* ref, const void* dis, int w, int h,
                                    ptrdiff_t stride, int bpc, uint64_t* bits, uint64_t* exact) {
  if (bad(ref, w, h, stride, bpc) || !dis || !bits || !exact) return -EINVAL;
  Plane r{ref, w, h, stride, bpc}, d{dis, w, h, stride, bpc};
  uint64_t tot = 0;
  volatile double acc = 0.0;
  for (int i = 0; i < h; ++i) {
    uint64_t row = 0;
    for (int j = 0; j < w; ++j) {
      const int32_t a = (int32_t)r.x(i, j) - (int32_t)d.x(i, j);
      row += fsq_units((uint32_t)(a < 0 ? -a : a));
    }
    tot += row;
    acc = acc + (double)row;  // rows added into one double, in order
  }
  const double v = acc;
  uint64_t b;
  __builtin_memcpy(&b, &v, 8);
  *bits = b;
  *exact = tot;
  return 0;
}

extern "C" int bef_host_fast_units(const void* plane, int w, int h, ptrdiff_t stride, int bpc,
                                   uint64_t out[3]) {
  if (bad(plane, w, h, stride, bpc) || !out) return -EINVAL;
  Fast f{Plane{plane, w, h, stride, bpc}, {}, {}};
  f.run(out);
  return 0;
}

extern "C" int bef_host_fast_noise(const void* ref, const void* dis, int w, int h,
                                   ptrdiff_t stride, int bpc, uint64_t out[3]) {
  if (bad(ref, w, h, stride, bpc) || !dis || !out) return -EINVAL;
  fast_noise(Plane{ref, w, h, stride, bpc}, Plane{dis, w, h, stride, bpc}, out);
  return 0;
}

extern "C" uint64_t bef_host_rne53_add(uint64_t s, uint64_t t) { return rne53_add(s, t); }

extern "C" int bef_host_load_shape(const void* ref, const void* dis, int w, ptrdiff_t stride,
                                   ptrdiff_t frame_pitch, int nframes, int out[2]) {
  if (!out || w <= 0 || nframes <= 0) return -EINVAL;
  load_shape(ref, dis, w, stride, frame_pitch, nframes, &out[0], &out[1]);
  return 0;
}

extern "C" int bef_host_run_pair(const uint32_t* terms, int n, int e, uint64_t out[2]) {
  if (!terms || n < 0 || n > 32768 || e < 53 || e > 62 || !out) return -EINVAL;
  uint64_t E = 0;
  for (int j = 0; j < n; ++j) E += terms[j];
  const Pair64 p = widen_pair(run_pair([&](int j) { return (double)terms[j]; }, n, e), E);
  out[0] = p.a0;
  out[1] = p.a1;
  return 0;
}
