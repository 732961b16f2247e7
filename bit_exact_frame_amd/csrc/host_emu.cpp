// host_emu.cpp -- the device algorithm's steps run serially on the host.
//
// Test entry points only (bef_host_*): they take HOST planes and follow the
// same decisions as the kernels, with the integer steps of ordsum.h.  The
// fast path: the plan as five threshold edges, exact and closed-form
// segments, rows and terms at an edge one by one, noise stretches as
// composed row pairs.  The general walk: exact per-row sums, a per-row plan
// from the exact prefix, row pairs from 64 lane runs joined by an ordered
// tree, a walk over stretches of rows with the same plan, a fallback of
// each unfit row to 256 runs (planned by their own exact prefix) and of
// each unfit run to single terms -- with the integer steps of ordsum.h.
// The pages' own host test does the same with the twins' steps (ADR-1497,
// Decision: the host test runs the kernels' steps against the CPU loop,
// with real and with deliberately wrong plans).  Nothing on the product
// path calls this file.
#include <errno.h>
#include <stdint.h>
#include <stdlib.h>

#include <vector>

#include "../../include/bef.h"
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

// Balanced ordered tree over leaves (the shape of a shuffle-down tree).
Pair64 tree64(std::vector<Pair64> v, int sh) {
  if (v.empty()) return pair64_id();
  size_t n = 1;
  while (n < v.size()) n <<= 1;
  v.resize(n, pair64_id());
  for (size_t off = 1; off < n; off <<= 1)
    for (size_t l = 0; l + off < n; l += 2 * off) v[l] = then64(v[l], v[l + off], sh);
  return v[0];
}
Pair32 tree32(std::vector<Pair32> v, int sh) {
  if (v.empty()) return pair32_id();
  size_t n = 1;
  while (n < v.size()) n <<= 1;
  v.resize(n, pair32_id());
  for (size_t off = 1; off < n; off <<= 1)
    for (size_t l = 0; l + off < n; l += 2 * off) v[l] = then32(v[l], v[l + off], sh);
  return v[0];
}

// Composite of items [a, b) the way a 256-thread block forms it: each
// thread folds a contiguous chunk in order, then an ordered tree.
template <class PairOf>
Pair64 block_compose(int a, int b, int sh, PairOf pair_of) {
  const int n = b - a;
  const int c = (n + 255) / 256;
  std::vector<Pair64> leaves(256, pair64_id());
  for (int t = 0; t < 256; ++t) {
    Pair64 acc = pair64_id();
    for (int k = a + t * c; k < a + (t + 1) * c && k < b; ++k) acc = then64(acc, pair_of(k), sh);
    leaves[t] = acc;
  }
  return tree64(leaves, sh);
}

struct Emu {
  Plane pl;
  unsigned dbg;
  std::vector<uint64_t> R, P, C;
  std::vector<int> plan;
  std::vector<Pair64> pair;

  uint32_t T(int i, int j) const { return fsq_units(pl.x(i, j)); }

  // Row pair under binade e.  In the binades of 2^53 and 2^54 it follows
  // from the row's exact sum and its count of odd float squares (every
  // float square in units is 0 or 1 mod 4: see the walk kernel); otherwise
  // 64 lane runs of ceil(w/64) terms, each a two-trajectory fold, joined by
  // an ordered tree and widened with R.
  Pair64 row_pair(int i, int e) const {
    if (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM)) return closed_pair(R[i], C[i], e);
    const int sh = e - 52;
    const int L = (pl.w + 63) / 64;
    std::vector<Pair32> lanes(64);
    for (int l = 0; l < 64; ++l) {
      const int s0 = l * L;
      const int n = s0 >= pl.w ? 0 : (s0 + L <= pl.w ? L : pl.w - s0);
      lanes[l] = run_pair([&](int j) { return T(i, s0 + j); }, n, sh);
    }
    return widen_pair(tree32(lanes, sh), R[i]);
  }

  uint64_t terms(uint64_t s, int i, int j0, int j1) const {
    for (int j = j0; j < j1; ++j) s = rne53_add(s, T(i, j));
    return s;
  }

  // Generic walk over items with plans (stretches first, then item steps).
  template <class PlanOf, class EOf, class PairOf, class Step>
  uint64_t walk(uint64_t s, int n, PlanOf plan_of_item, EOf e_of, PairOf pair_of,
                Step step) const {
    int i = 0;
    while (i < n) {
      const int e = plan_of_item(i);
      int j = i + 1;
      while (j < n && plan_of_item(j) == e) ++j;
      bool done = false;
      if (e == kPlanExact) {
        uint64_t E = 0;
        for (int k = i; k < j; ++k) E += e_of(k);
        done = try_exact(&s, E);
      } else if (e >= 53 && !(dbg & BEF_DBG_NO_STRETCH)) {
        done = try_apply(&s, block_compose(i, j, e - 52, pair_of), e);
      }
      if (!done)
        for (int k = i; k < j; ++k) s = step(s, k);
      i = j;
    }
    return s;
  }

  // A row the plan does not fit: 256 runs under the binade S is in and the
  // next one, planned from their own exact prefix; unfit runs by terms.
  uint64_t fallback_row(uint64_t s, int i) const {
    if (dbg & BEF_DBG_TERMS_ONLY) return terms(s, i, 0, pl.w);
    const int eA = (s < kTwo53) ? 53 : binade(s);
    const int eB = eA + 1;
    const int L = (pl.w + 255) / 256;
    std::vector<uint64_t> E(256), Q(256);
    std::vector<Pair64> pA(256), pB(256);
    std::vector<int> rp(256);
    std::vector<int> j0(256), j1(256);
    uint64_t q = s;
    const uint64_t Mr = (uint64_t)pl.w << (eB - 53);
    for (int t = 0; t < 256; ++t) {
      j0[t] = t * L < pl.w ? t * L : pl.w;
      j1[t] = t * L + L < pl.w ? t * L + L : pl.w;
      uint64_t e = 0;
      for (int j = j0[t]; j < j1[t]; ++j) e += T(i, j);
      E[t] = e;
      auto tt = [&](int j) { return T(i, j0[t] + j); };
      pA[t] = widen_pair(run_pair(tt, j1[t] - j0[t], eA - 52), e);
      pB[t] = widen_pair(run_pair(tt, j1[t] - j0[t], eB - 52), e);
      Q[t] = q;
      rp[t] = plan_of(q, e, Mr);
      q += e;
    }
    return walk(
        s, 256, [&](int t) { return rp[t]; }, [&](int t) { return E[t]; },
        [&](int t) { return rp[t] == eA ? pA[t] : pB[t]; },
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
    P.assign(h, 0);
    C.assign(h, 0);
    plan.assign(h, kPlanExact);
    pair.assign(h, pair64_id());
    uint64_t s1 = 0, tot = 0;
    for (int i = 0; i < h; ++i) {
      uint64_t r = 0;
      uint64_t c = 0;
      for (int j = 0; j < w; ++j) {
        s1 += pl.x(i, j);
        r += T(i, j);
        c += T(i, j) & 1u;
      }
      R[i] = r;
      C[i] = c;
      P[i] = tot;
      tot += r;
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
      if (e >= 53) pair[i] = row_pair(i, e);
    }
    out[2] = walk(
        0, h, [&](int i) { return plan[i]; }, [&](int i) { return R[i]; },
        [&](int i) { return pair[i]; },
        [&](uint64_t s, int i) {
          if (try_exact(&s, R[i])) return s;
          if (try_apply(&s, pair[i], plan[i])) return s;
          return fallback_row(s, i);
        });
  }
};

// ---------------------------------------------------------------------------
// The fast path's decisions, serially: each edge of the plan is the first
// item meeting its condition (edge_conds), then the segments in order --
// exact adds, closed-form pairs, and the items across an edge one by one.
// The device finds the same first items with lane chunks and a second
// scan; the decisions and every arithmetic step are these.

struct Edges {
  int x[kEdges + 1];
  uint64_t P[kEdges + 1], PC[kEdges + 1];
};

template <class EAt, class CAt>
Edges first_items(int n, uint64_t base, uint64_t M, EAt e_at, CAt c_at) {
  Edges r;
  uint64_t q = base, qc = 0;
  unsigned seen = 0;
  for (int j = 0; j <= kEdges; ++j) r.x[j] = n;
  for (int k = 0; k < n; ++k) {
    const uint64_t e = e_at(k);
    const unsigned now = edge_conds(q, q + e, M), fresh = now & ~seen;
    for (int j = 0; j < kEdges; ++j)
      if ((fresh >> j) & 1u) r.x[j] = k, r.P[j] = q, r.PC[j] = qc;
    seen |= now;
    q += e;
    qc += c_at(k);
  }
  for (int j = 0; j <= kEdges; ++j)
    if (r.x[j] == n) r.P[j] = q, r.PC[j] = qc;
  return r;
}

struct Fast {
  Plane pl;
  std::vector<uint64_t> R, C;

  uint32_t T(int i, int j) const { return fsq_units(pl.x(i, j)); }

  // A row across an edge: its terms' edges from the actual S with margin
  // w * u/2, closed forms, and the terms at an edge by the one-term step.
  bool cross_row(uint64_t* sp, int i) const {
    const uint64_t s0 = *sp;
    const int eB = (s0 < kTwo53 ? 53 : binade(s0)) + 1;
    const uint64_t Mr = (uint64_t)pl.w << (eB - 53);
    const Edges ed = first_items(
        pl.w, s0, Mr, [&](int k) { return (uint64_t)T(i, k); },
        [&](int k) { return (uint64_t)(T(i, k) & 1u); });
    uint64_t s = s0, Pa = s0, PCa = 0;
    int a = 0;
    for (int g = 0; g <= kEdges; ++g) {
      const int b = ed.x[g];
      if (b < a) return false;
      if (b > a) {
        if (g == 1 || g == 3) {
          for (int k = a; k < b; ++k) s = rne53_add(s, T(i, k));
        } else if (!fast_apply(&s, g, ed.P[g] - Pa, ed.PC[g] - PCa)) {
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

  // out = {handled, S_cpu, S_exact}
  void run(uint64_t out[3]) {
    const int h = pl.h, w = pl.w;
    R.assign(h, 0);
    C.assign(h, 0);
    for (int i = 0; i < h; ++i)
      for (int j = 0; j < w; ++j) {
        R[i] += T(i, j);
        C[i] += T(i, j) & 1u;
      }
    const Edges ed = first_items(
        h, 0, 2ull * (uint64_t)w * (uint64_t)h, [&](int k) { return R[k]; },
        [&](int k) { return C[k]; });
    out[0] = 0;
    out[2] = ed.P[kEdges];
    if (ed.P[kEdges] >= (1ull << 55)) return;
    uint64_t s = 0, Pa = 0, PCa = 0;
    int a = 0;
    for (int g = 0; g <= kEdges; ++g) {
      const int b = ed.x[g];
      if (b < a) return;
      if (b > a) {
        if (g == 1 || g == 3) {
          for (int i = a; i < b; ++i) {
            if (try_exact(&s, R[i])) continue;
            if (s >= kTwo53) {
              const int e = binade(s);
              if (e <= 54 && try_apply(&s, closed_pair(R[i], C[i], e), e)) continue;
            }
            if (!cross_row(&s, i)) return;
          }
        } else if (!fast_apply(&s, g, ed.P[g] - Pa, ed.PC[g] - PCa)) {
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
  Emu em{Plane{plane, w, h, stride, bpc}, dbg_flags, {}, {}, {}, {}, {}};
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

extern "C" int bef_host_run_pair(const uint32_t* terms, int n, int e, uint64_t out[2]) {
  if (!terms || n < 0 || n > 32768 || e < 53 || e > 62 || !out) return -EINVAL;
  uint64_t E = 0;
  for (int j = 0; j < n; ++j) E += terms[j];
  const Pair64 p = widen_pair(run_pair([&](int j) { return terms[j]; }, n, e - 52), E);
  out[0] = p.a0;
  out[1] = p.a1;
  return 0;
}
