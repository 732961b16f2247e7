// ordsum.h -- integer steps of the CPU's double accumulation, in units.
//
// Everything here counts in units of 1/s^2 (s = 2^(bpc-8)), where every
// second-moment or noise term is an integer below 2^32 and every running sum
// of the CPU's double loop is an integer (ADR-1497, Decision; ADR-1499,
// Decision, argument step 1).  Shared by the HIP kernels and the host
// emulation of their algorithm; the CPU oracle never includes it.
//
// Facts used (ADR-1497, Decision):
//  * One CPU step S <- fl64(S + t) is, in units, the exact integer S + t
//    rounded to 53 significant bits, ties to even.
//  * Binade e (S in [2^e, 2^(e+1)), e >= 53) has last place u = 2^(e-52);
//    there S is a multiple of u and adding t moves S by t rounded to a
//    multiple of u, a tie going to the multiple that leaves S/u even.
//  * A run of terms added inside one binade is therefore described by two
//    increments, one for each parity of S/u at its start; two runs compose
//    associatively, in order (not commutatively).
//
// Representation: a "pair" {a0, a1} holds the increment a run applies to S
// when S/u is even (a0) or odd (a1).  Inside a lane the increments are kept
// modulo 2^32 (they differ from the run's exact sum by less than 2^31, so
// the exact sum restores them); across rows they are full 64-bit values.
//
// BEF_MUTANT (host test builds only) plants one of the breaks the pages list
// for this header (ADR-1497, Consequences), or a break in the group step of
// a crossing row, so that the host tests can show each one is caught.
// 0 = none.
#pragma once

#include <stdint.h>

#ifndef BEF_MUTANT
#define BEF_MUTANT 0
#endif

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define BEF_HD __host__ __device__ __forceinline__
#else
#define BEF_HD static inline
#endif

namespace bef {

static constexpr uint64_t kTwo53 = 1ull << 53;

// Shape of the ordered kernels' decomposition, shared with the host
// emulation of their steps so that the two cannot drift apart.
static constexpr int kWalkThreads = 512;  // threads of a walk block; runs of a crossing row
static constexpr int kWalkChunk = 4352;   // rows of a plane a walk block holds at a time
static constexpr int kWalkMaxSeg = 64;    // segments of equal plan a walk takes as segments
static constexpr int kPairSeg = 4096;     // samples of a row a pair wave stages at a time
static constexpr int kPairLanes = 64;     // runs of a staged segment, one per lane

// Plan codes for a row or a run.
static constexpr int kPlanExact = -1;  // every add stays at or below 2^53
static constexpr int kPlanCross = 0;   // no single binade can be promised
// any value >= 53: the binade the item is expected to stay in

// floor(log2(s)) for s > 0.
BEF_HD int binade(uint64_t s) { return 63 - __builtin_clzll(s); }

// The CPU's step S <- fl64(S + t) in units.  S and t below 2^62.
BEF_HD uint64_t rne53_add(uint64_t s, uint64_t t) {
  uint64_t n = s + t;
#if BEF_MUTANT == 5 || BEF_MUTANT == 6
  return n;  // mutant: term-by-term adds done exactly / no rounding at all
#else
  if (n <= kTwo53) return n;
  const int sh = binade(n) - 52;
  const uint64_t r = n & ((1ull << sh) - 1);
  uint64_t q = n - r;
  const uint64_t half = 1ull << (sh - 1);
#if BEF_MUTANT == 1
  if (r > half || (r == half && !((q >> sh) & 1))) q += 1ull << sh;  // mutant: a tie to the odd value
#else
  if (r > half || (r == half && ((q >> sh) & 1))) q += 1ull << sh;
#endif
  return q;
#endif
}

// Float32 square of a codeword x, in units: RNE24(x^2) for x < 2^16 (the
// float multiply of the exact float x rounds exactly that).
BEF_HD uint32_t fsq_units(uint32_t x) {
  const float f = (float)x;
#if defined(__HIP_DEVICE_COMPILE__)
  return (uint32_t)__fmul_rn(f, f);
#else
  volatile float p = f * f;  // a float multiply, never contracted
  return (uint32_t)p;
#endif
}

// The same float square as a double (exact: it has 24 significant bits).
BEF_HD double fsq_f64(uint32_t x) {
  const float f = (float)x;
#if defined(__HIP_DEVICE_COMPILE__)
  return (double)__fmul_rn(f, f);
#else
  volatile float p = f * f;  // a float multiply, never contracted
  return (double)p;
#endif
}

// 2^e as a double (-1022 <= e <= 1023).
BEF_HD double pow2(int e) {
  const uint64_t b = (uint64_t)(e + 1023) << 52;
  double d;
  __builtin_memcpy(&d, &b, 8);
  return d;
}

struct Pair32 {
  uint32_t a0, a1;
};
struct Pair64 {
  uint64_t a0, a1;
};

// Identity of composition.
BEF_HD Pair32 pair32_id() { return Pair32{0u, 0u}; }
BEF_HD Pair64 pair64_id() { return Pair64{0ull, 0ull}; }

// Run A then run B (both inside binade sh): from parity p, A moves S by
// A[p], which flips the parity by bit sh of A[p]; B then starts there.
BEF_HD Pair32 then32(Pair32 A, Pair32 B, int sh) {
#if BEF_MUTANT == 3
  Pair32 t = A; A = B; B = t;  // mutant: tree composed in reverse
#endif
  Pair32 r;
#if BEF_MUTANT == 2
  r.a0 = A.a0 + B.a0;  // mutant: parity ignored
  r.a1 = A.a1 + B.a1;
#else
  r.a0 = A.a0 + (((A.a0 >> sh) & 1u) ? B.a1 : B.a0);
  r.a1 = A.a1 + (((A.a1 >> sh) & 1u) ? B.a0 : B.a1);
#endif
  return r;
}

BEF_HD Pair64 then64(Pair64 A, Pair64 B, int sh) {
#if BEF_MUTANT == 3
  Pair64 t = A; A = B; B = t;  // mutant: tree composed in reverse
#endif
  Pair64 r;
#if BEF_MUTANT == 2
  r.a0 = A.a0 + B.a0;  // mutant: parity ignored
  r.a1 = A.a1 + B.a1;
#else
  r.a0 = A.a0 + (((A.a0 >> sh) & 1ull) ? B.a1 : B.a0);
  r.a1 = A.a1 + (((A.a1 >> sh) & 1ull) ? B.a0 : B.a1);
#endif
  return r;
}

// Increments of a run known modulo 2^32 -> full values, given the run's
// exact sum E (|increment - E| < 2^31 always holds for a run of at most
// 2^15 terms: each term moves by at most u/2 <= 2^8 from its exact value).
BEF_HD uint64_t widen(uint32_t d, uint64_t E) {
  const int32_t adj = (int32_t)(d - (uint32_t)E);
  return E + (uint64_t)(int64_t)adj;
}
BEF_HD Pair64 widen_pair(Pair32 p, uint64_t E) {
  return Pair64{widen(p.a0, E), widen(p.a1, E)};
}

// The increment a pair applies to S (S inside the pair's binade).
BEF_HD uint64_t pick(Pair64 p, uint64_t s, int sh) {
#if BEF_MUTANT == 2
  (void)s; (void)sh;
  return p.a0;  // mutant: parity ignored
#else
  return ((s >> sh) & 1ull) ? p.a1 : p.a0;
#endif
}

// Try to add an item (row, stretch of rows, or run) whose pair was formed
// inside binade e.  Accepted only when S is inside binade e and the result
// stays strictly below 2^(e+1): terms are non-negative, so every partial
// sum of the item then stayed inside binade e, where the pair's steps are
// the CPU's steps (the add-chunk acceptance of ADR-1497, Decision, read as
// this test).  Returns false (S untouched) otherwise.
BEF_HD bool try_apply(uint64_t* s, Pair64 p, int e) {
  if (e < 53 || *s < kTwo53 || binade(*s) != e) return false;
  const uint64_t a = pick(p, *s, e - 52);
  const uint64_t n = *s + a;
#if BEF_MUTANT == 6
  (void)n;
  return false;
#else
  if (n >= (1ull << (e + 1))) return false;
  *s = n;
  return true;
#endif
}

// Exact add, allowed while the result stays at or below 2^53.
BEF_HD bool try_exact(uint64_t* s, uint64_t E) {
  if (*s + E > kTwo53) return false;
  *s += E;
  return true;
}

// Plan of an item from its exact prefix P (sum of everything before it,
// exactly) and exact sum E, given a bound M on |S_cpu - P| where rounding
// may already have happened.
BEF_HD int plan_of(uint64_t P, uint64_t E, uint64_t M) {
  if (P + E <= kTwo53) return kPlanExact;
  const uint64_t lo = P > M ? P - M : 0;
  const uint64_t hi = P + E + M;
  if (lo < kTwo53) return kPlanCross;
  const int e = binade(lo);
  return binade(hi) == e ? e : kPlanCross;
}

// Pair of a stretch of terms inside the binade of 2^53 or 2^54 from its
// exact sum E and its count c of odd terms.  Every float square in units is
// 0 or 1 modulo 4 (odd exactly when x is odd and below 4096).  In the
// binade of 2^53 (u = 2) an even term moves S exactly and keeps its
// parity, and an odd term is a tie: it moves by t - 1 + 2 * (parity before)
// and leaves the parity even; so the stretch moves by E - c from an even
// start and by E - c + 2 from an odd one when it holds an odd term.  In the
// binade of 2^54 (u = 4) an odd term rounds down: E - c from either start.
BEF_HD Pair64 closed_pair(uint64_t E, uint64_t c, int e) {
  const uint64_t a0 = E - c;
#if BEF_MUTANT == 8
  (void)e;
  return Pair64{a0, a0};  // mutant: the tie's +2 from an odd start forgotten
#else
  return Pair64{a0, (e == 53 && c > 0) ? a0 + 2 : a0};
#endif
}

// Pair of one noise row t (any integer) inside binade e (sh = e - 52, u =
// 2^sh): the double add moves S by t rounded to a multiple of u, ties to
// the even multiple, which depends on S only through its parity p = (S /
// u) mod 2.  With v = p * u standing in for S: RNE_u(v + t) - v for p = 0
// and 1.
BEF_HD Pair64 noise_row_pair(uint64_t t, int sh) {
  const uint64_t u = 1ull << sh, half = u >> 1;
  const uint64_t z0 = t, z1 = u + t;
#if BEF_MUTANT == 9
  const uint64_t r0 = (z0 + (half - 1) + (1 - ((z0 >> sh) & 1))) & ~(u - 1);  // mutant: ties to odd
  const uint64_t r1 = (z1 + (half - 1) + (1 - ((z1 >> sh) & 1))) & ~(u - 1);
#else
  const uint64_t r0 = (z0 + (half - 1) + ((z0 >> sh) & 1)) & ~(u - 1);
  const uint64_t r1 = (z1 + (half - 1) + ((z1 >> sh) & 1)) & ~(u - 1);
#endif
  return Pair64{r0, r1 - u};
}

// The plan as five edges.  With every sum below 2^55 a stretch's plan
// follows from where its exact interval [P - M, P + E + M] lies against
// 2^53, 2^54 and 2^55 (P the exact sum before it, E its exact sum, M a bound
// on how far the CPU's rounded sum can stray from P).  Each edge is the
// first item at which a non-decreasing quantity reaches a threshold:
//   x0: P + E > 2^53        (end of the exact items)
//   x1: P - M >= 2^53       (first item inside the binade of 2^53)
//   x2: P + E + M >= 2^54   (first item that may leave it)
//   x3: P - M >= 2^54       (first item inside the binade of 2^54)
//   x4: P + E + M >= 2^55   (first item that may leave that one)
// The segments, in order: exact [0, x0), across [x0, x1), 53 [x1, x2),
// across [x2, x3), 54 [x3, x4), beyond [x4, n).
//
// Planes whose exact sum lies in [2^55, 2^56) (their rows' pairs in the
// binade of 2^55 formed beforehand) take seven edges, the same five and
//   x5: P - M >= 2^55       (first item inside the binade of 2^55)
//   x6: P + E + M >= 2^56   (first item that may leave it)
// with the segments exact, across, 53, across, 54, across [x4, x5), 55
// [x5, x6), beyond [x6, n).
constexpr int kEdges = 5;
constexpr int kEdges56 = 7;

// Bit j: whether item k (exact prefix pk before it, pk1 after it) has met
// the condition of edge j (of NE edges).
template <int NE = kEdges>
BEF_HD unsigned edge_conds(uint64_t pk, uint64_t pk1, uint64_t M) {
  constexpr uint64_t T53 = 1ull << 53, T54 = 1ull << 54, T55 = 1ull << 55, T56 = 1ull << 56;
  const uint64_t lo = pk > M ? pk - M : 0;
  unsigned c = (unsigned)(pk1 > T53) | (unsigned)(lo >= T53) << 1 |
               (unsigned)(pk1 + M >= T54) << 2 | (unsigned)(lo >= T54) << 3 |
               (unsigned)(pk1 + M >= T55) << 4;
  if constexpr (NE == kEdges56) c |= (unsigned)(lo >= T55) << 5 | (unsigned)(pk1 + M >= T56) << 6;
  return c;
}

// Segment g's plan (0 exact, 1 across, 2 the binade of 2^53, 3 across, 4
// the binade of 2^54, then 5 beyond with five edges; with seven, 5 across,
// 6 the binade of 2^55, 7 beyond).
template <int NE = kEdges>
BEF_HD int fast_plan(int g) {
  if (g == 0) return kPlanExact;
  if (g == 2) return 53;
  if (g == 4) return 54;
  if (NE == kEdges56 && g == 6) return 55;
  return g == NE ? -2 : kPlanCross;
}

// Applies segment g's exact or closed-form plan to s (Eg, Cg its exact sum
// and odd count); false when it does not apply, and beyond the last edge
// and in the binade of 2^55, whose pairs the caller composes.
template <int NE = kEdges>
BEF_HD bool fast_apply(uint64_t* s, int g, uint64_t Eg, uint64_t Cg) {
  const int e = fast_plan<NE>(g);
  if (e == kPlanExact) return try_exact(s, Eg);
  if (e == 53 || e == 54) return try_apply(s, closed_pair(Eg, Cg, e), e);
  return false;
}

// A row the plan does not fit, as at most three groups of consecutive runs
// (a row adds less than 2^47 units, so it meets at most one binade edge):
// group 0 exact (S below 2^53: low) or inside binade eA, the binade S is
// in; group 1 across the edge; group 2 inside e2, eA when low and eA + 1
// otherwise.  G[k].start is group k's first run (-1 when empty), G[k].P
// and G[k].PC the exact sum and odd count of the row's terms before it;
// G[3] is the row's end.  terms(s, a, b) adds the terms of runs [a, b) to
// s one at a time with the CPU's step; pair_of(k, e, E, C) is group k's
// pair inside binade e given its exact sum E and odd count C.  Returns
// false (S untouched) when a group's step does not apply.
struct GroupStart {
  uint64_t P, PC;
  int start;
};

template <class Terms, class PairOf>
BEF_HD bool apply_groups(uint64_t* sp, const GroupStart* G, bool low, int eA, Terms terms,
                         PairOf pair_of) {
  const int e2 = low ? eA : eA + 1;
  uint64_t s = *sp;
  for (int k = 0; k < 3; ++k) {
    const GroupStart A = G[k];
    if (A.start < 0) continue;
    // the group ends where the next non-empty group (or the row) starts
    const GroupStart B =
        G[k + 1].start >= 0 ? G[k + 1] : (k == 0 && G[2].start >= 0) ? G[2] : G[3];
    if (k == 1) {
#if BEF_MUTANT == 10
      s += B.P - A.P;  // mutant: the terms across the edge added as one exact sum
#else
      s = terms(s, A.start, B.start);
#endif
      continue;
    }
    if (k == 0 && low) {
      if (!try_exact(&s, B.P - A.P)) return false;
      continue;
    }
    const int e = k == 0 ? eA : e2;
#if BEF_MUTANT == 11
    const uint64_t C = B.PC - G[0].PC;  // mutant: the odd count taken from the row's first group
#else
    const uint64_t C = B.PC - A.PC;
#endif
    if (!try_apply(&s, pair_of(k, e, B.P - A.P, C), e)) return false;
  }
  *sp = s;
  return true;
}

// A run of terms added inside binade e (e >= 53), with the double add
// itself.  Inside a binade a term's move depends on S only through the
// parity of S/u, u = 2^(e-52) (ADR-1497, Decision), so the two starts S = 2^e
// (S/u even) and 2^e + u (odd) stand for every S of the binade.  From each,
// every term is added as the CPU adds it: the double add rounds the exact
// sum to a multiple of u, the ulp there, ties to the even multiple.  The
// sums stay inside the binade while the run adds less than 2^e - u: a run
// of at most 2^15 terms adds less than 2^47.  The pair is the two moves,
// kept modulo 2^32 like every lane-level pair.
struct RunF64 {
  double v0, v1;
};
BEF_HD RunF64 run_start(int e) {
#if BEF_MUTANT == 4
  e = e - 1;  // mutant: the run's units taken from the wrong binade
#endif
  const double b = pow2(e);
  return RunF64{b, b + pow2(e - 52)};
}
BEF_HD void run_add(RunF64& r, double t) {
  r.v0 = r.v0 + t;
  r.v1 = r.v1 + t;
}
BEF_HD Pair32 run_end(const RunF64& r, int e) {
#if BEF_MUTANT == 4
  e = e - 1;
#endif
  const double b = pow2(e), u = pow2(e - 52);
  return Pair32{(uint32_t)(uint64_t)(r.v0 - b), (uint32_t)(uint64_t)(r.v1 - b - u)};
}

// Pair of a run of n terms (terms(j): each term as a double) inside binade e.
template <class Terms>
BEF_HD Pair32 run_pair(const Terms& terms, int n, int e) {
  RunF64 r = run_start(e);
#if BEF_MUTANT == 7
  for (int j = n - 1; j >= 0; --j) run_add(r, terms(j));  // mutant: run order reversed in a lane
#else
  for (int j = 0; j < n; ++j) run_add(r, terms(j));
#endif
  return run_end(r, e);
}

}  // namespace bef
