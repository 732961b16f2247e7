// walk.hip -- the ordered part: plan, pairs and the walk of each plane.
//
//   k_plan     (only for frames that can pass 2^55 units, or under a test
//              flag) exact row prefix and per-row binade plan, for k_pairs
//              and the walk, and each plane's exact sums, for the walk.
//   k_pairs    (same condition) the row's pair under its planned binade,
//              one wave per row staged in LDS: 64 lane runs joined by an
//              ordered tree, segments of 4096 samples joined in row order
//              (ADR-1497 Decision).
//   k_walk     one 512-thread block per (frame, plane) takes the rows in
//              order: exact adds up to 2^53, stretches of rows inside one
//              binade applied as one pair (closed form in the binades of
//              2^53 and 2^54), rows that cross a binade edge split into runs
//              taken as at most three groups (inside a binade or exact,
//              across the edge, inside the next binade), runs that cross
//              added term by term with the double add (ADR-1497
//              Decision); one block per frame takes the noise rows
//              in order the same way, a chunk of rows at a time, each row
//              a double add as on the CPU or inside a stretch's composed
//              pair (ADR-1499 Decision); then the divisions.
//
// Units: 1/s^2 for squares, 1/s for first moments (s = 2^(bpc-8)).  No
// atomics anywhere: every sum has one owner and a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bef_internal.h"
#include "ordsum.h"
#include "wave.h"

using namespace bef;

namespace {

// ---------------------------------------------------------------------------
// Block-level helpers for the plan and walk kernels (kT threads = kWaves
// waves).  Every thread calls them with the same arguments; results are
// uniform.

constexpr int kT = kWalkThreads;
constexpr int kWaves = kT / 64;

struct BlockScratch {
  uint64_t w64[2 * kWaves];
  uint64_t v[4];
  int iv[kWaves];
};

__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, BlockScratch& sm) {
  const uint64_t s = wave_sum_u64(v);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.w64[wv] = s;
  __syncthreads();
  uint64_t t = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) t += sm.w64[k];
  return t;
}

// Minimum of non-negative ints.
__device__ __forceinline__ int block_min_int(int v, BlockScratch& sm) {
  v = (int)wave_min_u32((uint32_t)v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.iv[threadIdx.x >> 6] = v;
  __syncthreads();
  int m = sm.iv[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) m = min(m, sm.iv[k]);
  return m;
}

// Exclusive prefix of v over the block's threads in order; *total = sum.
__device__ __forceinline__ uint64_t block_excl_scan_u64(uint64_t v, uint64_t* total,
                                                        BlockScratch& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t inc = wave_incl_scan_u64(v);
  __syncthreads();
  if (lane == 63) sm.w64[wv] = inc;
  __syncthreads();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    const uint64_t x = sm.w64[k];
    before += k < wv ? x : 0;
    all += x;
  }
  *total = all;
  return before + inc - v;
}

// Two-value exclusive block scan (one set of barriers).
__device__ __forceinline__ void block_excl_scan2(uint64_t v, uint64_t u, uint64_t* ev,
                                                 uint64_t* eu, uint64_t* tv, uint64_t* tu,
                                                 BlockScratch& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t iv = wave_incl_scan_u64(v), iu = wave_incl_scan_u64(u);
  __syncthreads();
  if (lane == 63) {
    sm.w64[2 * wv] = iv;
    sm.w64[2 * wv + 1] = iu;
  }
  __syncthreads();
  uint64_t bv = 0, bu = 0, av = 0, au = 0;
  for (int k = 0; k < kWaves; ++k) {
    const uint64_t x = sm.w64[2 * k], y = sm.w64[2 * k + 1];
    if (k < wv) {
      bv += x;
      bu += y;
    }
    av += x;
    au += y;
  }
  *ev = bv + iv - v;
  *eu = bu + iu - u;
  *tv = av;
  *tu = au;
}

// Ordered composition of one pair per lane (lane 0 first) inside a wave:
// lane l takes lane l+1 (quad_perm xor 1), l+2 (quad_perm xor 2), l+4
// (row_shl:4), l+8 (row_shl:8); the four 16-lane row composites are read
// into scalars and joined in order.  Uniform result.
__device__ __forceinline__ Pair64 wave_then(Pair64 p, int sh) {
  const int lane = threadIdx.x & 63;
  Pair64 o;
  o = Pair64{dpp64<0xB1>(p.a0), dpp64<0xB1>(p.a1)};
  if (!(lane & 1)) p = then64(p, o, sh);
  o = Pair64{dpp64<0x4E>(p.a0), dpp64<0x4E>(p.a1)};
  if (!(lane & 3)) p = then64(p, o, sh);
  o = Pair64{dpp64<0x104>(p.a0), dpp64<0x104>(p.a1)};
  if (!(lane & 7)) p = then64(p, o, sh);
  o = Pair64{dpp64<0x108>(p.a0), dpp64<0x108>(p.a1)};
  if (!(lane & 15)) p = then64(p, o, sh);
  const Pair64 r0 = {rdl64(p.a0, 0), rdl64(p.a1, 0)}, r1 = {rdl64(p.a0, 16), rdl64(p.a1, 16)};
  const Pair64 r2 = {rdl64(p.a0, 32), rdl64(p.a1, 32)}, r3 = {rdl64(p.a0, 48), rdl64(p.a1, 48)};
  return then64(then64(r0, r1, sh), then64(r2, r3, sh), sh);
}

// Block version: the waves' composites joined by an ordered tree.
__device__ __forceinline__ Pair64 block_then(Pair64 p, int sh, BlockScratch& sm) {
  const Pair64 w = wave_then(p, sh);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sm.w64[2 * wv] = w.a0;
    sm.w64[2 * wv + 1] = w.a1;
  }
  __syncthreads();
  Pair64 q[kWaves];
#pragma unroll
  for (int k = 0; k < kWaves; ++k) q[k] = Pair64{sm.w64[2 * k], sm.w64[2 * k + 1]};
#pragma unroll
  for (int off = 1; off < kWaves; off <<= 1)
#pragma unroll
    for (int k = 0; k + off < kWaves; k += 2 * off) q[k] = then64(q[k], q[k + off], sh);
  return q[0];
}

// ---------------------------------------------------------------------------
// Plan (shared by k_plan and k_walk), one pass: thread t owns a contiguous
// chunk of rows; one block scan of the chunk totals gives every row's exact
// prefix, hence its plan.

__device__ int debug_plan(int e, int i, unsigned dbg) {
  if (e >= 53 && (dbg & BEF_DBG_PLAN_NONE)) return kPlanCross;
  if (e >= 53 && (dbg & BEF_DBG_PLAN_WRONG)) return (i & 1) ? (e > 53 ? e - 1 : e + 2) : e + 1;
  return e;
}

constexpr int kChunk = kWalkChunk;  // rows held in LDS by the walk

struct RowLds {
  uint64_t R[kChunk];
  uint16_t C[kChunk];
  int8_t plan[kChunk];
};

// Returns the exact plane sum.  When cl is given and h <= kChunk, the rows'
// sums, odd counts and plans are left in LDS, indexed by row, and the global
// plan array is not written; *s1 (if given) receives the plane's
// first-moment sum from r1.  kHoldRows lets a thread with at most 16 rows
// keep them in registers between the two passes.
template <bool kHoldRows = false>
__device__ uint64_t plan_plane(const uint64_t* R, int8_t* plan, int w, int h, unsigned dbg,
                               BlockScratch& sm, RowLds* cl = nullptr,
                               const uint32_t* C = nullptr, const uint32_t* r1 = nullptr,
                               uint64_t* s1 = nullptr) {
  const int c = (h + kT - 1) / kT;
  const int a = min((int)threadIdx.x * c, h), b = min(a + c, h);
  const bool keep = cl != nullptr && h <= kChunk;
  constexpr int kHold = 16;  // rows per thread held in registers between the passes
  const bool hold = kHoldRows && !keep && c <= kHold;
  uint64_t hv[kHold];
  uint64_t loc = 0, s1l = 0;
  if (keep) {
    // every load issued before the first is used: one memory round trip
    constexpr int U = (kChunk + kT - 1) / kT;
    uint64_t rv[U];
    uint32_t cv[U], sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = threadIdx.x + u * kT;
      rv[u] = i < h ? R[i] : 0;
      cv[u] = i < h ? C[i] : 0;
      sv[u] = (i < h && r1) ? r1[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = threadIdx.x + u * kT;
      if (i < h) {
        cl->R[i] = rv[u];
        cl->C[i] = (uint16_t)cv[u];
      }
      s1l += sv[u];
    }
    if (s1) *s1 = block_sum_u64(s1l, sm);  // also the barrier before reading cl
    else __syncthreads();
    for (int i = a; i < b; ++i) loc += cl->R[i];
  } else if (hold) {
    // the thread's rows in one round trip, kept for the second pass
    uint32_t sv[kHold];
#pragma unroll
    for (int u = 0; u < kHold; ++u) {
      const int i = a + u;
      hv[u] = i < b ? R[i] : 0;
      sv[u] = (r1 && i < b) ? r1[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kHold; ++u) {
      loc += hv[u];
      s1l += sv[u];
    }
  } else {
    // the thread's own rows, eight loads in flight at a time
    for (int i0 = a; i0 < b; i0 += 8) {
      uint64_t rv[8];
      uint32_t sv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u;
        rv[u] = i < b ? R[i] : 0;
        sv[u] = (r1 && i < b) ? r1[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        loc += rv[u];
        s1l += sv[u];
      }
    }
  }
  uint64_t E, p;
  if (s1 && !keep) {  // the first-moment sum rides on the scan's barriers
    uint64_t ps1;
    block_excl_scan2(loc, s1l, &p, &ps1, &E, s1, sm);
  } else {
    p = block_excl_scan_u64(loc, &E, sm);
  }
  const uint64_t M = E > kTwo53 ? ((uint64_t)w * (uint64_t)h) << (binade(E) - 53) : 0;
  auto emit = [&](int i, uint64_t r) {  // row i's plan from its exact prefix p
    const int e = debug_plan(plan_of(p, r, M), i, dbg);
    if (keep) cl->plan[i] = (int8_t)e;
    else plan[i] = (int8_t)e;
    p += r;
  };
  if (hold) {
#pragma unroll
    for (int u = 0; u < kHold; ++u)
      if (a + u < b) emit(a + u, hv[u]);
  } else {
    for (int i0 = a; i0 < b; i0 += 8) {
      uint64_t rv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u;
        rv[u] = i < b ? (keep ? cl->R[i] : R[i]) : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u < b) emit(i0 + u, rv[u]);
    }
  }
  if (keep) __syncthreads();  // the plans in LDS visible to the whole block
  return E;
}

__device__ __forceinline__ bool may_round(uint64_t E, unsigned dbg) {
  return E > kTwo53 || (dbg & BEF_DBG_FORCE_ROUND);
}

// Also leaves the plane's exact sums of r2 and r1 in psum, so that the
// general walk need not plan the plane again.
__global__ void __launch_bounds__(kT) k_plan(Geometry g, RowArrays ra, unsigned dbg) {
  __shared__ BlockScratch sm;
  const int f = blockIdx.x >> 1, pl = blockIdx.x & 1;
  const long off = (long)(pl * g.nframes + f) * g.h;
  uint64_t s1 = 0;
  const uint64_t E =
      plan_plane<true>(ra.r2 + off, ra.plan + off, g.w, g.h, dbg, sm, nullptr, nullptr, ra.r1 + off, &s1);
  if (threadIdx.x == 0) {
    ra.psum[2 * (pl * g.nframes + f)] = E;
    ra.psum[2 * (pl * g.nframes + f) + 1] = s1;
  }
}

// ---------------------------------------------------------------------------
// k_pairs: the pair of a row under its planned binade.  One wave per row:
// the row is staged in LDS a segment at a time with coalesced loads, each
// lane forms the pair of its run of consecutive terms from LDS, an ordered
// shuffle-down tree joins the 64 runs, and the segments' pairs are joined
// in row order.

__device__ __forceinline__ bool needs_pair(int e, unsigned dbg) {
  return e >= 55 || (e >= 53 && (dbg & BEF_DBG_NO_CLOSED_FORM));
}

// Samples [s0, s0 + n) of a row into buf (n <= kPairSeg) by one wave: every
// load is issued before the first store.
template <typename T>
__device__ __forceinline__ void wave_stage_segment(uint16_t* buf, const T* row, int s0, int n) {
  const int lane = threadIdx.x & 63;
  if (sizeof(T) == 2 && ((uintptr_t)(row + s0) & 15) == 0) {
    // 16-byte loads of whole 8-sample chunks, then the tail sample by sample
    const int nv = n >> 3;
    constexpr int UV = kPairSeg / 8 / 64;
    v4u v[UV];
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int c = u * 64 + lane;
      v[u] = c < nv ? ((const v4u*)(row + s0))[c] : (v4u){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int c = u * 64 + lane;
      if (c < nv) ((v4u*)buf)[c] = v[u];
    }
    for (int j = nv * 8 + lane; j < n; j += 64) buf[j] = (uint16_t)row[s0 + j];
    return;
  }
  constexpr int U = 16;  // loads in flight per lane per round
  for (int j0 = 0; j0 < n; j0 += U * 64) {
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * 64 + lane;
      v[u] = j < n ? (uint32_t)row[s0 + j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * 64 + lane;
      if (j < n) buf[j] = (uint16_t)v[u];
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(256) k_pairs(Geometry g, RowArrays ra, unsigned dbg,
                                                long task0) {
  __shared__ __attribute__((aligned(16))) uint16_t seg[4][kPairSeg];
  const int lane = threadIdx.x & 63;
  const long task = task0 + (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long per = 2L * g.nframes;
  if (task >= per * g.h) return;
  const int i = g.h - 1 - (int)(task / per);  // last rows first
  const int rem = (int)(task % per);
  const int pl = rem / g.nframes, f = rem % g.nframes;
  const long k = (long)(pl * g.nframes + f) * g.h + i;
  const int e = ra.plan[k];
  if (!needs_pair(e, dbg)) return;  // the whole wave: one task per wave
  const int sh = e - 52;
  const T* row = (const T*)(pl == 0 ? g.ref : g.dis) + (long)f * g.pitch + (long)i * g.stride;
  uint16_t* buf = seg[threadIdx.x >> 6];
  Pair32 acc = {0u, 0u};  // the identity
  for (int s0 = 0; s0 < g.w; s0 += kPairSeg) {
    const int n = min(kPairSeg, g.w - s0);
    wave_stage_segment(buf, row, s0, n);
    wave_lds_sync();
    const int L = (n + 63) >> 6;
    const int j0 = min(lane * L, n), j1 = min(j0 + L, n);
    Pair32 p;
    if ((L & 7) == 0 && (j1 - j0) == L) {
      // a whole run of 8-sample chunks: one 16-byte LDS read per 8 terms,
      // each term added from both starts with the double add, in order
      RunF64 r = run_start(e);
      for (int c = j0 >> 3; c < (j0 + L) >> 3; ++c) {
        const v4u x = ((const v4u*)buf)[c];
#pragma unroll
        for (int q = 0; q < 8; ++q) run_add(r, fsq_f64((x[q >> 1] >> (16 * (q & 1))) & 0xFFFFu));
      }
      p = run_end(r, e);
    } else {
      p = run_pair([&](int j) { return fsq_f64(buf[j0 + j]); }, j1 - j0, e);
    }
    for (int off = 1; off < 64; off <<= 1) {
      Pair32 o;
      o.a0 = __shfl_down(p.a0, off);
      o.a1 = __shfl_down(p.a1, off);
      if ((lane & (2 * off - 1)) == 0) p = then32(p, o, sh);
    }
    acc = then32(acc, p, sh);  // meaningful in lane 0
    wave_lds_sync();  // the next segment reuses buf
  }
  if (lane == 0) {
    const Pair64 q = widen_pair(acc, ra.r2[k]);
    ra.pairs[2 * k] = q.a0;
    ra.pairs[2 * k + 1] = q.a1;
  }
}


// The pair pass for 16-bit planes whose rows start on 16-byte boundaries and
// hold whole 8-sample chunks: each wave takes kPipeRows consecutive tasks
// and runs their segments as one stream, the next segment's 16-byte loads
// in flight (in registers) while the current one is summed from LDS.  The
// arithmetic is k_pairs': the same runs, trees and joins, in the same order.
// One row per wave: with more, too few waves have work (a wave's tasks are
// one row of the same planes, which need pairs together or not at all).
constexpr int kPipeRows = 1;

__device__ __forceinline__ const uint16_t* pair_row(const Geometry& g, long task, long* k) {
  const long per = 2L * g.nframes;
  const int i = g.h - 1 - (int)(task / per);  // last rows first
  const int rem = (int)(task % per);
  const int pl = rem / g.nframes, f = rem % g.nframes;
  *k = (long)(pl * g.nframes + f) * g.h + i;
  return (const uint16_t*)(pl == 0 ? g.ref : g.dis) + (long)f * g.pitch + (long)i * g.stride;
}

__global__ void __launch_bounds__(256) k_pairs_pipe(Geometry g, RowArrays ra, unsigned dbg,
                                                     long task0) {
  __shared__ __attribute__((aligned(16))) uint16_t seg[4][kPairSeg];
  const int lane = threadIdx.x & 63;
  const long ntask = 2L * g.nframes * g.h;
  const long t0 = task0 + ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * kPipeRows;
  uint16_t* buf = seg[threadIdx.x >> 6];
  // the wave's rows that need a pair (bit r: task t0 + r)
  unsigned need = 0;
#pragma unroll
  for (int r = 0; r < kPipeRows; ++r) {
    if (t0 + r < ntask) {
      long k;
      pair_row(g, t0 + r, &k);
      if (needs_pair(ra.plan[k], dbg)) need |= 1u << r;
    }
  }
  if (need == 0) return;  // wave-uniform
  const int nseg = (g.w + kPairSeg - 1) / kPairSeg;
  constexpr int UV = kPairSeg / 8 / 64;
  int r = __builtin_ctz(need), sg = 0;
  long k;
  const uint16_t* row = pair_row(g, t0 + r, &k);
  v4u v[UV];
  auto issue = [&](const uint16_t* rw, int s0) {  // the segment's loads, not waited for
    const int nv = min(kPairSeg, g.w - s0) >> 3;
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int c = u * 64 + lane;
      v[u] = c < nv ? __builtin_nontemporal_load((const v4u*)(rw + s0) + c) : (v4u){0u, 0u, 0u, 0u};
    }
  };
  issue(row, 0);
  Pair32 acc = {0u, 0u};
  int sh = ra.plan[k] - 52;
  while (true) {
    const int s0 = sg * kPairSeg, n = min(kPairSeg, g.w - s0), nv = n >> 3;
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int c = u * 64 + lane;
      if (c < nv) ((v4u*)buf)[c] = v[u];
    }
    wave_lds_sync();
    // the next segment: this row's next one, else the first of the next row with a pair
    int rn = r, sn = sg + 1;
    if (sn == nseg) {
      const unsigned rest = need & ~((2u << r) - 1u);
      rn = rest ? __builtin_ctz(rest) : kPipeRows;
      sn = 0;
    }
    long kn = k;
    const uint16_t* rown = row;
    if (rn < kPipeRows) {
      if (rn != r) rown = pair_row(g, t0 + rn, &kn);
      issue(rown, sn * kPairSeg);
    }
    const int L = (n + 63) >> 6;
    const int j0 = min(lane * L, n), j1 = min(j0 + L, n);
    Pair32 p;
    if ((L & 7) == 0 && (j1 - j0) == L) {
      RunF64 r = run_start(sh + 52);
      for (int c = j0 >> 3; c < (j0 + L) >> 3; ++c) {
        const v4u x = ((const v4u*)buf)[c];
#pragma unroll
        for (int q = 0; q < 8; ++q) run_add(r, fsq_f64((x[q >> 1] >> (16 * (q & 1))) & 0xFFFFu));
      }
      p = run_end(r, sh + 52);
    } else {
      p = run_pair([&](int j) { return fsq_f64(buf[j0 + j]); }, j1 - j0, sh + 52);
    }
    for (int off = 1; off < 64; off <<= 1) {
      Pair32 o;
      o.a0 = __shfl_down(p.a0, off);
      o.a1 = __shfl_down(p.a1, off);
      if ((lane & (2 * off - 1)) == 0) p = then32(p, o, sh);
    }
    acc = then32(acc, p, sh);  // meaningful in lane 0
    if (sg == nseg - 1) {
      if (lane == 0) {
        const Pair64 q = widen_pair(acc, ra.r2[k]);
        ra.pairs[2 * k] = q.a0;
        ra.pairs[2 * k + 1] = q.a1;
      }
      acc = Pair32{0u, 0u};
    }
    wave_lds_sync();  // the next segment reuses buf
    if (rn == kPipeRows) break;
    if (rn != r) sh = ra.plan[kn] - 52;
    r = rn;
    sg = sn;
    k = kn;
    row = rown;
  }
}

// ---------------------------------------------------------------------------
// k_walk.
//
// The walk is latency-bound: one block per (frame, plane) and a short
// sequential path.  The general walk (any geometry, any sum, every test
// mode; the fast path below covers the common case with one wave): items
// (the rows of a plane, or the runs of a row that
// leaves its plan) are grouped into segments of equal plan by one pass that
// also records the exact prefix of the item sums and of the odd-square
// counts at every segment start.  A segment planned exact adds its sum; a
// segment planned in the binade of 2^53 or 2^54 adds its closed-form pair
// from the two prefix differences alone; other binades compose
// their items' pairs with an ordered tree.  A segment that does not fit goes
// item by item: a row to its runs, a run to its terms.
//
// Closed form (closed_pair in the step header): every float square in units
// is 0 or 1 modulo 4, so in the binades of 2^53 and 2^54 a stretch's pair
// follows from its exact sum and its count of odd squares.

constexpr int kStage = 8192;  // samples of one row staged in LDS by the fast walk (max w)
constexpr int kStageRound = 8;  // 16-byte chunks a lane of the fast walk has in flight at once
constexpr int kRowMax = 32768;  // samples of one row staged in LDS by the general walk (max w)
constexpr int kMaxSeg = kWalkMaxSeg;  // segments a walk handles as segments

struct Seg {
  uint64_t P;   // exact sum of the items before the segment
  uint64_t PC;  // odd squares before the segment
  int start;
  int plan;
};

// One run per thread of a fallback row: exact sum, odd count, plan, and the
// pairs under the binade S is in (A) and the next one (B) as signed offsets
// from the exact sum (a run of at most 32 terms moves less than 2^31).
struct RunLds {
  uint64_t E[kT];
  uint32_t C[kT];
  int32_t A0[kT], A1[kT], B0[kT], B1[kT];
  int8_t plan[kT];
};

// Segment table of items [0, n) whose sums E, odd counts C and plans are in
// LDS (plan already final and visible).  Thread t owns items
// [t*c, t*c + c).  Returns the number of segments; the table holds
// min(n_seg, kMaxSeg) entries plus a closing entry at n when it fits.
template <class EAt, class CAt, class PlanAt>
__device__ __forceinline__ int build_segments(int n, EAt e_at, CAt c_at, PlanAt plan_at,
                                              Seg* tab, BlockScratch& sm) {
  const int c = (n + kT - 1) / kT;
  const int a = min((int)threadIdx.x * c, n), b = min(a + c, n);
  uint64_t le = 0, lc = 0, ln = 0;
  for (int k = a; k < b; ++k) {
    le += e_at(k);
    lc += c_at(k);
    ln += (k == 0 || plan_at(k) != plan_at(k - 1)) ? 1 : 0;
  }
  uint64_t pe, pcn, te, tcn;
  // odd counts (< 2^31) and boundary counts (< 2^31) share one 64-bit scan
  block_excl_scan2(le, (lc << 32) | ln, &pe, &pcn, &te, &tcn, sm);
  uint64_t P = pe, PC = pcn >> 32;
  int idx = (int)(pcn & 0xFFFFFFFFu);
  for (int k = a; k < b; ++k) {
    if (k == 0 || plan_at(k) != plan_at(k - 1)) {
      if (idx < kMaxSeg) tab[idx] = Seg{P, PC, k, plan_at(k)};
      ++idx;
    }
    P += e_at(k);
    PC += c_at(k);
  }
  const int nseg = (int)(tcn & 0xFFFFFFFFu);
  if (threadIdx.x == 0 && nseg <= kMaxSeg) tab[nseg] = Seg{te, tcn >> 32, n, 0};
  __syncthreads();
  return nseg;
}

template <class PairAt>
__device__ __forceinline__ Pair64 compose_items(int a, int b, int sh, PairAt pair_at,
                                                BlockScratch& sm) {
  const int c = (b - a + kT - 1) / kT;
  Pair64 acc = pair64_id();
  const int k0 = a + threadIdx.x * c;
  for (int k = k0; k < k0 + c && k < b; ++k) acc = then64(acc, pair_at(k), sh);
  return block_then(acc, sh, sm);
}

// Rows [a, a + n) of a plane's row sums, odd counts and plans into LDS, every
// load issued before the first store (no barrier).
__device__ __forceinline__ void load_rows(RowLds& rows, const uint64_t* R, const uint32_t* C,
                                          const int8_t* plan, int a, int n) {
  constexpr int U = (kChunk + kT - 1) / kT;
  uint64_t rv[U];
  uint32_t cv[U];
  int8_t pv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = u * kT + (int)threadIdx.x;
    rv[u] = k < n ? R[a + k] : 0;
    cv[u] = k < n ? C[a + k] : 0;
    pv[u] = k < n ? plan[a + k] : (int8_t)0;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = u * kT + (int)threadIdx.x;
    if (k < n) {
      rows.R[k] = rv[u];
      rows.C[k] = (uint16_t)cv[u];
      rows.plan[k] = pv[u];
    }
  }
}

struct Walker {
  const void* plane;  // this frame's plane
  long stride;
  int w, h, bpc8;
  const uint64_t* R;  // global row sums, loaded a chunk at a time unless held in LDS
  const uint32_t* C;
  const int8_t* plan;
  const uint64_t* pairs;
  unsigned dbg;
  BlockScratch& sm;
  RowLds& rows;
  RunLds& runs;
  Seg* rseg;
  Seg* useg;
  uint16_t* rowbuf;
  int* staged;

  __device__ uint32_t sample(long k) const {
    return bpc8 ? ((const uint8_t*)plane)[k] : ((const uint16_t*)plane)[k];
  }
  // Term j of row i, which fallback_row has staged in rowbuf.
  __device__ uint32_t term(int, int j) const { return fsq_units(rowbuf[j]); }
  // Terms [j0, j1) of row i added to s one at a time with the double add,
  // the CPU's own step (s is a value its double holds); terms are read
  // eight ahead of the ordered adds.
  __device__ uint64_t terms(uint64_t s, int i, int j0, int j1) const {
    double d = (double)s;
    int j = j0;
    for (; j + 8 <= j1; j += 8) {
      double t[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) t[q] = (double)term(i, j + q);
#pragma unroll
      for (int q = 0; q < 8; ++q) d = d + t[q];
    }
    for (; j < j1; ++j) d = d + (double)term(i, j);
    return (uint64_t)d;
  }

  // Pair of row k of the chunk starting at row c0, under its plan e.
  __device__ Pair64 row_pair(int c0, int k, int e) const {
    if (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM)) return closed_pair(rows.R[k], rows.C[k], e);
    const long i = c0 + k;
    return Pair64{pairs[2 * i], pairs[2 * i + 1]};
  }
  __device__ Pair64 run_pair_at(int k, int e, int eA) const {
    const uint64_t E = runs.E[k];
    if (e == eA) return Pair64{E + (uint64_t)(int64_t)runs.A0[k], E + (uint64_t)(int64_t)runs.A1[k]};
    return Pair64{E + (uint64_t)(int64_t)runs.B0[k], E + (uint64_t)(int64_t)runs.B1[k]};
  }

  // A row the plan does not fit, by groups of runs: kT runs of ceil(w/kT)
  // terms, each planned from its exact prefix with the row's margin.  A
  // row meets at most one edge, so its runs fall in at most three groups
  // in row order: with S below 2^53 exact, across, binade eA; else binade
  // eA, across, binade eB.  A group inside a binade adds its closed-form
  // pair (binades of 2^53 and 2^54) or its runs' pairs joined in order; the
  // group across the edge goes term by term.  Returns false (S untouched)
  // when the runs do not form such groups or a group's step does not apply.
  __device__ bool row_groups(uint64_t* sp, int i) const {
    const uint64_t s0 = *sp;
    const bool low = s0 < kTwo53;
    const int eA = low ? 53 : binade(s0), eB = eA + 1;
    const int e2 = low ? eA : eB;  // binade of group 2 (group 0: exact or eA)
    const int L = (w + kT - 1) / kT, nr = (w + L - 1) / L;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int j0 = min(t * L, w), j1 = min(j0 + L, w);
    uint64_t E = 0;
    uint32_t c = 0;
    for (int j = j0; j < j1; j += 8) {  // eight LDS reads in flight at a time
      uint32_t x[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = j + q < j1 ? term(i, j + q) : 0u;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        E += x[q];
        c += x[q] & 1u;
      }
    }
    uint64_t Q, QC, tot, totc;
    block_excl_scan2(E, c, &Q, &QC, &tot, &totc, sm);
    int g = 3;  // the run's group; 3: none of the three
    if (t < nr) {
      const int p = plan_of(s0 + Q, E, (uint64_t)w << (eB - 53));
      g = p == kPlanCross ? 1 : (p == (low ? kPlanExact : eA)) ? 0 : p == e2 ? 2 : 3;
    }
    // pairs of the runs of groups in binades from 2^55 up, joined in order
    const bool tree0 = !low && eA >= 55, tree2 = e2 >= 55;
    Pair64 c0 = pair64_id(), c2 = pair64_id();
    if (tree0 || tree2) {
      const int e = g == 0 ? eA : e2;
      if ((g == 0 && tree0) || (g == 2 && tree2)) {
        // the run from both starts with the double add (run_pair's steps),
        // terms read eight at a time (a zero term moves nothing)
        RunF64 r = run_start(e);
        for (int j = j0; j < j1; j += 8) {
          uint32_t x[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) x[q] = j + q < j1 ? term(i, j + q) : 0u;
#pragma unroll
          for (int q = 0; q < 8; ++q) run_add(r, (double)x[q]);
        }
        const Pair64 pr = widen_pair(run_end(r, e), E);
        if (g == 0) c0 = pr;
        else c2 = pr;
      }
      if (tree0) c0 = wave_then(c0, eA - 52);
      if (tree2) c2 = wave_then(c2, e2 - 52);
      if (lane == 0) {
        runs.E[4 * wv] = c0.a0;
        runs.E[4 * wv + 1] = c0.a1;
        runs.E[4 * wv + 2] = c2.a0;
        runs.E[4 * wv + 3] = c2.a1;
      }
    }
    runs.plan[t] = (int8_t)g;
    if (t == 0) {
      sm.iv[0] = 0;  // set when the groups are not in order
      for (int k = 0; k < 3; ++k) useg[k].start = -1;
    }
    __syncthreads();
    if (t < nr) {
      const int gp = t > 0 ? runs.plan[t - 1] : -1;
      if (g == 3 || gp > g) sm.iv[0] = 1;
      if (gp != g && g < 3) useg[g] = Seg{Q, QC, t, g};
    }
    if (tree0 || tree2) {  // the waves' composites joined in order
      c0 = Pair64{runs.E[0], runs.E[1]};
      c2 = Pair64{runs.E[2], runs.E[3]};
      for (int k = 1; k < kWaves; ++k) {
        c0 = then64(c0, Pair64{runs.E[4 * k], runs.E[4 * k + 1]}, eA - 52);
        c2 = then64(c2, Pair64{runs.E[4 * k + 2], runs.E[4 * k + 3]}, e2 - 52);
      }
    }
    __syncthreads();
    if (sm.iv[0]) return false;
    GroupStart G[4];  // the three groups' starts (start -1: empty), then the end
#pragma unroll
    for (int k = 0; k < 3; ++k) G[k] = GroupStart{useg[k].P, useg[k].PC, useg[k].start};
    G[3] = GroupStart{tot, totc, nr};
    return apply_groups(
        sp, G, low, eA,
        [&](uint64_t s, int ra, int rb) { return terms(s, i, ra * L, min(rb * L, w)); },
        [&](int k, int e, uint64_t Eg, uint64_t Cg) {
          return e <= 54 ? closed_pair(Eg, Cg, e) : (k == 0 ? c0 : c2);
        });
  }

  // A row the plan does not fit, from S: kT runs of ceil(w/kT) terms, each
  // with its pairs under the binade S is in and the next one, planned from
  // their own exact prefix; a run that fits neither is added term by term.
  __device__ uint64_t fallback_row(uint64_t s, int i) const {
    if (*staged != i) {
      // the row into LDS (w <= kRowMax), coalesced, each round's loads all
      // issued before the first store
      __syncthreads();
      const long base = (long)i * stride;
      const uint16_t* row16 = (const uint16_t*)plane + base;
      if (!bpc8 && (w & 7) == 0 && ((uintptr_t)row16 & 15) == 0) {
        // 16-byte loads: 8 samples each, at most 8 per thread (w <= 32768)
        const int nv = w >> 3;
        v4u v[kRowMax / 8 / kT];
#pragma unroll
        for (int u = 0; u < kRowMax / 8 / kT; ++u) {
          const int c = u * kT + (int)threadIdx.x;
          v[u] = c < nv ? ((const v4u*)row16)[c] : (v4u){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kRowMax / 8 / kT; ++u) {
          const int c = u * kT + (int)threadIdx.x;
          if (c < nv) ((v4u*)rowbuf)[c] = v[u];
        }
      } else {
      constexpr int U = 16;
      for (int j0 = 0; j0 < w; j0 += U * kT) {
        uint32_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = j0 + u * kT + (int)threadIdx.x;
          v[u] = j < w ? sample(base + j) : 0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = j0 + u * kT + (int)threadIdx.x;
          if (j < w) rowbuf[j] = (uint16_t)v[u];
        }
      }
      }
      if (threadIdx.x == 0) *staged = i;
      __syncthreads();
    }
    if (dbg & BEF_DBG_TERMS_ONLY) return terms(s, i, 0, w);
    // (the test modes without stretches or closed forms keep to the segment walk)
    if (!(dbg & (BEF_DBG_NO_STRETCH | BEF_DBG_NO_CLOSED_FORM))) {
      uint64_t s2 = s;
      if (row_groups(&s2, i)) return s2;  // else the segment walk over the runs below
    }
    const int eA = s < kTwo53 ? 53 : binade(s);
    const int eB = eA + 1;
    const int L = (w + kT - 1) / kT;
    const int t = threadIdx.x;
    const int j0 = min(t * L, w), j1 = min(j0 + L, w);
    uint64_t E = 0;
    uint32_t c = 0;
    for (int j = j0; j < j1; ++j) {
      const uint32_t x = term(i, j);
      E += x;
      c += x & 1u;
    }
    int32_t d[4];
    for (int q = 0; q < 2; ++q) {
      const int e = q ? eB : eA;
      if (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM)) {
        const Pair64 p = closed_pair(E, c, e);
        d[2 * q] = (int32_t)(p.a0 - E);
        d[2 * q + 1] = (int32_t)(p.a1 - E);
      } else {
        const Pair32 p = run_pair([&](int j) { return (double)term(i, j0 + j); }, j1 - j0, e);
        d[2 * q] = (int32_t)(p.a0 - (uint32_t)E);
        d[2 * q + 1] = (int32_t)(p.a1 - (uint32_t)E);
      }
    }
    uint64_t q, tot;
    q = block_excl_scan_u64(E, &tot, sm);
    const uint64_t Mr = (uint64_t)w << (eB - 53);
    runs.E[t] = E;
    runs.C[t] = c;
    runs.A0[t] = d[0];
    runs.A1[t] = d[1];
    runs.B0[t] = d[2];
    runs.B1[t] = d[3];
    runs.plan[t] = (int8_t)plan_of(s + q, E, Mr);
    __syncthreads();
    const int nseg = build_segments(
        kT, [&](int k) { return runs.E[k]; }, [&](int k) { return (uint64_t)runs.C[k]; },
        [&](int k) { return (int)runs.plan[k]; }, useg, sm);
    auto step = [&](uint64_t s2, int k) {
      if (try_exact(&s2, runs.E[k])) return s2;
      if (try_apply(&s2, run_pair_at(k, eA, eA), eA)) return s2;
      if (try_apply(&s2, run_pair_at(k, eB, eA), eB)) return s2;
      const int a = min(k * L, w);
      return terms(s2, i, a, min(a + L, w));
    };
    if (nseg > kMaxSeg) {
      for (int k = 0; k < kT; ++k) s = step(s, k);
    } else {
      for (int g = 0; g < nseg; ++g) {
        const Seg A = useg[g], B = useg[g + 1];
        const int e = A.plan;
        bool done = false;
        if (e == kPlanExact) {
          done = try_exact(&s, B.P - A.P);
        } else if (e >= 53 && !(dbg & BEF_DBG_NO_STRETCH)) {
          const Pair64 p = (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM))
                               ? closed_pair(B.P - A.P, B.PC - A.PC, e)
                               : compose_items(A.start, B.start, e - 52,
                                               [&](int k) { return run_pair_at(k, e, eA); }, sm);
          done = try_apply(&s, p, e);
        }
        if (!done)
          for (int k = A.start; k < B.start; ++k) s = step(s, k);
      }
    }
    __syncthreads();  // the run arrays are reused by the next fallback
    return s;
  }

  // Rows [0, n) of the chunk held in `rows` (first row c0), from s.
  __device__ uint64_t walk_chunk(int c0, int n, uint64_t s) const {
    const int nseg = build_segments(
        n, [&](int k) { return rows.R[k]; }, [&](int k) { return (uint64_t)rows.C[k]; },
        [&](int k) { return (int)rows.plan[k]; }, rseg, sm);
    auto step = [&](uint64_t s2, int k) {
      if (try_exact(&s2, rows.R[k])) return s2;
      const int e = rows.plan[k];
      if (e >= 53 && try_apply(&s2, row_pair(c0, k, e), e)) return s2;
      return fallback_row(s2, c0 + k);
    };
    if (nseg > kMaxSeg) {
      for (int k = 0; k < n; ++k) s = step(s, k);
      return s;
    }
    for (int g = 0; g < nseg; ++g) {
      const Seg A = rseg[g], B = rseg[g + 1];
      const int e = A.plan;
      bool done = false;
      if (e == kPlanExact) {
        done = try_exact(&s, B.P - A.P);
      } else if (e >= 53 && !(dbg & BEF_DBG_NO_STRETCH)) {
        const Pair64 p = (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM))
                             ? closed_pair(B.P - A.P, B.PC - A.PC, e)
                             : compose_items(A.start, B.start, e - 52,
                                             [&](int k) { return row_pair(c0, k, e); }, sm);
        done = try_apply(&s, p, e);
      }
      if (!done)
        for (int k = A.start; k < B.start; ++k) s = step(s, k);
    }
    return s;
  }

  // The plane from S = 0, a chunk of rows at a time (when `held`, plan_plane
  // has left the rows of a plane that fits one chunk in LDS).
  // (first_loaded: the caller has put the first chunk in LDS already)
  __device__ uint64_t walk_rows(bool held, bool first_loaded) const {
    if (held) return walk_chunk(0, h, 0);
    uint64_t s = 0;
    for (int a = 0; a < h; a += kChunk) {
      const int n = min(kChunk, h - a);
      if (a > 0 || !first_loaded) {
        __syncthreads();
        load_rows(rows, R, C, plan, a, n);
        __syncthreads();
      }
      s = walk_chunk(a, n, s);
    }
    return s;
  }
};

// ---------------------------------------------------------------------------
// Fast walk: the common case, with a short sequential path run by one wave.
// The plane's row sums sit in LDS; the plan is five threshold edges (below),
// found by two wave scans; stretches planned exact or in the binades of
// 2^53 and 2^54 are added from prefix differences (closed form); a row
// across an edge, staged beforehand by the whole block, is split into 64
// lane runs the same way, and only the terms at an edge go one at a time,
// with the double add.  Anything else (planes taller than one chunk, rows
// wider than kStage, sums from 2^56, a stretch that is refused, test modes)
// returns false and the general walk runs instead.

// With every sum below 2^55 an item's plan follows from where its exact
// interval [P - M, P + E + M] lies against 2^53, 2^54 and 2^55.  Each edge
// of a plan is the first item at which a non-decreasing quantity (P + E, or
// P - M, or P + E + M) reaches a threshold, so one scan over the lanes'
// chunks and one over the items of the chunk that holds the edge find each
// of them:
//   x0: P + E > 2^53        (end of the exact items)
//   x1: P - M >= 2^53       (first item inside the binade of 2^53)
//   x2: P + E + M >= 2^54   (first item that may leave it)
//   x3: P - M >= 2^54       (first item inside the binade of 2^54)
//   x4: P + E + M >= 2^55   (first item that may leave that one)
// The segments, in order, are exact [0, x0), across [x0, x1), 53 [x1, x2),
// across [x2, x3), 54 [x3, x4), beyond [x4, n); empty ones are skipped.

constexpr int kRowsPer = (kChunk + kT - 1) / kT;  // rows per thread when loading a plane's sums

// ---------------------------------------------------------------------------
// The fast path: one wave (64 lanes, no block barrier) per plane, with the
// plan as five threshold edges, or seven for planes whose sum lies in the
// binade of 2^55 (edge_conds, fast_plan, fast_apply in the step header).

// NE edges of n items (uniform over the wave): x[j], the exact prefix P[j]
// (base included) and odd count PC[j] before each edge; entry NE is n and
// the totals.
template <int NE>
struct WEdgesN {
  int x[NE + 1];
  uint64_t P[NE + 1];
  uint32_t PC[NE + 1];
  bool ok;
};
using WEdges = WEdgesN<kEdges>;

// Lane l owns items [l*c, l*c + c) with sum le, odd count lc and last item
// value elast; item_at(k, &e, &cnt) gives any single item.  Each condition
// is monotone in the item index, so an edge lies in the one lane whose
// chunk starts false and ends true; that lane's items are then spread one
// per lane, 64 at a time, and scanned again: the first item that meets the
// condition is the edge.
template <int NE = kEdges, class ItemAt>
__device__ __forceinline__ WEdgesN<NE> wave_edges(int n, int c, uint64_t le, uint32_t lc,
                                                  uint64_t elast, uint64_t base, uint64_t M,
                                                  ItemAt item_at) {
  const int lane = threadIdx.x & 63;
  const int a = min(lane * c, n), cl = min(c, n - a);
  const uint64_t P = base + wave_excl_scan_u64(le);
  const uint32_t PC = wave_excl_scan_u32(lc);
  const uint64_t T = rdl64(P + le, 63);
  const uint32_t TC = rdl32(PC + lc, 63);
  const uint64_t ep = lane_before_u64(elast);
  const unsigned before = (cl > 0 && a > 0) ? edge_conds<NE>(P - ep, P, M) : 0u;
  const unsigned last = cl > 0 ? edge_conds<NE>(P + le - elast, P + le, M) : 0u;
  const unsigned own = last & ~before;
  const unsigned occurs = rdl32(last, (n - 1) / c);  // conditions at item n - 1
  WEdgesN<NE> r;
  r.ok = true;
#pragma unroll
  for (int j = 0; j <= NE; ++j) {
    r.x[j] = n;
    r.P[j] = T;
    r.PC[j] = TC;
  }
  unsigned pending = occurs & ((1u << NE) - 1u);
  while (pending) {
    const int j0 = __builtin_ctz(pending);
    const uint64_t om = wave_ballot((own >> j0) & 1u);
    if (om == 0) {  // not monotone: not the premise
      r.ok = false;
      return r;
    }
    const int owner = __builtin_ctzll(om);
    const unsigned owned = rdl32(own, owner) & pending;
    const int b0 = owner * c, cnt = min(c, n - b0);
    uint64_t q0 = rdl64(P, owner);
    uint32_t qc0 = rdl32(PC, owner);
    unsigned todo = owned;
    for (int p0 = 0; p0 < cnt && todo; p0 += 64) {  // the owner's items, 64 at a time
      const int k = p0 + lane;
      uint64_t e = 0;
      uint32_t cc = 0;
      if (k < cnt) item_at(b0 + k, &e, &cc);
      const uint64_t q = q0 + wave_excl_scan_u64(e);
      const uint32_t qc = qc0 + wave_excl_scan_u32(cc);
      const unsigned now = k < cnt ? edge_conds<NE>(q, q + e, M) : 0u;
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        if ((todo >> j) & 1u) {
          const uint64_t m = wave_ballot((now >> j) & 1u);
          if (m != 0) {
            const int kk = __builtin_ctzll(m);
            r.x[j] = b0 + p0 + kk;
            r.P[j] = rdl64(q, kk);
            r.PC[j] = rdl32(qc, kk);
            todo &= ~(1u << j);
          }
        }
      }
      q0 = rdl64(q + e, 63);
      qc0 = rdl32(qc + cc, 63);
    }
    if (todo) {  // an owned edge not met: not the premise
      r.ok = false;
      return r;
    }
    pending &= ~owned;
  }
  return r;
}

// A crossing row staged in LDS by one wave: samples (zeros from w up to
// the lanes' last run), and each lane's run sums: the exact sum of its
// terms (float squares in units) and their odd count.
struct RowStage {
  uint16_t x[kStage];
  uint64_t runE[64];
  uint32_t runC[64];
};

// Samples of a row's term run: lane l takes chunks [l*cpl, l*cpl + cpl) of
// 8 samples, cpl = ceil(ceil(w / 8) / 64).
__device__ __forceinline__ int run_chunks(int w) { return (((w + 7) >> 3) + 63) >> 6; }

// Loads row i of the plane into st by one wave: each lane loads its own
// run (16-byte loads when the row allows them, kStageRound of them in
// flight at a time: one round for rows up to 4096 samples, two up to
// kStage) and sums its terms from the loaded registers.
__device__ void wave_stage_row(RowStage& st, int i, const void* plane, long stride, int w,
                               int bpc8) {
  const int lane = threadIdx.x & 63;
  const int cpl = run_chunks(w);
  uint64_t e = 0;
  uint32_t c = 0;
  if (!bpc8) {
    const uint16_t* row = (const uint16_t*)plane + (long)i * stride;
    if (((uintptr_t)row & 15) == 0 && (w & 7) == 0) {
      const int nv = w >> 3;
      for (int r0 = 0; r0 < cpl; r0 += kStageRound) {
        v4u v[kStageRound];
#pragma unroll
        for (int u = 0; u < kStageRound; ++u) {  // the round's loads issued before the first use
          const int cidx = lane * cpl + r0 + u;
          v[u] = r0 + u < cpl && cidx < nv ? ((const v4u*)row)[cidx] : (v4u){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kStageRound; ++u) {
          if (r0 + u < cpl) {
            ((v4u*)st.x)[lane * cpl + r0 + u] = v[u];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const uint32_t t = fsq_units((v[u][q >> 1] >> (16 * (q & 1))) & 0xFFFFu);
              e += t;
              c += t & 1u;
            }
          }
        }
      }
      st.runE[lane] = e;
      st.runC[lane] = c;
      return;
    }
    for (int j = lane * 8 * cpl, k = 0; k < 8 * cpl; ++j, ++k) {
      const uint32_t x = j < w ? row[j] : 0u;
      st.x[j] = (uint16_t)x;
      const uint32_t t = fsq_units(x);
      e += t;
      c += t & 1u;
    }
  } else {
    const uint8_t* row = (const uint8_t*)plane + (long)i * stride;
    for (int j = lane * 8 * cpl, k = 0; k < 8 * cpl; ++j, ++k) {
      const uint32_t x = j < w ? row[j] : 0u;
      st.x[j] = (uint16_t)x;
      const uint32_t t = fsq_units(x);
      e += t;
      c += t & 1u;
    }
  }
  st.runE[lane] = e;
  st.runC[lane] = c;
}

// The rows rr[0..2] of the plane (-1: none) staged in st[0..2] by the whole
// block, as wave_stage_row stages one: every thread loads its share of
// every row, coalesced, all loads in flight at once (16-byte chunks when
// the rows allow them, else sample by sample), with zeros from w up to the
// lanes' last run; after a block barrier, the eight threads [8l, 8l + 8) sum
// run l of each row (every eighth chunk each), joined by three DPP steps
// inside their group of eight lanes.  Ends with a block barrier: every
// thread of the block must call it, with the same rows.
__device__ void block_stage_rows(RowStage* st, const int* rr, const void* plane, long stride,
                                 int w, int bpc8) {
  const int t = threadIdx.x;
  const int cpl = run_chunks(w), nc = 64 * cpl;  // chunks held per row
  bool vec = !bpc8 && (w & 7) == 0;
  for (int r = 0; r < 3; ++r)
    if (rr[r] >= 0)
      vec = vec && ((uintptr_t)((const uint16_t*)plane + (long)rr[r] * stride) & 15) == 0;
  if (vec) {
    const int nv = w >> 3;
    constexpr int K = kStage / 8 / kT;  // chunks of a row per thread
    v4u v[3][K];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const v4u* row = (const v4u*)((const uint16_t*)plane + (long)max(rr[r], 0) * stride);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int c = t + k * kT;
        v[r][k] = rr[r] >= 0 && c < nv ? row[c] : (v4u){0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int c = t + k * kT;
        if (rr[r] >= 0 && c < nc) ((v4u*)st[r].x)[c] = v[r][k];
      }
  } else {
    for (int r = 0; r < 3; ++r) {
      if (rr[r] < 0) continue;
      for (int j = t; j < 8 * nc; j += kT) {
        uint32_t x = 0;
        if (j < w)
          x = bpc8 ? ((const uint8_t*)plane)[(long)rr[r] * stride + j]
                   : ((const uint16_t*)plane)[(long)rr[r] * stride + j];
        st[r].x[j] = (uint16_t)x;
      }
    }
  }
  __syncthreads();
  const int l = t >> 3, p = t & 7;
  for (int r = 0; r < 3; ++r) {
    if (rr[r] < 0) continue;
    uint64_t e = 0;
    uint32_t c = 0;
    for (int j = p; j < cpl; j += 8) {
      const v4u x = ((const v4u*)st[r].x)[l * cpl + j];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t tq = fsq_units((x[q >> 1] >> (16 * (q & 1))) & 0xFFFFu);
        e += tq;
        c += tq & 1u;
      }
    }
    e += dpp64<0xB1>(e);   // quad_perm [1,0,3,2]
    e += dpp64<0x4E>(e);   // quad_perm [2,3,0,1]
    e += dpp64<0x141>(e);  // row_half_mirror: the two quads of each group of eight
    c += dpp32<0xB1>(c);
    c += dpp32<0x4E>(c);
    c += dpp32<0x141>(c);
    if (p == 0) {
      st[r].runE[l] = e;
      st[r].runC[l] = c;
    }
  }
  __syncthreads();
}

// The pair, inside the binade of 2^55, of the terms [ia, b) of a row staged
// in st: lane l adds its share of its run (8-sample chunks [l*cpl, l*cpl +
// cpl), read 16 bytes at a time; a term outside [ia, b) counts as 0, which
// moves nothing) from both starts with the double add, and the lanes'
// pairs are joined in order.  Uniform.
__device__ Pair64 staged_pair55(const RowStage& st, int w, int ia, int b) {
  const int lane = threadIdx.x & 63;
  const int cpl = run_chunks(w);
  RunF64 r = run_start(55);
  uint64_t E = 0;
  for (int c = lane * cpl; c < lane * cpl + cpl; ++c) {
    const v4u x = ((const v4u*)st.x)[c];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int k = 8 * c + q;
      const uint32_t t =
          k >= ia && k < b ? fsq_units((x[q >> 1] >> (16 * (q & 1))) & 0xFFFFu) : 0u;
      E += t;
      run_add(r, (double)t);
    }
  }
  return wave_then(widen_pair(run_end(r, 55), E), 3);
}

// Row (staged in st) planned across an edge, from S = *sp: lane l takes
// the terms of its run, the terms' edges with margin w * u/2 (u the last
// place of the binade above S), closed forms, and the terms across an edge
// added with the double add (the CPU's step).  With seven edges (NE) the
// row's part inside the binade of 2^55 adds its pair from staged_pair55.
template <int NE = kEdges>
__device__ bool wave_cross_row(uint64_t* sp, const RowStage& st, int w) {
  const int lane = threadIdx.x & 63;
  const uint64_t s0 = *sp;
  const int L = 8 * run_chunks(w);
  const int a = min(lane * L, w), cl = min(L, w - a);
  const uint64_t le = st.runE[lane];
  const uint32_t lc = st.runC[lane];
  const uint64_t elast = cl > 0 ? fsq_units(st.x[a + cl - 1]) : 0;
  const int eB = (s0 < kTwo53 ? 53 : binade(s0)) + 1;
  const uint64_t Mr = (uint64_t)w << (eB - 53);
  const WEdgesN<NE> ed = wave_edges<NE>(w, L, le, lc, elast, s0, Mr, [&](int k, uint64_t* e, uint32_t* c) {
    const uint32_t x = fsq_units(st.x[k]);
    *e = x;
    *c = x & 1u;
  });
  if (!ed.ok) return false;
  uint64_t s = s0;
#pragma unroll
  for (int g = 0; g <= NE; ++g) {
    // the segment [ia, b) and the exact prefix and odd count at its start,
    // read from the edges (nothing carried from one segment to the next)
    const int ia = g == 0 ? 0 : ed.x[g > 0 ? g - 1 : 0], b = ed.x[g];
    const uint64_t Pa = g == 0 ? s0 : ed.P[g > 0 ? g - 1 : 0];
    const uint64_t PCa = g == 0 ? 0 : ed.PC[g > 0 ? g - 1 : 0];
    if (b < ia) return false;  // edges out of order: not the premise
    if (b > ia) {
      if (g == 1 || g == 3 || (NE == kEdges56 && g == 5)) {
        double d = (double)s;  // a value the CPU's double holds: exact
        for (int k = ia; k < b; ++k) d = d + (double)fsq_units(st.x[k]);
        s = (uint64_t)d;
      } else if (NE == kEdges56 && g == 6) {
        if (!try_apply(&s, staged_pair55(st, w, ia, b), 55)) return false;
      } else if (!fast_apply<NE>(&s, g, ed.P[g] - Pa, ed.PC[g] - PCa)) {
        return false;
      }
    }
  }
  *sp = s;
  return true;
}

// The fast walk of one plane: rows' exact sums and odd counts in lE / lC
// (LDS, h <= kChunk), and per block thread t the sums of rows [t*cs, t*cs +
// cs) in pe / pc; lane l takes the rows of threads [8l, 8l + 8).  Samples
// are read only for rows across an edge (w <= kStage).  Margin: with every
// sum below 2^55 the CPU's sum strays from the exact prefix by at most 2
// units per term added past 2^53.  With seven edges (NE, for a plane whose
// exact sum k_plan found in [2^55, 2^56)) the margin is 4 units per term
// (u/2 in the binade of 2^55), the rows across 2^55 are walked like the
// others, and the stretch inside the binade of 2^55 composes the rows'
// pairs that k_pairs left in rp (global, [row][2]): each lane a run of rows
// in order, then the lanes in order.
//
// In three steps: wave 0 finds the plane's edges (plane_edges), the block
// stages the first row of each stretch across an edge (block_stage_rows),
// then wave 0 walks the segments (walk_segments).

// The plane's edges, by one wave; ed.ok false when the plane is not the
// fast walk's (not the premise, or a sum past the form's last edge, or no
// pairs for a stretch in the binade of 2^55).
template <int NE = kEdges>
__device__ WEdgesN<NE> plane_edges(const uint64_t* lE, const uint16_t* lC, const uint64_t* pe,
                                   const uint32_t* pc, int cs, int h, int w,
                                   const uint64_t* rp) {
  const int lane = threadIdx.x & 63;
  constexpr int PER = kT / 64;
  const int c = PER * cs;
  const int a = min(lane * c, h), cl = min(c, h - a);
  uint64_t le = 0;
  uint32_t lc = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    le += pe[lane * PER + q];
    lc += pc[lane * PER + q];
  }
  const uint64_t elast = cl > 0 ? lE[a + cl - 1] : 0;
  const uint64_t M = (NE == kEdges56 ? 4ull : 2ull) * (uint64_t)w * (uint64_t)h;
  WEdgesN<NE> ed = wave_edges<NE>(h, c, le, lc, elast, 0, M, [&](int k, uint64_t* e, uint32_t* cc) {
    *e = lE[k];
    *cc = lC[k];
  });
  if (ed.P[NE] >= (NE == kEdges56 ? (1ull << 56) : (1ull << 55))) ed.ok = false;
  if (NE == kEdges56 && ed.x[5] < ed.x[6] && !rp) ed.ok = false;  // no pairs for the binade of 2^55
  return ed;
}

// The first row of each stretch across an edge (g = 1, 3 and, with seven
// edges, 5), or -1 where the stretch is empty.
template <int NE = kEdges>
__device__ __forceinline__ int across_row(const WEdgesN<NE>& ed, int k) {
  if (k == 2 && NE != kEdges56) return -1;
  return ed.x[2 * k] < ed.x[2 * k + 1] ? ed.x[2 * k] : -1;
}

// The segments in order, by one wave, from S = 0: st[k] holds row
// staged[k], the first row of stretch g = 2k + 1; a further row of such a
// stretch is staged by the wave in its turn.  Returns false when the plane
// needs the general walk.
template <int NE = kEdges>
__device__ bool walk_segments(uint64_t* out, const WEdgesN<NE>& ed, const uint64_t* lE,
                              const uint16_t* lC, const void* plane, long stride, int w, int bpc8,
                              RowStage* st, int* staged, const uint64_t* rp) {
  const int lane = threadIdx.x & 63;
  uint64_t s = 0;
#pragma unroll
  for (int g = 0; g <= NE; ++g) {
    // the segment [ia, b) and the exact prefix and odd count at its start,
    // read from the edges (nothing carried from one segment to the next)
    const int ia = g == 0 ? 0 : ed.x[g > 0 ? g - 1 : 0], b = ed.x[g];
    const uint64_t Pa = g == 0 ? 0 : ed.P[g > 0 ? g - 1 : 0];
    const uint64_t PCa = g == 0 ? 0 : ed.PC[g > 0 ? g - 1 : 0];
    if (b < ia) return false;  // edges out of order: not the premise
    if (b > ia) {
      if (g == 1 || g == 3 || (NE == kEdges56 && g == 5)) {
        RowStage& sg = st[g >> 1];
        for (int i = ia; i < b; ++i) {
          // a row that, from the actual S, adds exactly or stays inside its
          // binade needs no samples (rows of zeros after a crossing, say)
          if (try_exact(&s, lE[i])) continue;
          if (s >= kTwo53) {
            const int e = binade(s);
            if (e <= 54 && try_apply(&s, closed_pair(lE[i], lC[i], e), e)) continue;
          }
          if (i != staged[g >> 1]) {  // a further row of the stretch
            wave_lds_sync();
            wave_stage_row(sg, i, plane, stride, w, bpc8);
            wave_lds_sync();
            staged[g >> 1] = i;
          }
          if (!wave_cross_row<NE>(&s, sg, w)) return false;
        }
      } else if (NE == kEdges56 && g == 6) {
        // lane l composes rows [ia + l*rs, ...) in order, eight loads in flight
        const int rs = (b - ia + 63) >> 6;
        const int r0 = min(ia + lane * rs, b), r1 = min(r0 + rs, b);
        Pair64 acc = pair64_id();
        for (int i0 = r0; i0 < r1; i0 += 8) {
          Pair64 q[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            q[u] = i0 + u < r1 ? Pair64{rp[2 * (i0 + u)], rp[2 * (i0 + u) + 1]} : pair64_id();
#pragma unroll
          for (int u = 0; u < 8; ++u) acc = then64(acc, q[u], 3);
        }
        if (!try_apply(&s, wave_then(acc, 3), 55)) return false;
      } else if (!fast_apply<NE>(&s, g, ed.P[g] - Pa, ed.PC[g] - PCa)) {
        return false;
      }
    }
  }
  *out = s;
  return true;
}

// The fast walk by the whole block (every thread calls it): on success *S
// (the CPU's sum), *E (the exact sum) and *s1 (the first-moment sum, from
// pz) are set in wave 0.  xs: four ints of LDS for wave 0's word to the
// block; ok: an int of LDS.
template <int NE = kEdges>
__device__ bool block_fast_walk(uint64_t* S, uint64_t* E, uint64_t* s1, const RowLds& rows,
                                const uint64_t* pe, const uint32_t* pc, const uint64_t* pz,
                                int cs, int h, const void* plane, long stride, int w, int bpc8,
                                RowStage* st, const uint64_t* rp, int* xs, int* ok) {
  const int wave = threadIdx.x >> 6;
  WEdgesN<NE> ed;
  if (wave == 0) {
    ed = plane_edges<NE>(rows.R, rows.C, pe, pc, cs, h, w, rp);
    *E = ed.P[NE];
    uint64_t zz = 0;  // the first-moment sum, off the walk's path
#pragma unroll
    for (int q = 0; q < kT / 64; ++q) zz += pz[(threadIdx.x & 63) * (kT / 64) + q];
    *s1 = wave_sum_u64(zz);
    if (threadIdx.x == 0) {
      for (int k = 0; k < 3; ++k) xs[k] = across_row<NE>(ed, k);
      xs[3] = ed.ok;
    }
  }
  __syncthreads();
  if (!xs[3]) return false;  // uniform: every thread read the same word
  int staged[3] = {xs[0], xs[1], xs[2]};
  block_stage_rows(st, staged, plane, stride, w, bpc8);
  if (wave == 0) {
    const bool okw =
        walk_segments<NE>(S, ed, rows.R, rows.C, plane, stride, w, bpc8, st, staged, rp);
    if (threadIdx.x == 0) *ok = okw;
  }
  __syncthreads();
  return *ok != 0;
}

// The fast PSNR noise by one wave, over one chunk of n rows: their exact
// sums in lR (LDS, n <= kChunk) and per block thread t the sum of chunk rows
// [t*cs, t*cs + cs) in pe (lane l takes the rows of threads [8l, 8l + 8)).
// *sp is the CPU's running sum in units before the chunk (an integer its
// double holds) and P0 the exact sum of the rows before it; M bounds how far
// the CPU's sum strays from the exact prefix over the whole plane (2 per
// row: each add past 2^53 rounds by at most u/2 <= 2 units below 2^55).
// The same edges as the moment walk: exact rows added as integers, rows
// across an edge added with the double add, and each stretch of rows inside
// one binade applied as one pair composed in row order (the stretch spread
// evenly over the lanes, then an ordered tree).  On success *sp is the
// running sum after the chunk; *exact is the exact sum after it either
// way.  False when it does not apply.
__device__ bool wave_noise(uint64_t* sp, uint64_t* exact, const uint64_t* lR, const uint64_t* pe,
                           int cs, int n, uint64_t P0, uint64_t M) {
  const int lane = threadIdx.x & 63;
  constexpr int PER = kT / 64;
  const int c = PER * cs;
  const int a = min(lane * c, n), cl = min(c, n - a);
  uint64_t le = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) le += pe[lane * PER + q];
  const uint64_t elast = cl > 0 ? lR[a + cl - 1] : 0;
  const WEdges ed = wave_edges(n, c, le, 0u, elast, P0, M,
                               [&](int k, uint64_t* e, uint32_t* cc) {
                                 *e = lR[k];
                                 *cc = 0;
                               });
  *exact = ed.P[kEdges];
  if (!ed.ok || ed.P[kEdges] >= (1ull << 55)) return false;
  uint64_t s = *sp;
#pragma unroll
  for (int g = 0; g <= kEdges; ++g) {
    // the segment [ia, b) and the exact prefix at its start, read from the
    // edges (nothing carried from one segment to the next)
    const int ia = g == 0 ? 0 : ed.x[g > 0 ? g - 1 : 0], b = ed.x[g];
    const uint64_t Pa = g == 0 ? P0 : ed.P[g > 0 ? g - 1 : 0];
    if (b < ia) return false;  // edges out of order: not the premise
    if (b > ia) {
      const int ep = fast_plan(g);
      if (ep == kPlanExact) {
        if (!try_exact(&s, ed.P[g] - Pa)) return false;
      } else if (ep == kPlanCross) {
        double d = (double)s;  // a value the CPU's double holds: exact
        for (int i = ia; i < b; ++i) d = d + (double)lR[i];
        s = (uint64_t)d;
      } else if (ep == 53 || ep == 54) {
        const int sh = ep - 52;
        const int rs = (b - ia + 63) >> 6;
        const int r0 = min(ia + lane * rs, b), r1 = min(r0 + rs, b);
        Pair64 acc = pair64_id();
        for (int i = r0; i < r1; ++i) acc = then64(acc, noise_row_pair(lR[i], sh), sh);
        if (!try_apply(&s, wave_then(acc, sh), ep)) return false;
      } else {
        return false;
      }
    }
  }
  *sp = s;
  return true;
}

// The PSNR noise: rows added into a double in order.  Exact while the sum
// stays at or below 2^53 units; from the first row that takes it past, one
// hardware double add per row, as the CPU does (ADR-1499, Decision).  The
// rows go through LDS (stage, kChunk values) a chunk at a time.
__device__ double noise_chain(const uint64_t* RN, int h, BlockScratch& sm, uint64_t* stage,
                              uint64_t* exact) {
  uint64_t E = 0, p = 0;
  int first = h;
  uint64_t pfirst = 0;
  {
    const int c = (h + kT - 1) / kT;
    const int a = min((int)threadIdx.x * c, h), b = min(a + c, h);
    uint64_t loc = 0;
    for (int i = a; i < b; ++i) loc += RN[i];
    p = block_excl_scan_u64(loc, &E, sm);
    for (int i = a; i < b && first == h; ++i) {
      const uint64_t r = RN[i];
      if (p + r > kTwo53) {
        first = i;
        pfirst = p;
      }
      p += r;
    }
  }
  const int i0 = block_min_int(first, sm);
  *exact = E;
  if (i0 >= h) return (double)E;
  __syncthreads();
  if (first == i0) sm.v[0] = pfirst;
  __syncthreads();
  double d = (double)sm.v[0];  // exact: at most 2^53
  for (int base = i0; base < h; base += kChunk) {
    const int n = min(kChunk, h - base);
    __syncthreads();
    uint64_t v[kRowsPer];
#pragma unroll
    for (int q = 0; q < kRowsPer; ++q) {  // every load issued before the first store
      const int k = q * kT + (int)threadIdx.x;
      v[q] = k < n ? RN[base + k] : 0;
    }
#pragma unroll
    for (int q = 0; q < kRowsPer; ++q) {
      const int k = q * kT + (int)threadIdx.x;
      if (k < n) stage[k] = v[q];
    }
    __syncthreads();
    // the adds stay in row order; eight rows are read ahead of them
    int k = 0;
    for (; k + 8 <= n; k += 8) {
      double r[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) r[q] = (double)stage[k + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) d = d + r[q];
    }
    for (; k < n; ++k) d = d + (double)stage[k];
  }
  return d;
}

// The general walk of one plane (any geometry, any plan, every test mode):
// plan, then the Walker.  Not inlined: the common case never calls it.
__device__ __noinline__ void general_walk(const char* plane, long stride, int w, int h, int bpc8,
                                          const uint64_t* r2, const uint32_t* codd,
                                          const uint32_t* r1, int8_t* plan, uint64_t* pairs,
                                          const uint64_t* psum, unsigned dbg,
                                          BlockScratch& sm, RowLds& rows, RunLds& runs,
                                          Seg* rseg, Seg* useg, uint16_t* rowbuf, int* staged,
                                          uint64_t* res) {
  __syncthreads();
  uint64_t E, s1 = 0;
  if (psum) {  // planned by k_plan; the first chunk's rows come with the sums
    E = psum[0];
    s1 = psum[1];
    load_rows(rows, r2, codd, plan, 0, min(kChunk, h));
  } else {
    E = plan_plane(r2, plan, w, h, dbg, sm, &rows, codd, r1, &s1);
  }
  uint64_t S = E;
  if (may_round(E, dbg)) {
    if (threadIdx.x == 0) *staged = -1;
    __syncthreads();
    const Walker wk{plane, stride, w,   h,     bpc8, r2,   codd,  plan,   pairs,
                    dbg,   sm,     rows, runs, rseg, useg, rowbuf, staged};
    S = wk.walk_rows(!psum && h <= kChunk, psum != nullptr);
  }
  if (threadIdx.x == 0) {
    res[0] = S;
    res[1] = E;
    res[2] = s1;
  }
  __syncthreads();
}

// One 512-thread block per (frame, job): jobs 0 and 1 the moments of ref and
// dis, job 2 the PSNR noise (a call may ask for the moments or the noise
// alone: jobs [job0, job0 + njobs)).  Fast path: every thread loads the rows' sums
// into LDS, then wave 0 finds the plane's edges, the block stages the rows
// across them, and wave 0 alone walks the segments while the other waves
// wait at the next barrier (its walk has no block barrier); when it does
// not apply, the whole block takes the general walk.
__global__ void __launch_bounds__(kT) k_walk(Geometry g, RowArrays ra, double* results,
                                             uint64_t* units, unsigned dbg) {
  __shared__ BlockScratch sm;
  __shared__ RowLds rows;
  __shared__ RunLds runs;
  __shared__ Seg rseg[kMaxSeg + 1], useg[kMaxSeg + 1];
  __shared__ uint64_t pe[kT], pz[kT];
  __shared__ uint32_t pc[kT];
  // one buffer for both walks, which never run at once in a block: the
  // fast walk's two staged rows, or the row the general walk leaves its
  // plan in (a block barrier separates a failed fast walk from the general
  // walk)
  __shared__ __attribute__((aligned(16))) union RowBuf {
    RowStage stage[3];
    uint16_t wide[kRowMax];
  } rowbuf;
  static_assert(sizeof(RowStage) * 3 <= sizeof(uint16_t) * kRowMax,
                "staged rows fit the row buffer");
  __shared__ int xs[4];
  RowStage* const stage = rowbuf.stage;
  uint16_t* const wide_row = rowbuf.wide;
  __shared__ int staged, fast_ok;
  __shared__ uint64_t res[3];
  const int f = blockIdx.x / g.njobs, job = g.job0 + blockIdx.x % g.njobs;
  if (threadIdx.x == 0 && job == g.job0)  // jobs the call did not ask for
    for (int j = 0; j < 3; ++j)
      if (j < g.job0 || j >= g.job0 + g.njobs) ra.paths[3 * f + j] = kPathSkipped;
  const int k = g.bpc - 8;
  const double n = (double)g.w * (double)g.h;
  const int wave = threadIdx.x >> 6;
  // the fast path stops below 2^56: a plane k_plan has summed past it goes
  // straight to the general walk, and one it has summed into the binade of
  // 2^55 takes the fast path's seven-edge form
  const uint64_t planned_sum =
      g.planned && job < 2 ? ra.psum[2 * (job * g.nframes + f)] : 0;
  const bool try_fast = dbg == 0 && g.may_round && g.h <= kChunk && g.w <= kStage &&
                        planned_sum < (1ull << 56);
  if (job == 2) {
    uint64_t ex = 0;
    double d = 0.0;
    const uint64_t* RN = ra.rn + (long)f * g.h;
    bool fast = false;
    if (dbg == 0 && g.may_round) {
      // kChunk rows at a time: loaded into LDS by every thread, walked by
      // wave 0 from the running sum while the other waves wait at the barrier
      uint64_t srun = 0, P = 0;  // the CPU's running sum, the exact one
      bool ok = true;
      for (int base = 0; base < g.h && ok; base += kChunk) {
        const int nr = min(kChunk, g.h - base);
        const int cs = (nr + kT - 1) / kT, i0 = (int)threadIdx.x * cs;
        uint64_t v[kRowsPer];
#pragma unroll
        for (int q = 0; q < kRowsPer; ++q)  // every load issued before the first use
          v[q] = q < cs && i0 + q < nr ? RN[base + i0 + q] : 0;
        uint64_t e = 0;
#pragma unroll
        for (int q = 0; q < kRowsPer; ++q) {
          if (q < cs && i0 + q < nr) rows.R[i0 + q] = v[q];
          e += v[q];
        }
        pe[threadIdx.x] = e;
        __syncthreads();
        if (wave == 0) {
          const bool okc = wave_noise(&srun, &P, rows.R, pe, cs, nr, P, 2ull * (uint64_t)g.h);
          if (threadIdx.x == 0) fast_ok = okc;
        }
        __syncthreads();  // after it, rows.R and pe are free for the next chunk
        ok = fast_ok != 0;
      }
      if (ok) {
        d = (double)srun;  // an integer the CPU's double holds: exact
        ex = P;
        fast = true;
      }
    }
    if (!fast) d = noise_chain(RN, g.h, sm, rows.R, &ex);
    if (threadIdx.x == 0) {
      const double noise = d * (1.0 / (double)(1u << (2 * k)));
      results[6 * f + 4] = noise;
      results[6 * f + 5] = noise / n;
      units[8 * f + 6] = ex;
      units[8 * f + 7] = __builtin_bit_cast(uint64_t, d);
      ra.paths[3 * f + 2] = fast ? kPathFast : g.may_round ? kPathChain : kPathSums;
    }
    return;
  }
  const int pl = job;
  const long off = (long)(pl * g.nframes + f) * g.h;
  const char* plane =
      (const char*)(pl == 0 ? g.ref : g.dis) + (long)f * g.pitch * (g.bpc == 8 ? 1 : 2);
  uint64_t S = 0, E = 0, s1 = 0;
  uint8_t path = kPathSums;
  if (!g.may_round) {
    uint64_t a = 0, b = 0;
    for (int i = threadIdx.x; i < g.h; i += kT) {
      a += ra.r1[off + i];
      b += ra.r2[off + i];
    }
    s1 = block_sum_u64(a, sm);
    E = S = block_sum_u64(b, sm);
  } else {
    bool fast = false;
    if (try_fast) {
      // the rows' sums into LDS, coalesced, every load issued before the
      // first use; then each thread's contiguous run of cs rows from LDS
      const int cs = (g.h + kT - 1) / kT, i0 = (int)threadIdx.x * cs;
      uint64_t v[kRowsPer];
      uint32_t cv[kRowsPer], zv[kRowsPer];
#pragma unroll
      for (int q = 0; q < kRowsPer; ++q) {
        const int i = q * kT + (int)threadIdx.x;
        v[q] = i < g.h ? ra.r2[off + i] : 0;
        cv[q] = i < g.h ? ra.codd[off + i] : 0;
        zv[q] = i < g.h ? ra.r1[off + i] : 0;
      }
      uint64_t z = 0;
#pragma unroll
      for (int q = 0; q < kRowsPer; ++q) {
        const int i = q * kT + (int)threadIdx.x;
        if (i < g.h) {
          rows.R[i] = v[q];
          rows.C[i] = (uint16_t)cv[q];  // at most w <= kStage
        }
        z += zv[q];
      }
      __syncthreads();
      uint64_t e = 0;
      uint32_t c = 0;
      for (int q = 0; q < cs && i0 + q < g.h; ++q) {
        e += rows.R[i0 + q];
        c += rows.C[i0 + q];
      }
      pe[threadIdx.x] = e;
      pc[threadIdx.x] = c;
      pz[threadIdx.x] = z;
      __syncthreads();
      fast = planned_sum >= (1ull << 55)
                 ? block_fast_walk<kEdges56>(&S, &E, &s1, rows, pe, pc, pz, cs, g.h, plane,
                                             g.stride, g.w, g.bpc == 8, stage, ra.pairs + 2 * off,
                                             xs, &fast_ok)
                 : block_fast_walk<kEdges>(&S, &E, &s1, rows, pe, pc, pz, cs, g.h, plane,
                                           g.stride, g.w, g.bpc == 8, stage, nullptr, xs,
                                           &fast_ok);
    }
    path = fast ? kPathFast : kPathGeneral;
    if (!fast) {
      general_walk(plane, g.stride, g.w, g.h, g.bpc == 8, ra.r2 + off, ra.codd + off,
                   ra.r1 + off, ra.plan + off, ra.pairs + 2 * off,
                   g.planned ? ra.psum + 2 * (pl * g.nframes + f) : nullptr, dbg, sm, rows, runs,
                   rseg, useg, wide_row, &staged, res);
      S = res[0];
      E = res[1];
      s1 = res[2];
    }
  }
  if (threadIdx.x == 0) {
    const double m1 = ((double)s1 * (1.0 / (double)(1u << k))) / n;
    const double m2 = ((double)S * (1.0 / (double)(1u << (2 * k)))) / n;
    results[6 * f + pl] = m1;
    results[6 * f + 2 + pl] = m2;
    units[8 * f + pl] = s1;
    units[8 * f + 2 + pl] = E;
    units[8 * f + 4 + pl] = S;
    ra.paths[3 * f + pl] = path;
  }
}

// PSNR in dB of n planes-frames from their MSE (results[6 * k + 5]), read
// as 10 log10(peak^2 / MSE) with peak the largest normalised sample,
// (2^bpc - 1) / 2^(bpc - 8); MSE 0 gives +infinity.  The pages name the
// per-plane PSNR scores but give no formula (Metal kernel batch digest,
// Feature scope): this is the project's reading.
__global__ void __launch_bounds__(256) k_psnr_db(const double* results, int n, int bpc,
                                                 double* db) {
  const int k = (int)(blockIdx.x * 256 + threadIdx.x);
  if (k >= n) return;
  const double peak = (double)((1u << bpc) - 1u) / (double)(1u << (bpc - 8));
  db[k] = 10.0 * log10(peak * peak / results[6 * (long)k + 5]);
}

}  // namespace

namespace bef {

hipError_t launch_psnr_db(const double* results, int n, int bpc, double* db, hipStream_t st) {
  hipLaunchKernelGGL(k_psnr_db, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, results, n,
                     bpc, db);
  return hipGetLastError();
}

hipError_t launch_plan(const Geometry& g, const RowArrays& ra, unsigned dbg, hipStream_t st,
                       hipEvent_t ev0, hipEvent_t ev1) {
  hipExtLaunchKernelGGL(k_plan, dim3(2 * g.nframes), dim3(kT), 0, st, ev0, ev1, 0, g, ra, dbg);
  return hipGetLastError();
}

hipError_t launch_pairs(const Geometry& g, const RowArrays& ra, unsigned dbg, hipStream_t st,
                        hipEvent_t ev0, hipEvent_t ev1) {
  const long tasks = 2L * g.nframes * g.h;
  // 16-bit rows on 16-byte boundaries, whole 8-sample chunks: the pipelined pass
  const bool pipe = g.bpc != 8 && g.vec && (g.w & 7) == 0;
  const int rpb = pipe ? 4 * kPipeRows : 4;  // rows per block
  const long blocks = (tasks + rpb - 1) / rpb;
  // a dispatch's grid, in work-items, must stay below 2^32
  const long kMaxBlocks = (dbg & BEF_DBG_SPLIT_LAUNCH) ? 64 : 1L << 23;
  for (long b0 = 0; b0 < blocks; b0 += kMaxBlocks) {
    const unsigned nb = (unsigned)(blocks - b0 < kMaxBlocks ? blocks - b0 : kMaxBlocks);
    hipEvent_t e0 = b0 == 0 ? ev0 : nullptr, e1 = b0 + nb >= blocks ? ev1 : nullptr;
    const long t0 = b0 * rpb;
    if (pipe)
      hipExtLaunchKernelGGL(k_pairs_pipe, dim3(nb), dim3(256), 0, st, e0, e1, 0, g, ra, dbg, t0);
    else if (g.bpc == 8)
      hipExtLaunchKernelGGL(k_pairs<uint8_t>, dim3(nb), dim3(256), 0, st, e0, e1, 0, g, ra, dbg, t0);
    else
      hipExtLaunchKernelGGL(k_pairs<uint16_t>, dim3(nb), dim3(256), 0, st, e0, e1, 0, g, ra, dbg, t0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_walk(const Geometry& g, const RowArrays& ra, double* results, uint64_t* units,
                       unsigned dbg, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  hipExtLaunchKernelGGL(k_walk, dim3(g.njobs * g.nframes), dim3(kT), 0, st, ev0, ev1, 0, g, ra,
                        results, units, dbg);
  return hipGetLastError();
}

}  // namespace bef
