// kernels.hip -- gfx950 kernels of the bit-exact frame reductions.
//
// Pipeline for a batch of frames (all on the caller's stream):
//   k_rows     one wave per (row, frame): reads the row of both planes once
//              (16-byte loads), forms every term in registers and writes the
//              row's exact integer sums: sum of x per plane, sum of float
//              squares per plane, noise sum, and the count of odd squares.
//              Per-row sums: ADR-1497 Decision (each row's exact sum);
//              ADR-1499 Decision (blocks of one row, exact 64-bit row sums).
//   k_plan     (only for frames that can pass 2^55 units) exact row prefix
//              and per-row binade plan, for k_pairs.
//   k_pairs    (same condition) the row's pair under its planned binade:
//              64 lane runs joined by an ordered tree (ADR-1497 Decision).
//   k_walk     one 256-thread block per (frame, plane) walks the rows in
//              order: exact adds up to 2^53, stretches of rows that share a
//              planned binade applied as one composed pair, unfit rows
//              split into 256 runs, unfit runs added term by term (ADR-1497
//              Decision); one block per frame adds the noise rows into a
//              double in row order (ADR-1499 Decision); then the divisions.
//
// Units: 1/s^2 for squares, 1/s for first moments (s = 2^(bpc-8)).  No
// atomics anywhere: every sum has one owner and a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bef_internal.h"
#include "ordsum.h"

using namespace bef;

namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Wave-level reductions (64 lanes).  Within each 16-lane row: DPP
// quad_perm xor-1, quad_perm xor-2, row_half_mirror, row_mirror; across the
// four rows: lanes 15, 31, 47 and 63 read into scalars.  64-bit values move
// as two 32-bit halves and are added with carry.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = dpp32<CTRL>((uint32_t)v), hi = dpp32<CTRL>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t rdl32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ __forceinline__ uint64_t rdl64(uint64_t v, int lane) {
  return ((uint64_t)rdl32((uint32_t)(v >> 32), lane) << 32) | rdl32((uint32_t)v, lane);
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  v += dpp64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp64<0x141>(v);  // row_half_mirror
  v += dpp64<0x140>(v);  // row_mirror
  return rdl64(v, 15) + rdl64(v, 31) + rdl64(v, 47) + rdl64(v, 63);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp32<0xB1>(v);
  v += dpp32<0x4E>(v);
  v += dpp32<0x141>(v);
  v += dpp32<0x140>(v);
  return rdl32(v, 15) + rdl32(v, 31) + rdl32(v, 47) + rdl32(v, 63);
}
// Doubles holding integers below 2^53: every partial sum is exact, so the
// order of this tree does not matter.
__device__ __forceinline__ double wave_sum_f64i(double x) {
  uint64_t b = __builtin_bit_cast(uint64_t, x);
#define BEF_DSTEP(C)                                                \
  {                                                                 \
    const double o = __builtin_bit_cast(double, dpp64<C>(b));       \
    x += o;                                                         \
    b = __builtin_bit_cast(uint64_t, x);                            \
  }
  BEF_DSTEP(0xB1) BEF_DSTEP(0x4E) BEF_DSTEP(0x141) BEF_DSTEP(0x140)
#undef BEF_DSTEP
  const double a0 = __builtin_bit_cast(double, rdl64(b, 15));
  const double a1 = __builtin_bit_cast(double, rdl64(b, 31));
  const double a2 = __builtin_bit_cast(double, rdl64(b, 47));
  const double a3 = __builtin_bit_cast(double, rdl64(b, 63));
  return (a0 + a1) + (a2 + a3);
}

// ---------------------------------------------------------------------------
// k_rows: per-row exact sums.

struct Acc16 {
  double m2r0, m2r1, m2d0, m2d1, mn0, mn1;  // float squares, exact in f64
  uint32_t s1r, s1d;                        // first-moment sums
  us2 oddr, oddd;                           // odd squares (per half-word)
};

// Two 16-bit samples of each plane.
template <bool ODD>
__device__ __forceinline__ void take_dword16(uint32_t a, uint32_t b, Acc16& q) {
  const uint32_t a0 = a & 0xFFFFu, a1 = a >> 16, b0 = b & 0xFFFFu, b1 = b >> 16;
  const float fa0 = (float)a0, fa1 = (float)a1, fb0 = (float)b0, fb1 = (float)b1;
  q.m2r0 += (double)__fmul_rn(fa0, fa0);
  q.m2r1 += (double)__fmul_rn(fa1, fa1);
  q.m2d0 += (double)__fmul_rn(fb0, fb0);
  q.m2d1 += (double)__fmul_rn(fb1, fb1);
  const float e0 = (float)((int32_t)a0 - (int32_t)b0);
  const float e1 = (float)((int32_t)a1 - (int32_t)b1);
  q.mn0 += (double)__fmul_rn(e0, e0);
  q.mn1 += (double)__fmul_rn(e1, e1);
  q.s1r = __builtin_amdgcn_udot2(__builtin_bit_cast(us2, a), (us2){1, 1}, q.s1r, false);
  q.s1d = __builtin_amdgcn_udot2(__builtin_bit_cast(us2, b), (us2){1, 1}, q.s1d, false);
  if (ODD) {
    // A float square is odd exactly when x is odd and below 4096:
    // min(x, 4096) & 1.
    const us2 cap = {4096, 4096}, one = {1, 1};
    q.oddr += __builtin_elementwise_min(__builtin_bit_cast(us2, a), cap) & one;
    q.oddd += __builtin_elementwise_min(__builtin_bit_cast(us2, b), cap) & one;
  }
}

template <bool ODD>
__device__ __forceinline__ void take_sample16(uint32_t a, uint32_t b, Acc16& q) {
  const float fa = (float)a, fb = (float)b;
  q.m2r0 += (double)__fmul_rn(fa, fa);
  q.m2d0 += (double)__fmul_rn(fb, fb);
  const float e = (float)((int32_t)a - (int32_t)b);
  q.mn0 += (double)__fmul_rn(e, e);
  q.s1r += a;
  q.s1d += b;
  if (ODD) {
    q.oddr.x += (unsigned short)((a < 4096u ? a : 4096u) & 1u);
    q.oddd.x += (unsigned short)((b < 4096u ? b : 4096u) & 1u);
  }
}

constexpr int kRowsU = 8;  // 16-byte loads in flight per lane per plane

template <bool ODD, bool VEC>
__global__ void __launch_bounds__(256) k_rows16(Geometry g, RowArrays ra) {
  const int lane = threadIdx.x & 63;
  const long task = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= (long)g.nframes * g.h) return;  // whole wave leaves together
  const int i = (int)(task / g.nframes), f = (int)(task % g.nframes);
  const uint16_t* rr = (const uint16_t*)g.ref + (long)f * g.pitch + (long)i * g.stride;
  const uint16_t* dr = (const uint16_t*)g.dis + (long)f * g.pitch + (long)i * g.stride;
  Acc16 q = {0, 0, 0, 0, 0, 0, 0u, 0u, {0, 0}, {0, 0}};
  int j0 = 0;
  if (VEC) {
    const int nv = g.w >> 3;  // 8 samples per 16-byte vector
    const v4u* rv = (const v4u*)rr;
    const v4u* dv = (const v4u*)dr;
    for (int base = 0; base < nv; base += 64 * kRowsU) {
      v4u a[kRowsU], b[kRowsU];
#pragma unroll
      for (int u = 0; u < kRowsU; ++u) {
        const int c = base + u * 64 + lane;
        if (c < nv) {
          a[u] = __builtin_nontemporal_load(rv + c);
          b[u] = __builtin_nontemporal_load(dv + c);
        } else {
          a[u] = (v4u){0u, 0u, 0u, 0u};  // zero samples add nothing
          b[u] = (v4u){0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < kRowsU; ++u) {
        take_dword16<ODD>(a[u].x, b[u].x, q);
        take_dword16<ODD>(a[u].y, b[u].y, q);
        take_dword16<ODD>(a[u].z, b[u].z, q);
        take_dword16<ODD>(a[u].w, b[u].w, q);
      }
    }
    j0 = nv << 3;
  }
  for (int j = j0 + lane; j < g.w; j += 64) take_sample16<ODD>(rr[j], dr[j], q);

  const double m2r = wave_sum_f64i(q.m2r0 + q.m2r1);
  const double m2d = wave_sum_f64i(q.m2d0 + q.m2d1);
  const double mn = wave_sum_f64i(q.mn0 + q.mn1);
  const uint32_t s1r = wave_sum_u32(q.s1r), s1d = wave_sum_u32(q.s1d);
  uint32_t odr = 0, odd = 0;
  if (ODD) {
    odr = wave_sum_u32((uint32_t)q.oddr.x + q.oddr.y);
    odd = wave_sum_u32((uint32_t)q.oddd.x + q.oddd.y);
  }
  if (lane == 0) {
    const long k = (long)f * g.h + i, k2 = (long)(g.nframes + f) * g.h + i;
    ra.r1[k] = s1r;
    ra.r1[k2] = s1d;
    ra.r2[k] = (uint64_t)m2r;
    ra.r2[k2] = (uint64_t)m2d;
    ra.rn[k] = (uint64_t)mn;
    ra.codd[k] = odr;
    ra.codd[k2] = odd;
  }
}

// 8-bit planes: squares are exact integers (x <= 255), summed with 4-way
// byte dot products; the noise is r^2 + d^2 - 2rd per pixel, exactly.
__global__ void __launch_bounds__(256) k_rows8(Geometry g, RowArrays ra) {
  const int lane = threadIdx.x & 63;
  const long task = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= (long)g.nframes * g.h) return;
  const int i = (int)(task / g.nframes), f = (int)(task % g.nframes);
  const uint8_t* rr = (const uint8_t*)g.ref + (long)f * g.pitch + (long)i * g.stride;
  const uint8_t* dr = (const uint8_t*)g.dis + (long)f * g.pitch + (long)i * g.stride;
  uint32_t s1r = 0, s1d = 0, s2r = 0, s2d = 0, x = 0;
  int j0 = 0;
  if (g.vec) {
    const int nv = g.w >> 4;
    const uint4* rv = (const uint4*)rr;
    const uint4* dv = (const uint4*)dr;
    for (int c = lane; c < nv; c += 64) {
      const uint4 a = rv[c], b = dv[c];
      const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s1r = __builtin_amdgcn_udot4(av[k], 0x01010101u, s1r, false);
        s1d = __builtin_amdgcn_udot4(bv[k], 0x01010101u, s1d, false);
        s2r = __builtin_amdgcn_udot4(av[k], av[k], s2r, false);
        s2d = __builtin_amdgcn_udot4(bv[k], bv[k], s2d, false);
        x = __builtin_amdgcn_udot4(av[k], bv[k], x, false);
      }
    }
    j0 = nv << 4;
  }
  for (int j = j0 + lane; j < g.w; j += 64) {
    const uint32_t a = rr[j], b = dr[j];
    s1r += a;
    s1d += b;
    s2r += a * a;
    s2d += b * b;
    x += a * b;
  }
  const uint32_t S1r = wave_sum_u32(s1r), S1d = wave_sum_u32(s1d);
  const uint64_t S2r = wave_sum_u64(s2r), S2d = wave_sum_u64(s2d), X = wave_sum_u64(x);
  if (lane == 0) {
    const long k = (long)f * g.h + i, k2 = (long)(g.nframes + f) * g.h + i;
    ra.r1[k] = S1r;
    ra.r1[k2] = S1d;
    ra.r2[k] = S2r;
    ra.r2[k2] = S2d;
    ra.rn[k] = S2r + S2d - 2 * X;
    ra.codd[k] = 0;
    ra.codd[k2] = 0;
  }
}

// ---------------------------------------------------------------------------
// Block-level helpers (256 threads = 4 waves).  Every thread calls them with
// the same arguments; results are uniform.

struct BlockScratch {
  uint64_t w64[8];
  uint64_t v[4];
  int iv[4];
};

__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, BlockScratch& sm) {
  const uint64_t s = wave_sum_u64(v);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.w64[wv] = s;
  __syncthreads();
  return sm.w64[0] + sm.w64[1] + sm.w64[2] + sm.w64[3];
}

__device__ __forceinline__ int block_min_int(int v, BlockScratch& sm) {
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.iv[threadIdx.x >> 6] = v;
  __syncthreads();
  return min(min(sm.iv[0], sm.iv[1]), min(sm.iv[2], sm.iv[3]));
}

// Exclusive prefix of v over the block's threads in order; *total = sum.
__device__ __forceinline__ uint64_t block_excl_scan_u64(uint64_t v, uint64_t* total,
                                                        BlockScratch& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t inc = v;
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  __syncthreads();
  if (lane == 63) sm.w64[wv] = inc;
  __syncthreads();
  uint64_t before = 0;
  for (int k = 0; k < wv; ++k) before += sm.w64[k];
  *total = sm.w64[0] + sm.w64[1] + sm.w64[2] + sm.w64[3];
  return before + inc - v;
}

// Ordered composition of one pair per thread (thread 0 first): a
// shuffle-down tree inside each wave, then (w0 then w1) then (w2 then w3).
__device__ __forceinline__ Pair64 block_then(Pair64 p, int sh, BlockScratch& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int off = 1; off < 64; off <<= 1) {
    Pair64 o;
    o.a0 = __shfl_down(p.a0, off);
    o.a1 = __shfl_down(p.a1, off);
    if ((lane & (2 * off - 1)) == 0) p = then64(p, o, sh);
  }
  __syncthreads();
  if (lane == 0) {
    sm.w64[2 * wv] = p.a0;
    sm.w64[2 * wv + 1] = p.a1;
  }
  __syncthreads();
  const Pair64 w0 = {sm.w64[0], sm.w64[1]}, w1 = {sm.w64[2], sm.w64[3]};
  const Pair64 w2 = {sm.w64[4], sm.w64[5]}, w3 = {sm.w64[6], sm.w64[7]};
  return then64(then64(w0, w1, sh), then64(w2, w3, sh), sh);
}

// ---------------------------------------------------------------------------
// Plan (shared by k_plan and k_walk): exact exclusive prefix of the rows'
// second-moment sums and each row's plan.  Writes P[], plan[]; returns the
// plane's exact total.

__device__ int debug_plan(int e, int i, unsigned dbg) {
  if (e >= 53 && (dbg & BEF_DBG_PLAN_NONE)) return kPlanCross;
  if (e >= 53 && (dbg & BEF_DBG_PLAN_WRONG)) return (i & 1) ? (e > 53 ? e - 1 : e + 2) : e + 1;
  return e;
}

__device__ uint64_t plan_plane(const uint64_t* R, uint64_t* P, int8_t* plan, int w, int h,
                               unsigned dbg, BlockScratch& sm) {
  uint64_t carry = 0;
  for (int base = 0; base < h; base += 256) {
    const int i = base + threadIdx.x;
    const uint64_t r = i < h ? R[i] : 0;
    uint64_t tot;
    const uint64_t ex = block_excl_scan_u64(r, &tot, sm);
    if (i < h) P[i] = carry + ex;
    carry += tot;
  }
  const uint64_t E = carry;
  const uint64_t M = E > kTwo53 ? ((uint64_t)w * (uint64_t)h) << (binade(E) - 53) : 0;
  __syncthreads();
  for (int i = threadIdx.x; i < h; i += 256) plan[i] = (int8_t)debug_plan(plan_of(P[i], R[i], M), i, dbg);
  __syncthreads();
  return E;
}

__device__ __forceinline__ bool may_round(uint64_t E, unsigned dbg) {
  return E > kTwo53 || (dbg & BEF_DBG_FORCE_ROUND);
}

__global__ void __launch_bounds__(256) k_plan(Geometry g, RowArrays ra, unsigned dbg) {
  __shared__ BlockScratch sm;
  const int f = blockIdx.x >> 1, pl = blockIdx.x & 1;
  const long off = (long)(pl * g.nframes + f) * g.h;
  plan_plane(ra.r2 + off, ra.prefix + off, ra.plan + off, g.w, g.h, dbg, sm);
}

// ---------------------------------------------------------------------------
// k_pairs: the pair of a row under its planned binade, from 64 lane runs of
// ceil(w/64) consecutive terms joined by an ordered shuffle-down tree.

__device__ __forceinline__ bool needs_pair(int e, unsigned dbg) {
  return e >= 55 || (e >= 53 && (dbg & BEF_DBG_NO_CLOSED_FORM));
}

template <typename T>
__global__ void __launch_bounds__(256) k_pairs(Geometry g, RowArrays ra, unsigned dbg) {
  const int lane = threadIdx.x & 63;
  const long task = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long per = 2L * g.nframes;
  if (task >= per * g.h) return;
  const int i = g.h - 1 - (int)(task / per);  // last rows first
  const int rem = (int)(task % per);
  const int pl = rem / g.nframes, f = rem % g.nframes;
  const long k = (long)(pl * g.nframes + f) * g.h + i;
  const int e = ra.plan[k];
  if (!needs_pair(e, dbg)) return;
  const int sh = e - 52;
  const T* row = (const T*)(pl == 0 ? g.ref : g.dis) + (long)f * g.pitch + (long)i * g.stride;
  const int L = (g.w + 63) >> 6;
  const int j0 = min(lane * L, g.w), j1 = min(j0 + L, g.w);
  Pair32 p = run_pair([&](int j) { return fsq_units(row[j0 + j]); }, j1 - j0, sh);
  for (int off = 1; off < 64; off <<= 1) {
    Pair32 o;
    o.a0 = __shfl_down(p.a0, off);
    o.a1 = __shfl_down(p.a1, off);
    if ((lane & (2 * off - 1)) == 0) p = then32(p, o, sh);
  }
  if (lane == 0) {
    const Pair64 q = widen_pair(p, ra.r2[k]);
    ra.pairs[2 * k] = q.a0;
    ra.pairs[2 * k + 1] = q.a1;
  }
}

// ---------------------------------------------------------------------------
// k_walk.

struct RunLds {
  uint64_t E[256];
  uint64_t A0[256], A1[256], B0[256], B1[256];
  int8_t plan[256];
};

template <typename T>
struct Walker {
  const T* row0;  // plane of this frame
  long stride;
  int w, h;
  const uint64_t* R;
  const uint32_t* C;
  const uint64_t* pairs;
  const int8_t* plan;
  unsigned dbg;
  BlockScratch& sm;
  RunLds& rl;

  __device__ uint32_t term(int i, int j) const { return fsq_units(row0[(long)i * stride + j]); }

  // Pair of row i under its plan e (e >= 53): closed form in the binades of
  // 2^53 and 2^54, else from k_pairs.
  //
  // Closed form: every float square in units is 0 or 1 modulo 4 (an odd
  // square is 1 mod 8; an even one is a multiple of 4; squares past 2^24
  // are rounded to multiples of 2 whose significand is even, or coarser).
  // In the binade of 2^53 (last place 2) an even term is exact and leaves
  // S/2's parity alone, and an odd term is a tie: from S = 0 mod 4 it goes
  // down by 1, from S = 2 mod 4 up by 1, and leaves S = 0 mod 4.  So with c
  // odd terms the row adds R - c from an even start and R - c + 2 from an
  // odd one (R from both when c = 0).  In the binade of 2^54 (last place 4)
  // an odd term is 1 mod 4, below half a place: it goes down by 1 whatever
  // the parity, so both starts add R - c.
  __device__ Pair64 row_pair(int i, int e) const {
    if (e <= 54 && !(dbg & BEF_DBG_NO_CLOSED_FORM)) {
      const uint64_t c = C[i];
      const uint64_t a0 = R[i] - c;
      const uint64_t a1 = (e == 53 && c > 0) ? a0 + 2 : a0;
      return Pair64{a0, a1};
    }
    return Pair64{pairs[2 * (long)i], pairs[2 * (long)i + 1]};
  }

  __device__ uint64_t terms(uint64_t s, int i, int j0, int j1) const {
    for (int j = j0; j < j1; ++j) s = rne53_add(s, term(i, j));
    return s;
  }

  // First item index >= i+1 whose plan differs from e (n if none).
  template <class PlanAt>
  __device__ int segment_end(int i, int n, int e, PlanAt plan_at) const {
    for (int base = i + 1; base < n; base += 256) {
      const int k = base + threadIdx.x;
      const int hit = (k < n && plan_at(k) != e) ? k : n;
      const int m = block_min_int(hit, sm);
      if (m < n) return m;
    }
    return n;
  }

  // Items [a, b): each thread folds a contiguous chunk, then block tree.
  template <class PairAt>
  __device__ Pair64 compose_range(int a, int b, int sh, PairAt pair_at) const {
    const int c = (b - a + 255) >> 8;
    Pair64 acc = pair64_id();
    const int k0 = a + threadIdx.x * c;
    for (int k = k0; k < k0 + c && k < b; ++k) acc = then64(acc, pair_at(k), sh);
    return block_then(acc, sh, sm);
  }

  template <class EAt>
  __device__ uint64_t sum_range(int a, int b, EAt e_at) const {
    uint64_t v = 0;
    for (int k = a + threadIdx.x; k < b; k += 256) v += e_at(k);
    return block_sum_u64(v, sm);
  }

  // The walk over n items (rows or runs): stretches first, item steps when
  // a stretch does not fit.
  template <class PlanAt, class EAt, class PairAt, class Step>
  __device__ uint64_t walk(uint64_t s, int n, PlanAt plan_at, EAt e_at, PairAt pair_at,
                           Step step) const {
    int i = 0;
    while (i < n) {
      const int e = plan_at(i);
      const int j = segment_end(i, n, e, plan_at);
      bool done = false;
      if (e == kPlanExact) {
        done = try_exact(&s, sum_range(i, j, e_at));
      } else if (e >= 53 && !(dbg & BEF_DBG_NO_STRETCH)) {
        done = try_apply(&s, compose_range(i, j, e - 52, pair_at), e);
      }
      if (!done)
        for (int k = i; k < j; ++k) s = step(s, k);
      i = j;
    }
    return s;
  }

  // A row the plan does not fit, from S: 256 runs of ceil(w/256) terms with
  // their pairs under the binade S is in and the next one, planned from their
  // own exact prefix; a run that fits neither is added term by term.
  __device__ uint64_t fallback_row(uint64_t s, int i) const {
    if (dbg & BEF_DBG_TERMS_ONLY) return terms(s, i, 0, w);
    const int eA = s < kTwo53 ? 53 : binade(s);
    const int eB = eA + 1;
    const int L = (w + 255) >> 8;
    const int t = threadIdx.x;
    const int j0 = min(t * L, w), j1 = min(j0 + L, w);
    uint64_t E = 0;
    for (int j = j0; j < j1; ++j) E += term(i, j);
    auto tt = [&](int j) { return term(i, j0 + j); };
    const Pair64 pA = widen_pair(run_pair(tt, j1 - j0, eA - 52), E);
    const Pair64 pB = widen_pair(run_pair(tt, j1 - j0, eB - 52), E);
    uint64_t tot;
    const uint64_t q = s + block_excl_scan_u64(E, &tot, sm);
    const uint64_t Mr = (uint64_t)w << (eB - 53);
    __syncthreads();
    rl.E[t] = E;
    rl.A0[t] = pA.a0;
    rl.A1[t] = pA.a1;
    rl.B0[t] = pB.a0;
    rl.B1[t] = pB.a1;
    rl.plan[t] = (int8_t)plan_of(q, E, Mr);
    __syncthreads();
    const RunLds& r = rl;
    const uint64_t out = walk(
        s, 256, [&](int k) { return (int)r.plan[k]; }, [&](int k) { return r.E[k]; },
        [&](int k) {
          return r.plan[k] == eA ? Pair64{r.A0[k], r.A1[k]} : Pair64{r.B0[k], r.B1[k]};
        },
        [&](uint64_t s2, int k) {
          if (try_exact(&s2, r.E[k])) return s2;
          if (try_apply(&s2, Pair64{r.A0[k], r.A1[k]}, eA)) return s2;
          if (try_apply(&s2, Pair64{r.B0[k], r.B1[k]}, eB)) return s2;
          const int a = min(k * L, w);
          return terms(s2, i, a, min(a + L, w));
        });
    __syncthreads();  // rl is reused by the next fallback
    return out;
  }

  __device__ uint64_t walk_rows() const {
    return walk(
        0, h, [&](int i) { return (int)plan[i]; }, [&](int i) { return R[i]; },
        [&](int i) { return row_pair(i, plan[i]); },
        [&](uint64_t s, int i) {
          if (try_exact(&s, R[i])) return s;
          const int e = plan[i];
          if (e >= 53 && try_apply(&s, row_pair(i, e), e)) return s;
          return fallback_row(s, i);
        });
  }
};

// The PSNR noise: rows added into a double in order.  Exact while the sum
// stays at or below 2^53 units; from the first row that takes it past, one
// hardware double add per row, as the CPU does (ADR-1499, Decision).
__device__ double noise_chain(const uint64_t* RN, int h, BlockScratch& sm, uint64_t* exact) {
  __shared__ uint64_t stage[256];
  uint64_t carry = 0;
  int first = h;
  for (int base = 0; base < h; base += 256) {
    const int i = base + threadIdx.x;
    const uint64_t r = i < h ? RN[i] : 0;
    uint64_t tot;
    const uint64_t ex = carry + block_excl_scan_u64(r, &tot, sm);
    const int hit = (i < h && first == h && ex + r > kTwo53) ? i : h;
    const int m = block_min_int(hit, sm);
    if (first == h && m < h) first = m;
    carry += tot;
  }
  *exact = carry;
  if (first == h) return (double)carry;
  // exact prefix before the first row that passes 2^53
  uint64_t pre = 0;
  for (int i = threadIdx.x; i < first; i += 256) pre += RN[i];
  pre = block_sum_u64(pre, sm);
  double d = (double)pre;
  for (int base = first; base < h; base += 256) {
    const int n = min(256, h - base);
    __syncthreads();
    if ((int)threadIdx.x < n) stage[threadIdx.x] = RN[base + threadIdx.x];
    __syncthreads();
    for (int k = 0; k < n; ++k) d = d + (double)stage[k];
  }
  return d;
}

template <typename T>
__global__ void __launch_bounds__(256) k_walk(Geometry g, RowArrays ra, double* results,
                                              uint64_t* units, unsigned dbg) {
  __shared__ BlockScratch sm;
  __shared__ RunLds rl;
  const int f = blockIdx.x / 3, job = blockIdx.x % 3;
  const int k = g.bpc - 8;
  const double n = (double)g.w * (double)g.h;
  if (job == 2) {
    uint64_t ex;
    const double d = noise_chain(ra.rn + (long)f * g.h, g.h, sm, &ex);
    if (threadIdx.x == 0) {
      const double noise = d * (1.0 / (double)(1u << (2 * k)));
      results[6 * f + 4] = noise;
      results[6 * f + 5] = noise / n;
      units[8 * f + 6] = ex;
      units[8 * f + 7] = __builtin_bit_cast(uint64_t, d);
    }
    return;
  }
  const int pl = job;
  const long off = (long)(pl * g.nframes + f) * g.h;
  uint64_t s1 = 0;
  for (int i = threadIdx.x; i < g.h; i += 256) s1 += ra.r1[off + i];
  s1 = block_sum_u64(s1, sm);
  const uint64_t E = plan_plane(ra.r2 + off, ra.prefix + off, ra.plan + off, g.w, g.h, dbg, sm);
  uint64_t S = E;
  if (g.may_round && may_round(E, dbg)) {
    const Walker<T> wk{(const T*)(pl == 0 ? g.ref : g.dis) + (long)f * g.pitch,
                       g.stride, g.w, g.h, ra.r2 + off, ra.codd + off, ra.pairs + 2 * off,
                       ra.plan + off, dbg, sm, rl};
    S = wk.walk_rows();
  }
  if (threadIdx.x == 0) {
    const double m1 = ((double)s1 * (1.0 / (double)(1u << k))) / n;
    const double m2 = ((double)S * (1.0 / (double)(1u << (2 * k)))) / n;
    results[6 * f + pl] = m1;
    results[6 * f + 2 + pl] = m2;
    units[8 * f + pl] = s1;
    units[8 * f + 2 + pl] = E;
    units[8 * f + 4 + pl] = S;
  }
}

}  // namespace

namespace bef {

hipError_t launch_rows(const Geometry& g, const RowArrays& ra, hipStream_t st) {
  const long tasks = (long)g.nframes * g.h;
  const unsigned blocks = (unsigned)((tasks + 3) / 4);
  if (g.bpc == 8) {
    hipLaunchKernelGGL(k_rows8, dim3(blocks), dim3(256), 0, st, g, ra);
  } else if (g.need_odd) {
    if (g.vec) hipLaunchKernelGGL((k_rows16<true, true>), dim3(blocks), dim3(256), 0, st, g, ra);
    else hipLaunchKernelGGL((k_rows16<true, false>), dim3(blocks), dim3(256), 0, st, g, ra);
  } else {
    if (g.vec) hipLaunchKernelGGL((k_rows16<false, true>), dim3(blocks), dim3(256), 0, st, g, ra);
    else hipLaunchKernelGGL((k_rows16<false, false>), dim3(blocks), dim3(256), 0, st, g, ra);
  }
  return hipGetLastError();
}

hipError_t launch_plan(const Geometry& g, const RowArrays& ra, unsigned dbg, hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(2 * g.nframes), dim3(256), 0, st, g, ra, dbg);
  return hipGetLastError();
}

hipError_t launch_pairs(const Geometry& g, const RowArrays& ra, unsigned dbg, hipStream_t st) {
  const long tasks = 2L * g.nframes * g.h;
  const unsigned blocks = (unsigned)((tasks + 3) / 4);
  if (g.bpc == 8) hipLaunchKernelGGL(k_pairs<uint8_t>, dim3(blocks), dim3(256), 0, st, g, ra, dbg);
  else hipLaunchKernelGGL(k_pairs<uint16_t>, dim3(blocks), dim3(256), 0, st, g, ra, dbg);
  return hipGetLastError();
}

hipError_t launch_walk(const Geometry& g, const RowArrays& ra, double* results, uint64_t* units,
                       unsigned dbg, hipStream_t st) {
  if (g.bpc == 8)
    hipLaunchKernelGGL(k_walk<uint8_t>, dim3(3 * g.nframes), dim3(256), 0, st, g, ra, results,
                       units, dbg);
  else
    hipLaunchKernelGGL(k_walk<uint16_t>, dim3(3 * g.nframes), dim3(256), 0, st, g, ra, results,
                       units, dbg);
  return hipGetLastError();
}

}  // namespace bef
