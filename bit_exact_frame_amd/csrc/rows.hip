// rows.hip -- the streaming pass: per-row exact integer sums.
//
// k_rows16 / k_rows8: one wave per (row, frame).  The wave reads the row of
// both planes once (16-byte nontemporal loads when rows are aligned), forms
// every term in registers and writes, per row: the sum of codewords of each
// plane, the exact sum of float squares of each plane (units of 1/s^2), the
// exact noise sum (float squares of ref - dis) and the number of odd float
// squares.  Per-row exact sums: ADR-1497 Decision (each row's exact sum) and
// ADR-1499 Decision (blocks of one row, exact 64-bit row sums).  No atomics:
// every row sum has one owner.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bef_internal.h"
#include "ordsum.h"
#include "wave.h"

using namespace bef;

namespace {

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

constexpr int kRowsU = 4;  // 16-byte loads in flight per lane per plane

template <bool ODD, bool VEC>
__device__ __forceinline__ void rows16_body(const Geometry& g, const RowArrays& ra, int i, int f,
                                            int lane);

template <bool ODD, bool VEC>
__global__ void __launch_bounds__(256) k_rows16(Geometry g, RowArrays ra) {
  const int lane = threadIdx.x & 63;
  const long task = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= (long)g.nframes * g.h) return;  // whole wave leaves together
  const int i = (int)(task / g.nframes), f = (int)(task % g.nframes);
  // The odd-square count is only read for rows past 2^53; a row whose
  // prefix cannot reach 2^53 even with every sample at 65535 skips it.
  if (ODD && (uint64_t)(i + 1) * (uint64_t)g.w * 0xFFFE0000ull > kTwo53)
    rows16_body<true, VEC>(g, ra, i, f, lane);
  else
    rows16_body<false, VEC>(g, ra, i, f, lane);
}

template <bool ODD, bool VEC>
__device__ __forceinline__ void rows16_body(const Geometry& g, const RowArrays& ra, int i, int f,
                                            int lane) {
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

}  // namespace

namespace bef {

hipError_t launch_rows(const Geometry& g, const RowArrays& ra, hipStream_t st, hipEvent_t ev0,
                       hipEvent_t ev1) {
  const long tasks = (long)g.nframes * g.h;
  const unsigned blocks = (unsigned)((tasks + 3) / 4);
  if (g.bpc == 8) {
    hipExtLaunchKernelGGL(k_rows8, dim3(blocks), dim3(256), 0, st, ev0, ev1, 0, g, ra);
  } else if (g.need_odd) {
    if (g.vec) hipExtLaunchKernelGGL((k_rows16<true, true>), dim3(blocks), dim3(256), 0, st, ev0, ev1, 0, g, ra);
    else hipExtLaunchKernelGGL((k_rows16<true, false>), dim3(blocks), dim3(256), 0, st, ev0, ev1, 0, g, ra);
  } else {
    if (g.vec) hipExtLaunchKernelGGL((k_rows16<false, true>), dim3(blocks), dim3(256), 0, st, ev0, ev1, 0, g, ra);
    else hipExtLaunchKernelGGL((k_rows16<false, false>), dim3(blocks), dim3(256), 0, st, ev0, ev1, 0, g, ra);
  }
  return hipGetLastError();
}

}  // namespace bef
