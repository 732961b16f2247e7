// rows.hip -- the streaming pass: per-row exact integer sums.
//
// k_rows16 / k_rows8: one wave per (row, frame).  The wave reads the row of
// both planes once (8-byte nontemporal loads when the rows allow them, else
// 4-byte ones), forms
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
  uint32_t ob;          // odd squares, per byte: ref even, ref odd, dis even, dis odd
  uint32_t oddr, oddd;  // odd squares, flushed from ob
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
    // A float square is odd exactly when x is odd and below 4096, i.e. when
    // min(x, 4096) is odd.  The low bytes of the four capped samples go to
    // one word (a byte permute) and their low bits into byte counters.
    const us2 cap = {4096, 4096};
    const uint32_t ma = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(us2, a), cap));
    const uint32_t mb = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(us2, b), cap));
    // v_perm_b32 picks bytes of {mb, ma} (ma = bytes 0-3): the low bytes of
    // ma's two halves, then of mb's
    const uint32_t lo = __builtin_amdgcn_perm(mb, ma, 0x06040200u);
    q.ob += lo & 0x01010101u;
  }
}

// Byte counters into the plane counts (before any byte can reach 256).
__device__ __forceinline__ void flush_odd(Acc16& q) {
  q.oddr = __builtin_amdgcn_udot4(q.ob, 0x00000101u, q.oddr, false);
  q.oddd = __builtin_amdgcn_udot4(q.ob, 0x01010000u, q.oddd, false);
  q.ob = 0;
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
    q.oddr += (a < 4096u ? a : 4096u) & 1u;
    q.oddd += (b < 4096u ? b : 4096u) & 1u;
  }
}

// Loads of CB bytes (8 or 4), NG of them per plane per lane per group.
template <int CB>
struct Chunk;
template <>
struct Chunk<8> {
  typedef uint32_t T __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ uint32_t dw(const T& v, int k) { return v[k]; }
};
template <>
struct Chunk<4> {
  typedef uint32_t T;
  static __device__ __forceinline__ uint32_t dw(const T& v, int) { return v; }
};

template <bool ODD, int CB, int NG>
__device__ __forceinline__ void rows16_body(const Geometry& g, const RowArrays& ra, int i, int f,
                                            int lane);

// CB bytes per load (8 or 4; 0 = sample by sample, for rows not aligned to
// 4 bytes), NG load slots per lane per group (4, 5, 8 or 15).
template <bool ODD, int CB, int NG>
__global__ void __launch_bounds__(256) k_rows16(Geometry g, RowArrays ra) {
  const int lane = threadIdx.x & 63;
  // grid (ceil(h / 4), frames): wave w of block x takes row 4x + w of frame y
  // (row and frame are wave-uniform scalars)
  const int i = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int f = (int)blockIdx.y;
  if (i >= g.h) return;  // whole wave leaves together
  // The odd-square count is only read for rows past 2^53; a row whose
  // prefix cannot reach 2^53 even with every sample at 65535 skips it.
  if (ODD && (uint64_t)(i + 1) * (uint64_t)g.w * 0xFFFE0000ull > kTwo53)
    rows16_body<true, CB, NG>(g, ra, i, f, lane);
  else
    rows16_body<false, CB, NG>(g, ra, i, f, lane);
}

template <bool ODD, int CB, int NG>
__device__ __forceinline__ void rows16_body(const Geometry& g, const RowArrays& ra, int i, int f,
                                            int lane) {
  const uint16_t* rr = (const uint16_t*)g.ref + (long)f * g.pitch + (long)i * g.stride;
  const uint16_t* dr = (const uint16_t*)g.dis + (long)f * g.pitch + (long)i * g.stride;
  Acc16 q = {0, 0, 0, 0, 0, 0, 0u, 0u, 0u, 0u, 0u};
  int j0 = 0;
  if constexpr (CB > 0) {
    typedef typename Chunk<CB>::T T;
    const int nc = (g.w * 2) / CB;     // whole chunks in the row
    const int nper = (nc + 63) >> 6;   // chunk slots per lane
    const T* rv = (const T*)rr;
    const T* dv = (const T*)dr;
    for (int g0 = 0; g0 < nper; g0 += NG) {
      T a[NG], b[NG];
      if ((g0 + NG) * 64 <= nc) {  // uniform: a full group, every load unconditional
#pragma unroll
        for (int u = 0; u < NG; ++u) {
          a[u] = __builtin_nontemporal_load(rv + (g0 + u) * 64 + lane);
          b[u] = __builtin_nontemporal_load(dv + (g0 + u) * 64 + lane);
        }
      } else {  // the row's last group: clamped loads, zeroed past the end
#pragma unroll
        for (int u = 0; u < NG; ++u) {
          const int c = (g0 + u) * 64 + lane, cc = c < nc ? c : nc - 1;
          const T x = __builtin_nontemporal_load(rv + cc), y = __builtin_nontemporal_load(dv + cc);
          a[u] = c < nc ? x : T{};  // zero samples add nothing
          b[u] = c < nc ? y : T{};
        }
      }
#pragma unroll
      for (int u = 0; u < NG; ++u)
#pragma unroll
        for (int k = 0; k < CB / 4; ++k)
          take_dword16<ODD>(Chunk<CB>::dw(a[u], k), Chunk<CB>::dw(b[u], k), q);
      if (ODD) flush_odd(q);
    }
    j0 = nc * (CB / 2);
  }
  for (int j = j0 + lane; j < g.w; j += 64) take_sample16<ODD>(rr[j], dr[j], q);

  const double m2r = wave_sum_f64i(q.m2r0 + q.m2r1);
  const double m2d = wave_sum_f64i(q.m2d0 + q.m2d1);
  const double mn = wave_sum_f64i(q.mn0 + q.mn1);
  const uint32_t s1r = wave_sum_u32(q.s1r), s1d = wave_sum_u32(q.s1d);
  uint32_t odr = 0, odd = 0;
  if (ODD) {
    // both counts in one word: each is at most w <= 32768 < 2^16
    const uint32_t both = wave_sum_u32(q.oddr | (q.oddd << 16));
    odr = both & 0xFFFFu;
    odd = both >> 16;
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

// The memory side of the 16-bit row pass alone: the same grid, load shape
// and nontemporal loads, with the arithmetic replaced by an XOR of the
// loaded words (one word per row written to out[frame][row]).  A
// diagnostic: the practical read ceiling of this access pattern.
template <int CB, int NG>
__global__ void __launch_bounds__(256) k_read_ceiling(Geometry g, uint32_t* out) {
  typedef typename Chunk<CB>::T T;
  const int lane = threadIdx.x & 63;
  const int i = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int f = (int)blockIdx.y;
  if (i >= g.h) return;
  const T* rv = (const T*)((const uint16_t*)g.ref + (long)f * g.pitch + (long)i * g.stride);
  const T* dv = (const T*)((const uint16_t*)g.dis + (long)f * g.pitch + (long)i * g.stride);
  const int nc = (g.w * 2) / CB, nper = (nc + 63) >> 6;
  uint32_t acc = 0;
  for (int g0 = 0; g0 < nper; g0 += NG) {
    T a[NG], b[NG];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int c = (g0 + u) * 64 + lane, cc = c < nc ? c : nc - 1;
      a[u] = __builtin_nontemporal_load(rv + cc);
      b[u] = __builtin_nontemporal_load(dv + cc);
    }
#pragma unroll
    for (int u = 0; u < NG; ++u)
#pragma unroll
      for (int k = 0; k < CB / 4; ++k) acc ^= Chunk<CB>::dw(a[u], k) + Chunk<CB>::dw(b[u], k);
  }
  acc = wave_sum_u32(acc);
  if (lane == 0) out[(long)f * g.h + i] = acc;
}

// 8-bit planes: squares are exact integers (x <= 255), summed with 4-way
// byte dot products; the noise is r^2 + d^2 - 2rd per pixel, exactly.
__global__ void __launch_bounds__(256) k_rows8(Geometry g, RowArrays ra) {
  const int lane = threadIdx.x & 63;
  // grid (ceil(h / 4), frames), as the 16-bit kernel
  const int i = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int f = (int)blockIdx.y;
  if (i >= g.h) return;
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
  const dim3 grid16((unsigned)((g.h + 3) / 4), (unsigned)g.nframes);
  if (g.bpc == 8) {
    hipExtLaunchKernelGGL(k_rows8, grid16, dim3(256), 0, st, ev0, ev1, 0, g, ra);
  } else {
#define BEF_ROWS16(CB, NG)                                                                  \
  if (g.need_odd)                                                                             \
    hipExtLaunchKernelGGL((k_rows16<true, CB, NG>), grid16, dim3(256), 0, st, ev0, ev1,       \
                          0, g, ra);                                                          \
  else                                                                                        \
    hipExtLaunchKernelGGL((k_rows16<false, CB, NG>), grid16, dim3(256), 0, st, ev0, ev1,      \
                          0, g, ra)
    switch (g.cb * 16 + g.ng) {
      case 8 * 16 + 4: BEF_ROWS16(8, 4); break;
      case 8 * 16 + 5: BEF_ROWS16(8, 5); break;
      case 8 * 16 + 8: BEF_ROWS16(8, 8); break;
      case 8 * 16 + 15: BEF_ROWS16(8, 15); break;
      case 4 * 16 + 4: BEF_ROWS16(4, 4); break;
      case 4 * 16 + 5: BEF_ROWS16(4, 5); break;
      case 4 * 16 + 8: BEF_ROWS16(4, 8); break;
      case 4 * 16 + 15: BEF_ROWS16(4, 15); break;
      default: BEF_ROWS16(0, 1); break;
    }
#undef BEF_ROWS16
  }
  return hipGetLastError();
}

hipError_t launch_read_ceiling(const Geometry& g, uint32_t* out, hipStream_t st, hipEvent_t ev0,
                               hipEvent_t ev1) {
  const dim3 grid((unsigned)((g.h + 3) / 4), (unsigned)g.nframes);
#define BEF_CEIL(CB, NG)                                                                       \
  hipExtLaunchKernelGGL((k_read_ceiling<CB, NG>), grid, dim3(256), 0, st, ev0, ev1, 0, g, out)
  switch (g.cb * 16 + g.ng) {
    case 8 * 16 + 4: BEF_CEIL(8, 4); break;
    case 8 * 16 + 5: BEF_CEIL(8, 5); break;
    case 8 * 16 + 8: BEF_CEIL(8, 8); break;
    case 8 * 16 + 15: BEF_CEIL(8, 15); break;
    case 4 * 16 + 4: BEF_CEIL(4, 4); break;
    case 4 * 16 + 5: BEF_CEIL(4, 5); break;
    case 4 * 16 + 8: BEF_CEIL(4, 8); break;
    case 4 * 16 + 15: BEF_CEIL(4, 15); break;
    default: return hipErrorInvalidValue;  // no whole chunks: nothing to measure
  }
#undef BEF_CEIL
  return hipGetLastError();
}

}  // namespace bef
