// wave.h -- 64-lane wavefront reductions and scans for the gfx950 kernels.
//
// Within each 16-lane row of a wave: DPP quad_perm xor-1, quad_perm xor-2,
// row_half_mirror and row_mirror; across the four rows: lanes 15, 31, 47 and
// 63 read into scalars.  64-bit values move as two 32-bit halves and are
// added with carry.  Every result is uniform over the wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp32<0xB1>(v));
  v = min(v, dpp32<0x4E>(v));
  v = min(v, dpp32<0x141>(v));
  v = min(v, dpp32<0x140>(v));
  return min(min(rdl32(v, 15), rdl32(v, 31)), min(rdl32(v, 47), rdl32(v, 63)));
}

// Shift within each 16-lane row by CTRL (row_shr:k); lanes whose source is
// outside the row, or rows not in ROWMASK, read 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp64_or0(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWMASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWMASK, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp32_or0(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWMASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes: row_shr 1, 2, 4, 8 inside each row
// of 16 lanes, then row_bcast:15 into rows 1 and 3 and row_bcast:31 into
// rows 2 and 3.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  v += dpp64_or0<0x111, 0xF>(v);
  v += dpp64_or0<0x112, 0xF>(v);
  v += dpp64_or0<0x114, 0xF>(v);
  v += dpp64_or0<0x118, 0xF>(v);
  v += dpp64_or0<0x142, 0xA>(v);
  v += dpp64_or0<0x143, 0xC>(v);
  return v;
}

__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp32_or0<0x111, 0xF>(v);
  v += dpp32_or0<0x112, 0xF>(v);
  v += dpp32_or0<0x114, 0xF>(v);
  v += dpp32_or0<0x118, 0xF>(v);
  v += dpp32_or0<0x142, 0xA>(v);
  v += dpp32_or0<0x143, 0xC>(v);
  return v;
}

__device__ __forceinline__ uint64_t wave_excl_scan_u64(uint64_t v) {
  return wave_incl_scan_u64(v) - v;
}
__device__ __forceinline__ uint32_t wave_excl_scan_u32(uint32_t v) {
  return wave_incl_scan_u32(v) - v;
}

// Lanes whose predicate holds (bit l = lane l); uniform.
__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// The value held by lane (l - 1) (lane 0 reads its own).
__device__ __forceinline__ uint64_t lane_before_u64(uint64_t v) {
  const int lane = threadIdx.x & 63;
  const int addr = (lane > 0 ? lane - 1 : 0) << 2;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Orders this wave's earlier LDS writes before its later LDS reads (LDS
// serves one wave's accesses in order; this keeps the compiler from
// moving them).  No other wave is involved.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace
