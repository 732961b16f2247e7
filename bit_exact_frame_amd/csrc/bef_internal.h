// bef_internal.h -- types shared by the kernels and the host runtime.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bef.h"

namespace bef {

// One batch of frames: geometry in samples, device plane pointers.
struct Geometry {
  const void* ref;
  const void* dis;
  int w, h;
  long stride;   // samples between rows
  long pitch;    // samples between frames
  int nframes;
  int bpc;
  int vec;       // rows start on 16-byte boundaries (8-bit kernel)
  int cb;        // 16-bit kernel: bytes per load (8, 4; 0 = sample by sample)
  int ng;        // 16-bit kernel: load slots per lane per group (4, 5, 8, 15)
  int need_odd;  // count odd squares per row (frames that can pass 2^53)
  int may_round; // some frame can pass 2^53 units (or forced)
  int planned;   // k_plan runs before the walk (plan and psum filled)
  int job0, njobs;  // walk jobs [job0, job0 + njobs) of 0 ref moments, 1 dis moments, 2 noise
};

// Device scratch, [plane][frame][row] (plane 0 = ref, 1 = dis) unless noted.
struct RowArrays {
  uint32_t* r1;     // sum of codewords
  uint64_t* r2;     // exact sum of float squares, units
  uint64_t* rn;     // [frame][row] exact noise sum, units
  uint32_t* codd;   // number of odd float squares
  int8_t* plan;     // kPlanExact, kPlanCross or a binade
  uint64_t* pairs;  // [plane][frame][row][2] row pair (binades >= 55)
  uint64_t* psum;   // [plane][frame][2] exact plane sums of r2 and r1 (by k_plan)
  uint8_t* paths;   // [frame][3] path each walk block took (kPath*), diagnostics
};

// Walk paths, per (frame, job), jobs ref moments, dis moments, noise.
constexpr uint8_t kPathSums = 0;     // no sum can pass 2^53: exact sums only
constexpr uint8_t kPathFast = 1;     // the one-wave fast path (moments or noise)
constexpr uint8_t kPathGeneral = 2;  // the general walk (moments)
constexpr uint8_t kPathChain = 3;    // the row-by-row double chain (noise)
constexpr uint8_t kPathSkipped = 4;  // the call asked for no result of this job

// Each launch goes out with hipExtLaunchKernel; ev0 / ev1 (or null) are
// recorded by the dispatch itself at the kernel's start and end.
hipError_t launch_rows(const Geometry& g, const RowArrays& ra, hipStream_t st, hipEvent_t ev0,
                       hipEvent_t ev1);
hipError_t launch_plan(const Geometry& g, const RowArrays& ra, unsigned dbg, hipStream_t st,
                       hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_pairs(const Geometry& g, const RowArrays& ra, unsigned dbg, hipStream_t st,
                        hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_read_ceiling(const Geometry& g, uint32_t* out, hipStream_t st, hipEvent_t ev0,
                               hipEvent_t ev1);
hipError_t launch_psnr_db(const double* results, int n, int bpc, double* db, hipStream_t st);
hipError_t launch_walk(const Geometry& g, const RowArrays& ra, double* results, uint64_t* units,
                       unsigned dbg, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace bef
