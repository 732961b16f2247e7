// load_shape.h -- the 16-bit row kernel's load shape for a geometry
// (host code, shared by the runtime and the host emulation's test entry
// point, which checks the choice).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace bef {

// Load shape of the 16-bit row kernel: bytes per load and load slots per
// lane per group.  Measured at rows of 1920, 2560 and 3840 samples, 8-byte
// loads beat 16- and 4-byte ones at every width, so the width is 8 bytes
// whenever the plane starts, the row pitch and the frame pitch allow it,
// else 4.  A wave spreads a row's whole chunks over its 64 lanes in groups
// of 64 * ng: the group size that leaves the fewest idle slots in the
// last group wins (an idle slot still costs its arithmetic, on zeros), then
// the larger group (more loads in flight, fewer rounds).
inline void load_shape(const void* ref, const void* dis, int w, ptrdiff_t stride,
                       ptrdiff_t pitch, int nframes, int* cb_out, int* ng_out) {
  uint64_t al = 16;
  auto limit = [&](uint64_t v) {
    while (al > 1 && v % al) al >>= 1;
  };
  limit((uintptr_t)ref);
  limit((uintptr_t)dis);
  limit((uint64_t)stride * 2);
  if (nframes > 1) limit((uint64_t)pitch * 2);
  int cb = 0;
  for (int c : {8, 4})
    if (!cb && (uint64_t)c <= al && (uint64_t)w * 2 / c > 0) cb = c;
  int best_ng = 1;
  if (cb) {
    const uint64_t nc = (uint64_t)w * 2 / cb;
    const uint64_t nper = (nc + 63) / 64;
    uint64_t best_idle = ~0ull;
    for (int ng : {15, 8, 5, 4}) {
      const uint64_t idle = ((nper + ng - 1) / ng) * ng * 64 - nc;
      if (idle < best_idle) best_ng = ng, best_idle = idle;
    }
  }
  *cb_out = cb;
  *ng_out = best_ng;
}

}  // namespace bef
