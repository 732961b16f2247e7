// bef.cpp -- host runtime behind include/bef.h: argument checks, device
// scratch, the launch sequence on the caller's stream, read-back.
//
// Every step of the reductions runs in the kernels (rows.hip, walk.hip), the final
// divisions included; the host only validates, allocates scratch, launches
// and copies the per-frame results back.
#include <errno.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "bef_internal.h"
#include "load_shape.h"
#include "ordsum.h"

using namespace bef;

// Scratch of bef_frames_noalloc: a device array of fixed size in the
// library's code object, one copy per GPU, held until the process ends.
// Host code never uses the name itself (on the host it is only a stand-in
// symbol): each device's address comes from hipGetSymbolAddress, taken
// once per device with that device current, and goes to the kernels as an
// argument, as the arena's base does.
static constexpr size_t kStaticScratchBytes = 16ull << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

std::mutex g_mu;
thread_local char g_err[512];
unsigned g_dbg = 0;

constexpr int kMaxDev = 64;
constexpr int kMaxPlanes = 4;  // planes of one bef_planes call
constexpr int kPipeRowQ = 2;   // row streams of pipelined batches
constexpr int kPipeSlots = 8;  // scratch slots of pipelined batches
// A pipelined batch whose planes hold at most this many bytes runs whole on
// the walk stream: its row pass is too short to overlap anything, and the
// handoff between streams would cost the host more than the batch takes.
constexpr double kPipeSmallBytes = 1 << 20;

struct Layout {
  size_t r1, r2, rn, codd, plan, pairs, psum, results, units, paths, total;
  // results, units and paths are copied back together: bytes from results
  size_t readback() const { return total - results; }
};

struct Call {
  Geometry g;
  int dev;
  Layout L;
  RowArrays ra;
  double* d_results;
  uint64_t* d_units;
  bool need_pairs;
};

struct Arena {
  void* base = nullptr;
  size_t cap = 0;
  void* host = nullptr;  // pinned read-back staging
  size_t host_cap = 0;
  // frames from host memory: two device slots, two streams, their events
  void* pipe = nullptr;
  size_t pipe_cap = 0;
  hipStream_t copy_st = nullptr, comp_st = nullptr;
  hipEvent_t copied[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr};
  // pipelined batches: row streams on most CUs, a walk stream on the
  // others, scratch slots used in turn
  hipStream_t prow[kPipeRowQ] = {};
  hipStream_t pwalk = nullptr;
  int pwalk_cus = 0;
  hipEvent_t penter = nullptr, pjoin = nullptr;
  hipEvent_t prowdone[kPipeSlots] = {}, pwalkdone[kPipeSlots] = {};
  void* pslot = nullptr;  // kPipeSlots slots
  size_t pslot_cap = 0;   // bytes per slot
  unsigned long long pn = 0;  // batches submitted
};
Arena g_arena[kMaxDev];

// CUs reserved for the walk stream of pipelined batches.
int g_pipe_walk_cus = 16;

// Walk paths of the last synchronous batch (bef_walk_paths).
std::vector<uint8_t> g_paths;

// Per-device address of the static scratch (below), taken once per device.
void* g_static_ptr[kMaxDev] = {};

// Kernel timing (events recorded on the launch stream).
struct EvPair {
  int kernel;
  hipEvent_t a, b;
};
bool g_timing = false;
std::vector<EvPair> g_ev_live;
std::vector<hipEvent_t> g_ev_pool;
double g_ms[5] = {0, 0, 0, 0, 0};
long g_n[5] = {0, 0, 0, 0, 0};

int fail(int rc, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return rc;
}

void clear_err() { g_err[0] = 0; }

#define BEF_HIP(call)                                                              \
  do {                                                                             \
    const hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) return fail(-EIO, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

int validate(const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
             ptrdiff_t pitch, int nframes, int bpc) {
  if (!ref || !dis) return fail(-EINVAL, "NULL plane pointer");
  if (w <= 0 || h <= 0 || w > 32768 || h > 32768)
    return fail(-EINVAL, "w=%d h=%d outside 1..32768", w, h);
  if (stride < w) return fail(-EINVAL, "stride %ld < w %d", (long)stride, w);
  if (bpc < 8 || bpc > 16) return fail(-EINVAL, "bpc %d outside 8..16", bpc);
  if (nframes <= 0 || nframes > 65535) return fail(-EINVAL, "nframes %d outside 1..65535", nframes);
  if (pitch < 0) return fail(-EINVAL, "negative frame pitch");
  if (nframes > 1 && pitch == 0) return fail(-EINVAL, "frame pitch 0 with several frames");
  return 0;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(int F, int h) {
  const size_t rows = (size_t)F * h;
  Layout L;
  size_t o = 0;
  L.r1 = o; o = up256(o + 2 * rows * 4);
  L.r2 = o; o = up256(o + 2 * rows * 8);
  L.rn = o; o = up256(o + rows * 8);
  L.codd = o; o = up256(o + 2 * rows * 4);
  L.plan = o; o = up256(o + 2 * rows);
  L.pairs = o; o = up256(o + 4 * rows * 8);
  L.psum = o; o = up256(o + (size_t)F * 4 * 8);
  L.results = o; o = up256(o + (size_t)F * 6 * 8);
  L.units = o; o = up256(o + (size_t)F * 8 * 8);
  L.paths = o; o = up256(o + (size_t)F * 3);
  L.total = o;
  return L;
}

int ensure(int dev, size_t bytes, size_t host_bytes) {
  Arena& a = g_arena[dev];
  if (a.cap < bytes) {
    if (a.base) BEF_HIP(hipFree(a.base));
    a.base = nullptr;
    a.cap = 0;
    if (hipMalloc(&a.base, bytes) != hipSuccess) {
      (void)hipGetLastError();
      a.base = nullptr;
      return fail(-ENOMEM, "hipMalloc of %zu bytes of scratch failed", bytes);
    }
    a.cap = bytes;
  }
  if (a.host_cap < host_bytes) {
    if (a.host) BEF_HIP(hipHostFree(a.host));
    a.host = nullptr;
    a.host_cap = 0;
    if (hipHostMalloc(&a.host, host_bytes, hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      a.host = nullptr;
      return fail(-ENOMEM, "hipHostMalloc of %zu bytes failed", host_bytes);
    }
    a.host_cap = host_bytes;
  }
  return 0;
}

int device_of(const void* p, int* dev) {
  hipPointerAttribute_t at;
  memset(&at, 0, sizeof at);
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(-EINVAL, "plane pointer %p is not device memory (%s)", p, hipGetErrorString(e));
  }
  if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged)
    return fail(-EINVAL, "plane pointer %p is not device memory", p);
  if (at.device < 0 || at.device >= kMaxDev) return fail(-EINVAL, "device %d out of range", at.device);
  *dev = at.device;
  return 0;
}

hipEvent_t ev_get() {
  if (!g_ev_pool.empty()) {
    hipEvent_t e = g_ev_pool.back();
    g_ev_pool.pop_back();
    return e;
  }
  // timing only: read after the stream is synchronised, so no system-scope
  // fence (its cache writeback would land inside the measured intervals)
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Drain finished event pairs into the totals (blocking on each).
void ev_collect() {
  for (EvPair& p : g_ev_live) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      g_ms[p.kernel] += ms;
      g_n[p.kernel] += 1;
    }
    g_ev_pool.push_back(p.a);
    g_ev_pool.push_back(p.b);
  }
  g_ev_live.clear();
}

// launch(ev0, ev1): the events (null when timing is off) go with the
// dispatch, so the interval is the kernel's own execution.
template <class F>
hipError_t timed(int kernel, F launch) {
  if (!g_timing) return launch(nullptr, nullptr);
  hipEvent_t a = ev_get(), b = ev_get();
  if (!a || !b) return launch(nullptr, nullptr);
  const hipError_t e = launch(a, b);
  g_ev_live.push_back(EvPair{kernel, a, b});
  return e;
}

// Arguments, device and geometry of a call; allocates nothing.
int setup(Call& c, const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
          ptrdiff_t pitch, int nframes, int bpc) {
  int rc = validate(ref, dis, w, h, stride, pitch, nframes, bpc);
  if (rc) return rc;
  int dev2 = 0;
  if ((rc = device_of(ref, &c.dev)) || (rc = device_of(dis, &dev2))) return rc;
  if (dev2 != c.dev) return fail(-EINVAL, "ref and dis on different devices");
  BEF_HIP(hipSetDevice(c.dev));
  const int B = bpc == 8 ? 1 : 2;
  Geometry& g = c.g;
  g.ref = ref;
  g.dis = dis;
  g.w = w;
  g.h = h;
  g.stride = (long)stride;
  g.pitch = (long)pitch;
  g.nframes = nframes;
  g.bpc = bpc;
  g.vec = ((uintptr_t)ref % 16 == 0) && ((uintptr_t)dis % 16 == 0) &&
          ((long)stride * B) % 16 == 0 && (nframes == 1 || ((long)pitch * B) % 16 == 0);
  g.cb = 0;
  g.ng = 1;
  if (bpc != 8) load_shape(ref, dis, w, stride, pitch, nframes, &g.cb, &g.ng);
  // Largest possible exact plane sum: every sample at the container's top.
  const uint64_t tmax = bpc == 8 ? 65025ull : 0xFFFE0000ull;
  const uint64_t maxsum = (uint64_t)w * (uint64_t)h * tmax;
  const bool force = (g_dbg & BEF_DBG_FORCE_ROUND) != 0;
  g.may_round = (maxsum > kTwo53) || force;
  g.need_odd = g.may_round && bpc != 8;
  g.job0 = 0;
  g.njobs = 3;
  c.need_pairs = g.may_round && (maxsum >= (1ull << 55) || g_dbg != 0);
  g.planned = c.need_pairs;
  c.L = layout(nframes, h);
  return 0;
}

// The call's row arrays, units and results inside scratch memory at base
// (c.L.total bytes, 256-byte aligned).  Every element a kernel reads is
// written earlier in the same call, so the memory need not be cleared.
void bind(Call& c, char* base) {
  c.ra.r1 = (uint32_t*)(base + c.L.r1);
  c.ra.r2 = (uint64_t*)(base + c.L.r2);
  c.ra.rn = (uint64_t*)(base + c.L.rn);
  c.ra.codd = (uint32_t*)(base + c.L.codd);
  c.ra.plan = (int8_t*)(base + c.L.plan);
  c.ra.pairs = (uint64_t*)(base + c.L.pairs);
  c.ra.psum = (uint64_t*)(base + c.L.psum);
  c.d_results = (double*)(base + c.L.results);
  c.d_units = (uint64_t*)(base + c.L.units);
  c.ra.paths = (uint8_t*)(base + c.L.paths);
}

// setup, then the library's arena (grown on demand) as scratch.
int prepare(Call& c, const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
            ptrdiff_t pitch, int nframes, int bpc) {
  int rc = setup(c, ref, dis, w, h, stride, pitch, nframes, bpc);
  if (rc) return rc;
  if ((rc = ensure(c.dev, c.L.total, c.L.readback()))) return rc;
  bind(c, (char*)g_arena[c.dev].base);
  return 0;
}

// A caller's stream must belong to the planes' device (NULL: that device's
// default stream).
int check_stream(const Call& c, hipStream_t st) {
  if (!st) return 0;
  hipDevice_t sd = -1;
  BEF_HIP(hipStreamGetDevice(st, &sd));
  if (sd != c.dev) return fail(-EINVAL, "stream of device %d, planes on device %d", (int)sd, c.dev);
  return 0;
}

// The row pass, then (batches that can pass 2^55 units) the plan and the
// row pairs; may_time false: no event is created or recorded.
int enqueue_rows(const Call& c, hipStream_t st, bool may_time) {
  const unsigned dbg = g_dbg;
  if (!may_time) {
    BEF_HIP(launch_rows(c.g, c.ra, st, nullptr, nullptr));
    if (c.need_pairs) {
      BEF_HIP(launch_plan(c.g, c.ra, dbg, st, nullptr, nullptr));
      BEF_HIP(launch_pairs(c.g, c.ra, dbg, st, nullptr, nullptr));
    }
    return 0;
  }
  BEF_HIP(timed(0, [&](hipEvent_t a, hipEvent_t b) { return launch_rows(c.g, c.ra, st, a, b); }));
  if (c.need_pairs) {
    BEF_HIP(timed(1, [&](hipEvent_t a, hipEvent_t b) {
      return launch_plan(c.g, c.ra, dbg, st, a, b);
    }));
    BEF_HIP(timed(2, [&](hipEvent_t a, hipEvent_t b) {
      return launch_pairs(c.g, c.ra, dbg, st, a, b);
    }));
  }
  return 0;
}

// The walks, which write the frames' results to d_results.
int enqueue_walk(const Call& c, hipStream_t st, double* d_results, bool may_time) {
  const unsigned dbg = g_dbg;
  if (!may_time) {
    BEF_HIP(launch_walk(c.g, c.ra, d_results, c.d_units, dbg, st, nullptr, nullptr));
    return 0;
  }
  BEF_HIP(timed(3, [&](hipEvent_t a, hipEvent_t b) {
    return launch_walk(c.g, c.ra, d_results, c.d_units, dbg, st, a, b);
  }));
  return 0;
}

int enqueue(const Call& c, hipStream_t st, double* d_results, bool may_time = true) {
  int rc = enqueue_rows(c, st, may_time);
  return rc ? rc : enqueue_walk(c, st, d_results, may_time);
}

// Synchronous batch: results and units copied back to the host.
int run_sync(const void* ref, const void* dis, int w, int h, ptrdiff_t stride, ptrdiff_t pitch,
             int nframes, int bpc, void* stream, double* moments, double* psnr, uint64_t* units) {
  Call c;
  int rc = prepare(c, ref, dis, w, h, stride, pitch, nframes, bpc);
  if (rc) return rc;
  if (!units && !psnr) {  // the moments alone: no noise walk
    c.g.njobs = 2;
  } else if (!units && !moments) {  // the noise alone: no moment walk, plan or pairs
    c.g.job0 = 2;
    c.g.njobs = 1;
    c.need_pairs = false;
    c.g.planned = 0;
  }
  hipStream_t st = (hipStream_t)stream;
  if ((rc = check_stream(c, st)) || (rc = enqueue(c, st, c.d_results))) return rc;
  // results, units and walk paths lie together in the scratch: one copy
  char* hb = (char*)g_arena[c.dev].host;
  const double* hres = (const double*)hb;
  const uint64_t* hun = (const uint64_t*)(hb + (c.L.units - c.L.results));
  const uint8_t* hpath = (const uint8_t*)(hb + (c.L.paths - c.L.results));
  BEF_HIP(hipMemcpyAsync(hb, c.d_results, c.L.readback(), hipMemcpyDeviceToHost, st));
  BEF_HIP(hipStreamSynchronize(st));
  if (g_timing) ev_collect();
  g_paths.assign(hpath, hpath + 3 * (size_t)nframes);
  for (int f = 0; f < nframes; ++f) {
    if (moments)
      for (int k = 0; k < 4; ++k) moments[4 * f + k] = hres[6 * f + k];
    if (psnr)
      for (int k = 0; k < 2; ++k) psnr[2 * f + k] = hres[6 * f + 4 + k];
    if (units)
      for (int k = 0; k < 8; ++k) units[8 * f + k] = hun[8 * f + k];
  }
  return 0;
}

struct DevGuard {
  int prev = -1;
  DevGuard() {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
  }
  ~DevGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

// Frames from host memory, streamed in chunks through two device slots:
// the upload of chunk n (copy stream) overlaps the reductions of chunk
// n - 1 (compute stream); a slot is reloaded only after the chunk before
// last has been reduced from it.
constexpr size_t kPipeChunkBytes = 64ull << 20;  // per plane and chunk

int pipe_setup(int dev, size_t slot_bytes, size_t res_bytes) {
  Arena& a = g_arena[dev];
  if (!a.copy_st) {
    BEF_HIP(hipStreamCreateWithFlags(&a.copy_st, hipStreamNonBlocking));
    BEF_HIP(hipStreamCreateWithFlags(&a.comp_st, hipStreamNonBlocking));
    for (int k = 0; k < 2; ++k) {
      BEF_HIP(hipEventCreateWithFlags(&a.copied[k], hipEventDisableTiming));
      BEF_HIP(hipEventCreateWithFlags(&a.done[k], hipEventDisableTiming));
    }
  }
  const size_t need = 4 * slot_bytes + up256(res_bytes);  // 2 slots x 2 planes, results
  if (a.pipe_cap < need) {
    if (a.pipe) BEF_HIP(hipFree(a.pipe));
    a.pipe = nullptr;
    a.pipe_cap = 0;
    if (hipMalloc(&a.pipe, need) != hipSuccess) {
      (void)hipGetLastError();
      a.pipe = nullptr;
      return fail(-ENOMEM, "hipMalloc of %zu bytes of frame slots failed", need);
    }
    a.pipe_cap = need;
  }
  return 0;
}

int run_host(const void* ref, const void* dis, int w, int h, ptrdiff_t stride, ptrdiff_t pitch,
             int nframes, int bpc, int dev, double* moments, double* psnr) {
  if (!ref || !dis) return fail(-EINVAL, "NULL plane pointer");
  int ndev = 0;
  BEF_HIP(hipGetDeviceCount(&ndev));
  if (dev < 0 || dev >= ndev || dev >= kMaxDev) return fail(-EINVAL, "device %d out of range", dev);
  // geometry checks on the host side (device pointers are checked per chunk)
  int rc = validate(ref, dis, w, h, stride, pitch, nframes, bpc);
  if (rc) return rc;
  BEF_HIP(hipSetDevice(dev));
  const size_t B = bpc == 8 ? 1 : 2;
  const size_t fbytes = (size_t)h * (size_t)stride * B;  // one plane of one frame in a slot
  // what a frame's samples span in the caller's memory: up to sample w - 1
  // of row h - 1 (the padding after it is not read)
  const size_t span = ((size_t)(h - 1) * (size_t)stride + (size_t)w) * B;
  const int K = (int)std::max<size_t>(1, std::min<size_t>((size_t)nframes, kPipeChunkBytes / fbytes));
  const size_t slot = up256((size_t)K * fbytes);
  if ((rc = pipe_setup(dev, slot, (size_t)nframes * 6 * 8))) return rc;
  Arena& a = g_arena[dev];
  double* d_res = (double*)((char*)a.pipe + 4 * slot);  // every frame's results
  const bool contiguous = (size_t)pitch * B == fbytes || nframes == 1;
  const int nchunks = (nframes + K - 1) / K;
  for (int ci = 0; ci < nchunks; ++ci) {
    const int k0 = ci * K, kn = std::min(K, nframes - k0), sl = ci & 1;
    char* dref = (char*)a.pipe + (size_t)sl * 2 * slot;
    char* ddis = dref + slot;
    if (ci >= 2) BEF_HIP(hipStreamWaitEvent(a.copy_st, a.done[sl], 0));
    for (int pl = 0; pl < 2; ++pl) {
      const char* src = (const char*)(pl == 0 ? ref : dis) + (size_t)k0 * (size_t)pitch * B;
      char* dst = pl == 0 ? dref : ddis;
      if (contiguous) {
        BEF_HIP(hipMemcpyAsync(dst, src, (size_t)(kn - 1) * fbytes + span, hipMemcpyHostToDevice,
                               a.copy_st));
      } else {
        for (int f = 0; f < kn; ++f)
          BEF_HIP(hipMemcpyAsync(dst + (size_t)f * fbytes, src + (size_t)f * (size_t)pitch * B,
                                 span, hipMemcpyHostToDevice, a.copy_st));
      }
    }
    BEF_HIP(hipEventRecord(a.copied[sl], a.copy_st));
    BEF_HIP(hipStreamWaitEvent(a.comp_st, a.copied[sl], 0));
    Call c;
    if ((rc = prepare(c, dref, ddis, w, h, stride, (ptrdiff_t)(h * stride), kn, bpc))) break;
    if ((rc = enqueue(c, a.comp_st, d_res + 6 * (size_t)k0))) break;
    BEF_HIP(hipEventRecord(a.done[sl], a.comp_st));
  }
  if (rc == 0) {
    double* hres = (double*)g_arena[dev].host;
    const size_t rb = (size_t)nframes * 6 * 8;
    if ((rc = ensure(dev, 0, rb + 256)) == 0) {
      hres = (double*)g_arena[dev].host;
      BEF_HIP(hipMemcpyAsync(hres, d_res, rb, hipMemcpyDeviceToHost, a.comp_st));
      BEF_HIP(hipStreamSynchronize(a.comp_st));
      for (int f = 0; f < nframes; ++f) {
        if (moments)
          for (int k = 0; k < 4; ++k) moments[4 * f + k] = hres[6 * f + k];
        if (psnr)
          for (int k = 0; k < 2; ++k) psnr[2 * f + k] = hres[6 * f + 4 + k];
      }
    }
  }
  (void)hipStreamSynchronize(a.comp_st);
  (void)hipStreamSynchronize(a.copy_st);
  if (g_timing) ev_collect();
  return rc;
}

// Pipelined batches.  Batch n's rows (and plan and pairs) run on row
// stream n % kPipeRowQ, its walks on the walk stream once its rows are
// done; a small batch runs whole on the walk stream.  The row streams take
// turns, so one batch's row pass overlaps the tail of the one before (and
// the few microseconds a stream stalls after a dispatch that signals an
// event), and the walks overlap later row passes.  Slot n % kPipeSlots is rewritten by batch n + kPipeSlots only
// after batch n's walks have read it.  The walks get CUs of their own: a
// walk block needs a whole CU's LDS, which a busy row pass never frees.
void ovl_drain(Arena& a) {
  for (hipStream_t q : a.prow)
    if (q) (void)hipStreamSynchronize(q);
  if (a.pwalk) (void)hipStreamSynchronize(a.pwalk);
}

// Streams and events go only once the whole device is idle: a caller's
// stream may still hold a wait on a join event.
void ovl_destroy(Arena& a) {
  ovl_drain(a);
  (void)hipDeviceSynchronize();
  for (hipStream_t& q : a.prow) {
    if (q) (void)hipStreamDestroy(q);
    q = nullptr;
  }
  if (a.pwalk) (void)hipStreamDestroy(a.pwalk);
  a.pwalk = nullptr;
  std::vector<hipEvent_t*> evs = {&a.penter, &a.pjoin};
  for (int k = 0; k < kPipeSlots; ++k) {
    evs.push_back(&a.prowdone[k]);
    evs.push_back(&a.pwalkdone[k]);
  }
  for (hipEvent_t* e : evs) {
    if (*e) (void)hipEventDestroy(*e);
    *e = nullptr;
  }
  if (a.pslot) (void)hipFree(a.pslot);
  a.pslot = nullptr;
  a.pslot_cap = 0;
  a.pwalk_cus = 0;
  a.pn = 0;
}

// The streams and events of pipelined batches.  The walk stream is created
// last: the arena counts as set up only once it exists.
int ovl_create(Arena& a, int dev, int walk_cus) {
  int ncu = 0;
  BEF_HIP(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  if (walk_cus < 1 || walk_cus >= ncu)
    return fail(-EINVAL, "%d walk CUs outside 1..%d", walk_cus, ncu - 1);
  // the walk stream takes the last walk_cus CUs, the row streams the rest
  std::vector<uint32_t> mrow((ncu + 31) / 32, 0u), mwalk((ncu + 31) / 32, 0u);
  for (int i = 0; i < ncu; ++i) (i >= ncu - walk_cus ? mwalk : mrow)[i / 32] |= 1u << (i % 32);
  // the handoffs stay on this device: no system-scope fence
  const unsigned local = hipEventDisableTiming | hipEventDisableSystemFence;
  BEF_HIP(hipEventCreateWithFlags(&a.penter, hipEventDisableTiming));
  BEF_HIP(hipEventCreateWithFlags(&a.pjoin, hipEventDisableTiming));
  for (int k = 0; k < kPipeSlots; ++k) {
    BEF_HIP(hipEventCreateWithFlags(&a.prowdone[k], local));
    BEF_HIP(hipEventCreateWithFlags(&a.pwalkdone[k], local));
  }
  for (hipStream_t& q : a.prow)
    BEF_HIP(hipExtStreamCreateWithCUMask(&q, (uint32_t)mrow.size(), mrow.data()));
  BEF_HIP(hipExtStreamCreateWithCUMask(&a.pwalk, (uint32_t)mwalk.size(), mwalk.data()));
  a.pwalk_cus = walk_cus;
  return 0;
}

int ovl_setup(int dev, size_t slot_bytes, int walk_cus) {
  Arena& a = g_arena[dev];
  if (a.pwalk && a.pwalk_cus != walk_cus) ovl_destroy(a);
  if (!a.pwalk) {
    const int rc = ovl_create(a, dev, walk_cus);
    if (rc) {  // release whatever was made; the error text stays
      ovl_destroy(a);
      return rc;
    }
  }
  if (a.pslot_cap < slot_bytes) {  // after the batches that use the slots
    ovl_drain(a);
    if (a.pslot) BEF_HIP(hipFree(a.pslot));
    a.pslot = nullptr;
    a.pslot_cap = 0;
    if (hipMalloc(&a.pslot, kPipeSlots * slot_bytes) != hipSuccess) {
      (void)hipGetLastError();
      a.pslot = nullptr;
      return fail(-ENOMEM, "hipMalloc of %zu bytes of pipeline slots failed",
                  kPipeSlots * slot_bytes);
    }
    a.pslot_cap = slot_bytes;
  }
  return 0;
}

int ovl_submit(const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
               ptrdiff_t pitch, int nframes, int bpc, hipStream_t st, double* dev_results) {
  Call c;
  int rc = setup(c, ref, dis, w, h, stride, pitch, nframes, bpc);
  if (rc || (rc = check_stream(c, st))) return rc;
  if ((rc = ovl_setup(c.dev, c.L.total, g_pipe_walk_cus))) return rc;
  Arena& a = g_arena[c.dev];
  const int s = (int)(a.pn % kPipeSlots);
  const bool small = 2.0 * w * h * nframes * (bpc == 8 ? 1 : 2) <= kPipeSmallBytes;
  const hipStream_t rq = small ? a.pwalk : a.prow[a.pn % kPipeRowQ];
  bind(c, (char*)a.pslot + (size_t)s * a.pslot_cap);
  // the batch's reads follow the caller's earlier work on its stream
  if (hipStreamQuery(st) != hipSuccess) {
    (void)hipGetLastError();
    BEF_HIP(hipEventRecord(a.penter, st));
    BEF_HIP(hipStreamWaitEvent(rq, a.penter, 0));
  }
  // the slot's previous batch must have been walked; a wait costs the host
  // several microseconds, so it is skipped when that walk has already ended
  // (or, for a small batch, comes earlier on the same stream)
  if (!small && a.pn >= kPipeSlots && hipEventQuery(a.pwalkdone[s]) != hipSuccess) {
    (void)hipGetLastError();
    BEF_HIP(hipStreamWaitEvent(rq, a.pwalkdone[s], 0));
  }
  // the handoff events are the last dispatches' own completion (no
  // separate marker packet on either queue)
  const unsigned dbg = g_dbg;
  hipEvent_t rows_done = small ? nullptr : a.prowdone[s];
  if (c.need_pairs) {
    BEF_HIP(launch_rows(c.g, c.ra, rq, nullptr, nullptr));
    BEF_HIP(launch_plan(c.g, c.ra, dbg, rq, nullptr, nullptr));
    BEF_HIP(launch_pairs(c.g, c.ra, dbg, rq, nullptr, rows_done));
  } else {
    BEF_HIP(launch_rows(c.g, c.ra, rq, nullptr, rows_done));
  }
  if (!small) BEF_HIP(hipStreamWaitEvent(a.pwalk, a.prowdone[s], 0));
  BEF_HIP(launch_walk(c.g, c.ra, dev_results, c.d_units, dbg, a.pwalk, nullptr, a.pwalkdone[s]));
  a.pn += 1;
  return 0;
}

}  // namespace

extern "C" {

int bef_pipe_submit(const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
                    ptrdiff_t frame_pitch, int nframes, int bpc, void* stream,
                    double* dev_results) {
  std::lock_guard<std::mutex> lk(g_mu);
  clear_err();
  if (!dev_results) return fail(-EINVAL, "NULL dev_results");
  DevGuard dg;
  return ovl_submit(ref, dis, w, h, stride, frame_pitch, nframes, bpc, (hipStream_t)stream,
                     dev_results);
}

int bef_pipe_join(int device, void* stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  clear_err();
  if (device < 0 || device >= kMaxDev) return fail(-EINVAL, "device %d out of range", device);
  Arena& a = g_arena[device];
  if (!a.pwalk) return 0;  // nothing submitted on this device
  DevGuard dg;
  BEF_HIP(hipSetDevice(device));
  const hipStream_t st = (hipStream_t)stream;
  if (st) {
    hipDevice_t sd = -1;
    BEF_HIP(hipStreamGetDevice(st, &sd));
    if (sd != device) return fail(-EINVAL, "stream of device %d, joining device %d", (int)sd, device);
  }
  BEF_HIP(hipEventRecord(a.pjoin, a.pwalk));
  BEF_HIP(hipStreamWaitEvent(st, a.pjoin, 0));
  return 0;
}

int bef_pipe_set_walk_cus(int n) {
  std::lock_guard<std::mutex> lk(g_mu);
  clear_err();
  if (n < 0 || n > 128) return fail(-EINVAL, "%d walk CUs outside 1..128", n);
  const int old = g_pipe_walk_cus;
  if (n) g_pipe_walk_cus = n;
  return old;
}

int bef_frames(const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
               ptrdiff_t frame_pitch, int nframes, int bpc, void* stream, double* moments,
               double* psnr) {
  std::lock_guard<std::mutex> lk(g_mu);
  clear_err();
  DevGuard dg;
  return run_sync(ref, dis, w, h, stride, frame_pitch, nframes, bpc, stream, moments, psnr,
                  nullptr);
}

int bef_frames_units(const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
                     ptrdiff_t frame_pitch, int nframes, int bpc, void* stream, uint64_t* units) {
  std::lock_guard<std::mutex> lk(g_mu);
  clear_err();
  if (!units) return fail(-EINVAL, "NULL units");
  DevGuard dg;
  return run_sync(ref, dis, w, h, stride, frame_pitch, nframes, bpc, stream, nullptr, nullptr,
                  units);
}

int bef_frames_async(const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
                     ptrdiff_t frame_pitch, int nframes, int bpc, void* stream,
                     double* dev_results) {
  std::lock_guard<std::mutex> lk(g_mu);
  clear_err();
  if (!dev_results) return fail(-EINVAL, "NULL dev_results");
  DevGuard dg;
  Call c;
  int rc = prepare(c, ref, dis, w, h, stride, frame_pitch, nframes, bpc);
  if (rc || (rc = check_stream(c, (hipStream_t)stream))) return rc;
  return enqueue(c, (hipStream_t)stream, dev_results);
}

int bef_frames_noalloc(const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
                       ptrdiff_t frame_pitch, int nframes, int bpc, void* stream,
                       double* dev_results) {
  std::lock_guard<std::mutex> lk(g_mu);
  clear_err();
  if (!dev_results) return fail(-EINVAL, "NULL dev_results");
  DevGuard dg;
  Call c;
  int rc = setup(c, ref, dis, w, h, stride, frame_pitch, nframes, bpc);
  if (rc || (rc = check_stream(c, (hipStream_t)stream))) return rc;
  if (c.L.total > kStaticScratchBytes)
    return fail(-EINVAL, "%d frames of %d rows need %zu bytes of scratch; the static scratch "
                "holds %zu", nframes, h, c.L.total, kStaticScratchBytes);
  void*& ptr = g_static_ptr[c.dev];
  if (!ptr) {  // first call on this device (it is current: setup selected it)
    void* p = nullptr;
    BEF_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(-EIO, "hipGetSymbolAddress gave no address for the static scratch");
    ptr = p;
  }
  bind(c, (char*)ptr);
  return enqueue(c, (hipStream_t)stream, dev_results, false);
}

int bef_planes(const void* const* refs, const void* const* diss, const int* ws, const int* hs,
               const ptrdiff_t* strides, const ptrdiff_t* frame_pitches, int nplanes,
               int nframes, int bpc, void* stream, double* out) {
  std::lock_guard<std::mutex> lk(g_mu);
  clear_err();
  if (!refs || !diss || !ws || !hs || !strides || !frame_pitches || !out)
    return fail(-EINVAL, "NULL argument array or output");
  if (nplanes < 1 || nplanes > kMaxPlanes)
    return fail(-EINVAL, "nplanes %d outside 1..%d", nplanes, kMaxPlanes);
  DevGuard dg;
  Call c[kMaxPlanes];
  size_t rows_bytes = 0;
  for (int p = 0; p < nplanes; ++p) {
    int rc = setup(c[p], refs[p], diss[p], ws[p], hs[p], strides[p], frame_pitches[p], nframes,
                   bpc);
    if (rc) return rc;
    if (c[p].dev != c[0].dev) return fail(-EINVAL, "plane %d on another device", p);
    rows_bytes = std::max(rows_bytes, c[p].L.total);
  }
  const hipStream_t st = (hipStream_t)stream;
  int rc = check_stream(c[0], st);
  if (rc) return rc;
  // the planes run one after another on the stream and share the row arrays;
  // each plane's results, then every dB value, lie after them
  const size_t nres = (size_t)nplanes * nframes;
  const size_t res_off = up256(rows_bytes), db_off = res_off + up256(nres * 6 * 8);
  const size_t total = db_off + up256(nres * 8);
  if ((rc = ensure(c[0].dev, total, total - res_off))) return rc;
  char* base = (char*)g_arena[c[0].dev].base;
  double* d_res = (double*)(base + res_off);
  double* d_db = (double*)(base + db_off);
  for (int p = 0; p < nplanes; ++p) {
    bind(c[p], base);
    if ((rc = enqueue(c[p], st, d_res + (size_t)p * nframes * 6))) return rc;
  }
  BEF_HIP(launch_psnr_db(d_res, (int)nres, bpc, d_db, st));
  char* hb = (char*)g_arena[c[0].dev].host;
  BEF_HIP(hipMemcpyAsync(hb, d_res, total - res_off, hipMemcpyDeviceToHost, st));
  BEF_HIP(hipStreamSynchronize(st));
  if (g_timing) ev_collect();
  const double* hres = (const double*)hb;
  const double* hdb = (const double*)(hb + (db_off - res_off));
  for (size_t k = 0; k < nres; ++k) {
    for (int j = 0; j < 6; ++j) out[7 * k + j] = hres[6 * k + j];
    out[7 * k + 6] = hdb[k];
  }
  return 0;
}

int bef_read_ceiling(const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
                     ptrdiff_t frame_pitch, int nframes, void* stream, uint32_t* dev_out) {
  std::lock_guard<std::mutex> lk(g_mu);
  clear_err();
  if (!dev_out) return fail(-EINVAL, "NULL dev_out");
  DevGuard dg;
  Call c;
  int rc = prepare(c, ref, dis, w, h, stride, frame_pitch, nframes, 16);
  if (rc) return rc;
  if (c.g.cb == 0) return fail(-EINVAL, "rows hold no whole 4-byte chunks at this alignment");
  const hipStream_t st = (hipStream_t)stream;
  if ((rc = check_stream(c, st))) return rc;
  BEF_HIP(timed(4, [&](hipEvent_t a, hipEvent_t b) {
    return launch_read_ceiling(c.g, dev_out, st, a, b);
  }));
  return 0;
}

int bef_frames_host(const void* ref, const void* dis, int w, int h, ptrdiff_t stride,
                    ptrdiff_t frame_pitch, int nframes, int bpc, int device, double* moments,
                    double* psnr) {
  std::lock_guard<std::mutex> lk(g_mu);
  clear_err();
  DevGuard dg;
  return run_host(ref, dis, w, h, stride, frame_pitch, nframes, bpc, device, moments, psnr);
}

int moment_frame(const void* ref, const void* dis, int w, int h, ptrdiff_t stride, int bpc,
                 double out[4]) {
  if (!out) return fail(-EINVAL, "NULL out");
  return bef_frames(ref, dis, w, h, stride, 0, 1, bpc, nullptr, out, nullptr);
}

int psnr_noise(const void* ref, const void* dis, int w, int h, ptrdiff_t stride, int bpc,
               double out[2]) {
  if (!out) return fail(-EINVAL, "NULL out");
  return bef_frames(ref, dis, w, h, stride, 0, 1, bpc, nullptr, nullptr, out);
}

const char* bef_last_error(void) { return g_err; }

int bef_walk_paths(uint8_t* out, int n) {
  std::lock_guard<std::mutex> lk(g_mu);
  const int count = (int)g_paths.size();
  if (out)
    for (int k = 0; k < n && k < count; ++k) out[k] = g_paths[k];
  return count;
}

unsigned bef_debug_set(unsigned flags) {
  std::lock_guard<std::mutex> lk(g_mu);
  const unsigned old = g_dbg;
  g_dbg = flags;
  return old;
}

int bef_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_timing = on != 0;
  return 0;
}

int bef_timing_read(int kernel, double* ms, long* launches) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (kernel < 0 || kernel > 4 || !ms || !launches) return -EINVAL;
  ev_collect();
  *ms = g_ms[kernel];
  *launches = g_n[kernel];
  return 0;
}

void bef_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  ev_collect();
  for (int k = 0; k < 5; ++k) {
    g_ms[k] = 0;
    g_n[k] = 0;
  }
}

void bef_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  ev_collect();
  for (hipEvent_t e : g_ev_pool) (void)hipEventDestroy(e);
  g_ev_pool.clear();
  DevGuard dg;
  for (int d = 0; d < kMaxDev; ++d) {
    Arena& a = g_arena[d];
    if (!a.base && !a.host && !a.pipe && !a.copy_st && !a.pwalk) continue;
    (void)hipSetDevice(d);
    ovl_destroy(a);
    if (a.base) (void)hipFree(a.base);
    if (a.host) (void)hipHostFree(a.host);
    if (a.pipe) (void)hipFree(a.pipe);
    for (int k = 0; k < 2; ++k) {
      if (a.copied[k]) (void)hipEventDestroy(a.copied[k]);
      if (a.done[k]) (void)hipEventDestroy(a.done[k]);
    }
    if (a.copy_st) (void)hipStreamDestroy(a.copy_st);
    if (a.comp_st) (void)hipStreamDestroy(a.comp_st);
    a = Arena();
  }
}

}  // extern "C"
