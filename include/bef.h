/*
 * bef.h -- C ABI of libbef.so: bit-exact float_moment and float_psnr frame
 * reductions on MI355X (gfx950).
 *
 * What is computed (the CPU loops these calls reproduce bit for bit):
 *   Each codeword x of a luma plane is read as the float x / s with
 *   s = 2^(bpc-8) (Research-2081: Float moment Metal exact reduction
 *   restoration, Finding).
 *   - float_moment: the first moment of a plane is the sum of those floats,
 *     added into a double in raster order, over the pixel count; the second
 *     moment is the sum of their float32 squares, added into a double in
 *     raster order, over the pixel count (ADR-1497, Context).  Past 2^53
 *     units (1/s^2) the CPU's running double rounds as it adds; the result
 *     here is that rounded sum, not the exact one (ADR-1497, Decision).
 *   - float_psnr: each row's float32 squares of (ref - dis) / s are added
 *     into a row double, the rows are added into one double in row order
 *     (the noise), and MSE = noise / (w*h) (ADR-1499, Context and
 *     Decision).
 *   Every returned double equals the plain CPU loop's double (==).
 *
 * Conventions shared by every entry point:
 *   ref, dis   DEVICE pointers (e.g. a torch tensor's data_ptr()), owned by
 *              the caller, read only, not retained after the call.  Samples
 *              are uint8_t when bpc == 8 and native-endian uint16_t when
 *              9 <= bpc <= 16.  Values are used as they are (no clipping to
 *              2^bpc - 1).
 *   w, h       frame width and height in pixels, 1 <= w <= 32768 (a row
 *              then adds fewer than 2^47 units: ADR-1499, Decision, argument
 *              step 1) and 1 <= h <= 32768.
 *   stride     distance between row starts, in SAMPLES, >= w.  Samples
 *              between w and stride are never read.
 *   bpc        bits per sample, 8..16.
 *   device     ref and dis must be on one device; the work runs there.
 *   return     0 on success; -EINVAL (-22) for invalid arguments; -ENOMEM
 *              (-12) when scratch memory cannot be allocated; -EIO (-5) for
 *              a HIP runtime error (text in bef_last_error()).  Outputs are
 *              unspecified after an error.
 *   threads    calls are serialised by a process-wide lock; the library
 *              owns its device scratch (grown on demand, freed by
 *              bef_release()).
 */
#ifndef BEF_H
#define BEF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One frame's four moments, synchronously, on the default stream.
 * out (HOST, 4 doubles) = {ref_1st, dis_1st, ref_2nd, dis_2nd}
 * (ADR-1497, Context; output order of the float_moment feature in the
 * Metal kernel batch digest, Feature scope). */
int moment_frame(const void *ref, const void *dis, int w, int h,
                 ptrdiff_t stride, int bpc, double out[4]);

/* One frame's PSNR noise sum and MSE, synchronously, on the default stream.
 * out (HOST, 2 doubles) = {noise, mse}: noise is the CPU's double row-order
 * sum at true scale, mse = noise / (w*h) (ADR-1499, Decision). */
int psnr_noise(const void *ref, const void *dis, int w, int h,
               ptrdiff_t stride, int bpc, double out[2]);

/* Fused, batched: the float_moment and float_psnr results of nframes
 * frames, each frame as the CPU extractors compute it once per frame
 * (ADR-1497, Context; ADR-1499, Context and Decision).  Frames lie
 * frame_pitch samples apart (frames are only read, so a pitch below
 * h*stride, i.e. overlapping frames, is allowed).  Each plane is read once
 * for both reductions; a call with moments or psnr NULL skips the other's
 * ordered part.
 * stream: a hipStream_t of the planes' device (NULL = that device's default
 * stream; a stream of another device is -EINVAL).  The call enqueues its
 * kernels on that stream and waits once at the end for the results.
 * moments (HOST, [nframes][4]) and psnr (HOST, [nframes][2]) may each be
 * NULL.  1 <= nframes <= 65535. */
int bef_frames(const void *ref, const void *dis, int w, int h,
               ptrdiff_t stride, ptrdiff_t frame_pitch, int nframes, int bpc,
               void *stream, double *moments, double *psnr);

/* As bef_frames, but asynchronous: results go to DEVICE memory
 * dev_results ([nframes][6] doubles: ref_1st, dis_1st, ref_2nd, dis_2nd,
 * noise, mse), caller-owned, written when the stream reaches that point.
 * The call returns after enqueueing; it does not synchronise.  Calls share
 * the library's per-device scratch: two calls whose GPU work overlaps (on
 * different streams) race; enqueue them on one stream.
 * Graph capture: once a call of the same or a larger shape has grown the
 * scratch, the call enqueues kernel launches only (no allocation, memset
 * or synchronisation), so it may be captured into a HIP graph; a replay
 * reads whatever frames the captured buffers hold at that time.  A call
 * that must grow the scratch allocates and fails under capture. */
int bef_frames_async(const void *ref, const void *dis, int w, int h,
                     ptrdiff_t stride, ptrdiff_t frame_pitch, int nframes,
                     int bpc, void *stream, double *dev_results);

/* For callers that cannot allocate (code under HIP graph capture, serving
 * loops, harnesses that forbid hipMalloc): bef_frames_async with the
 * library's static scratch instead of its arena.  Same arguments, limits,
 * results (DEVICE dev_results, [nframes][6] doubles, caller-owned) and
 * asynchrony.  The call allocates nothing (no hipMalloc, hipFree, pinned
 * staging or timing events): its kernels use a fixed device array of
 * 16 MiB per GPU, part of the library, held until the process ends.  A
 * batch whose scratch would exceed it (about 74 bytes per row of each
 * frame plus 144 bytes per frame: e.g. 100 frames of 2160 rows fit) is
 * -EINVAL, with the sizes in bef_last_error().  Every call on a GPU shares
 * that GPU's array: calls whose GPU work overlaps on one GPU (different
 * streams) race; enqueue them on one stream.  The array keeps the last
 * call's contents; no call depends on them. */
int bef_frames_noalloc(const void *ref, const void *dis, int w, int h,
                       ptrdiff_t stride, ptrdiff_t frame_pitch, int nframes,
                       int bpc, void *stream, double *dev_results);

/* Pipelined batches: bef_frames_async's reductions with one batch's
 * ordered part overlapping later batches' plane reads.  The pages'
 * dispatch keeps two frames in flight, collecting frame N - 1 after frame
 * N is uploaded (ADR-1497, Context); here the library keeps several
 * batches in flight on streams of its own per device: batch n's row pass
 * (and plan and pairs) on row stream n % 2, so that consecutive row passes
 * overlap, and its per-plane walks on a walk stream once its rows are
 * done.  The row streams run on all but n_walk of the device's CUs, the
 * walk stream on the other n_walk (bef_pipe_set_walk_cus, default 16).  A
 * batch whose planes hold at most 1 MiB runs whole on the walk stream, in
 * order with the walks: its row pass is too short to overlap anything, and
 * the handoff between streams would cost more than the batch.  Each
 * batch's scratch is one of eight slots, reused in turn.
 * Arguments and limits as bef_frames_async; dev_results (DEVICE,
 * [nframes][6] doubles, caller-owned) receives the same bits.  The batch's
 * reads start after the work enqueued on `stream` before the call.  The
 * call returns after enqueueing (a batch larger than any before first
 * waits, on the host, for the batches in flight, then grows the slots).
 * Results are complete, and the planes may be changed again, only once
 * `stream` has passed a later bef_pipe_join(device, stream), which makes
 * `stream` wait (on the device, not the host) for every batch submitted
 * so far on that device.  The library's streams are blocking streams:
 * work on the legacy NULL stream waits for them, so a caller on the NULL
 * stream gets the same results without the overlap.  Batches of successive
 * calls may share dev_results (their walks run in submission order).  Not
 * for graph capture. */
int bef_pipe_submit(const void *ref, const void *dis, int w, int h,
                    ptrdiff_t stride, ptrdiff_t frame_pitch, int nframes,
                    int bpc, void *stream, double *dev_results);

/* Makes `stream` (NULL = the legacy default stream; else a stream of
 * `device`) wait for every batch bef_pipe_submit has enqueued on `device`
 * so far.  Returns at once; 0 when nothing was submitted there, -EINVAL
 * for a device outside 0..63 or a stream of another device. */
int bef_pipe_join(int device, void *stream);

/* CUs (1..128, fewer than the device has) reserved for the walk stream of
 * pipelined batches; n = 0 changes nothing.  Returns the count in effect
 * before the call, -EINVAL for n outside 0..128.  A new count takes effect
 * at the next bef_pipe_submit on each device, which first waits for that
 * device to go idle and then rebuilds its streams.  The runtime spreads a
 * stream's CUs over the device's XCDs and refuses a count it cannot
 * spread (on MI355X, fewer than 8). */
int bef_pipe_set_walk_cus(int n);

/* Several planes of each frame (luma and chroma, e.g. Y, Cb, Cr of 4:2:0
 * pictures, or any up to 4 planes), each with its own geometry, in one
 * synchronous call: per plane the float_moment and float_psnr results of
 * every frame (each plane as bef_frames computes it), and the plane's PSNR
 * in dB (the Metal kernel batch digest, Feature scope, names per-plane
 * PSNR features psnr_y / psnr_cb / psnr_cr without a formula; the dB value
 * here is the reading 10 log10(peak^2 / MSE), peak = (2^bpc - 1) /
 * 2^(bpc - 8), +infinity when MSE is 0 -- PARITY UNPINNED against the
 * pages).
 * refs[p], diss[p]: DEVICE planes of plane p; ws, hs, strides,
 * frame_pitches: per-plane geometry (samples), each as in bef_frames; all
 * planes on one device, common nframes and bpc; 1 <= nplanes <= 4.
 * out (HOST, [nplanes][nframes][7]) = {ref_1st, dis_1st, ref_2nd, dis_2nd,
 * noise, mse, psnr_db}.  The planes run one after another on stream. */
int bef_planes(const void *const *refs, const void *const *diss,
               const int *ws, const int *hs, const ptrdiff_t *strides,
               const ptrdiff_t *frame_pitches, int nplanes, int nframes,
               int bpc, void *stream, double *out);

/* As bef_frames, for frames in HOST memory (ref, dis: host pointers, same
 * layout and limits), on device `device`, synchronously.  The library
 * streams the frames through two device slots of up to 64 MiB per plane:
 * the upload of one chunk of frames (on a library copy stream) overlaps
 * the reductions of the previous chunk (on a library compute stream).
 * Pinned host memory (hipHostMalloc, torch pin_memory) lets the uploads run
 * at the link's rate; pageable memory is staged by the HIP runtime.  The
 * slots are kept until bef_release().  Each frame is read from its first
 * sample up to sample w - 1 of row h - 1: the padding after the last row is
 * neither read nor required.  moments / psnr: HOST, as in bef_frames
 * (either may be NULL). */
int bef_frames_host(const void *ref, const void *dis, int w, int h,
                    ptrdiff_t stride, ptrdiff_t frame_pitch, int nframes,
                    int bpc, int device, double *moments, double *psnr);

/* Diagnostics: per-frame integer sums in units, synchronously.  In units
 * of 1/s (first moments) and 1/s^2 (squares) every term and every running
 * sum of the CPU's double loop is an integer, each step rounding the exact
 * integer sum to 53 significant bits (ADR-1497, Decision; ADR-1499,
 * Decision, argument step 1).
 * units (HOST, [nframes][8]) = {S1_ref, S1_dis, S2_ref_exact, S2_dis_exact,
 * S2_ref_cpu, S2_dis_cpu, noise_exact, bits of the noise double in units}.
 * The *_cpu values are the CPU's rounded running sums (integers). */
int bef_frames_units(const void *ref, const void *dis, int w, int h,
                     ptrdiff_t stride, ptrdiff_t frame_pitch, int nframes,
                     int bpc, void *stream, uint64_t *units);

/* Diagnostics: the path the walk took for each frame of the last
 * synchronous batch (bef_frames, bef_frames_units, moment_frame,
 * psnr_noise) in the process: out[3f + j] for j = 0 ref moments, 1 dis
 * moments, 2 noise, with 0 = exact sums only (no sum can pass 2^53), 1 =
 * the fast walk (ordered steps by one wave), 2 = the general walk, 3 = the
 * row-by-row double chain (noise), 4 = not run (the call asked for no
 * result of that job).  Copies min(n, count) bytes to out (HOST; may be
 * NULL) and returns count = 3 * nframes of that batch (0 before any). */
int bef_walk_paths(uint8_t *out, int n);

/* Thread-local text of the last failure ("" if none). */
const char *bef_last_error(void);

/* Test hooks (process-wide, default 0).  Every setting must return the
 * same bits; they only change which path forms them: a plan, right or
 * wrong, decides only whether a row is added as one pair or falls back to
 * its runs and then its terms (ADR-1497, Decision), so forcing wrong or
 * missing plans and the fallbacks must leave every result unchanged.
 *   BEF_DBG_PLAN_WRONG  shift every planned binade by one
 *   BEF_DBG_PLAN_NONE   plan no row: every row past 2^53 goes to its runs
 *   BEF_DBG_TERMS_ONLY  rows that leave the plan are added term by term
 *   BEF_DBG_FORCE_ROUND run the ordered-sum kernels on every frame
 *   BEF_DBG_NO_STRETCH  apply planned rows one by one, not as stretches
 *   BEF_DBG_NO_CLOSED_FORM  form every planned row's pair from lane runs,
 *                       also in the binades of 2^53 and 2^54
 *   BEF_DBG_SPLIT_LAUNCH  split the row-pair pass into dispatches of 64
 *                       blocks (the split that very large batches take)
 * Returns the previous flags. */
#define BEF_DBG_PLAN_WRONG 1u
#define BEF_DBG_PLAN_NONE 2u
#define BEF_DBG_TERMS_ONLY 4u
#define BEF_DBG_FORCE_ROUND 8u
#define BEF_DBG_NO_STRETCH 16u
#define BEF_DBG_NO_CLOSED_FORM 32u
#define BEF_DBG_SPLIT_LAUNCH 64u
unsigned bef_debug_set(unsigned flags);

/* Diagnostic, not part of the reductions: the memory side of the 16-bit
 * row pass alone.  Reads both planes (16-bit, same arguments and limits as
 * bef_frames) with the row pass's grid, load width and nontemporal loads,
 * replacing the arithmetic by an XOR of the loaded words, and writes one
 * word per row to dev_out (DEVICE, [nframes][h] uint32_t, caller-owned).
 * Asynchronous on stream.  Its duration (timing kernel 4) is the practical
 * read ceiling of the row pass's access pattern.  -EINVAL also when no
 * whole 4-byte chunk fits the rows' alignment. */
int bef_read_ceiling(const void *ref, const void *dis, int w, int h,
                     ptrdiff_t stride, ptrdiff_t frame_pitch, int nframes,
                     void *stream, uint32_t *dev_out);

/* Kernel timing: when enabled, each kernel the library launches carries a
 * start and a stop HIP event recorded by its own dispatch (on the stream
 * it is launched on), and the library accumulates their durations.
 * kernel: 0 row sums, 1 plan, 2 row pairs, 3 walk, 4 read ceiling.
 * bef_timing_read returns the summed milliseconds and launch count since
 * the last reset (0 / -EINVAL). */
int bef_timing_enable(int on);
int bef_timing_read(int kernel, double *ms, long *launches);
void bef_timing_reset(void);

/* Free the device scratch of every device. */
void bef_release(void);

#ifdef __cplusplus
}
#endif
#endif
