/*
 * oracle.h -- plain CPU reference for the float_moment and float_psnr frame
 * reductions.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path includes, links or
 * calls this file or liboracle.so; only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (restated from the pages, not copied):
 *   - picture_copy(): each codeword x becomes the float x / s with
 *     s = 2^(bpc-8) (power-of-two normalisation; Research-2081, Finding).
 *   - first moment: the floats added into a double in raster order, divided
 *     by the pixel count (ADR-1497, Context; Research-2081, Selected
 *     restoration).
 *   - second moment: compute_2nd_moment() adds the float32 square of every
 *     float pixel into a double in raster order and divides by the pixel
 *     count (ADR-1497, Context).
 *   - PSNR noise: for each row, the float32 square of every sample
 *     difference is added into a row double (noise_line()); the row doubles
 *     are added into one frame double in row order; the frame double is the
 *     noise and noise / (w*h) the MSE (ADR-1499, Context and Decision).
 *
 * Samples: uint8_t when bpc == 8, native-endian uint16_t when 9 <= bpc <= 16.
 * stride is in samples.  Pointers are HOST pointers.
 * Every int function returns 0, or -22 (EINVAL) for a NULL pointer,
 * w <= 0, h <= 0, stride < w or bpc outside [8, 16].
 */
#ifndef BEF_ORACLE_H
#define BEF_ORACLE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* float32 square of x / 2^(bpc-8), the per-sample term of both loops. */
float oracle_fsq(unsigned x, int bpc);

/* Pre-division accumulators, true scale:
 * acc = {ref_1st_sum, dis_1st_sum, ref_2nd_sum, dis_2nd_sum}. */
int oracle_moment_sums(const void *ref, const void *dis, int w, int h,
                       ptrdiff_t stride, int bpc, double acc[4]);

/* out = {ref_1st, dis_1st, ref_2nd, dis_2nd}. */
int oracle_moment_frame(const void *ref, const void *dis, int w, int h,
                        ptrdiff_t stride, int bpc, double out[4]);

/* Frame noise accumulator (true scale) before the division by w*h. */
int oracle_psnr_sum(const void *ref, const void *dis, int w, int h,
                    ptrdiff_t stride, int bpc, double *noise);

/* out = {noise, mse}. */
int oracle_psnr_noise(const void *ref, const void *dis, int w, int h,
                      ptrdiff_t stride, int bpc, double out[2]);

/* Batch helper: nframes frames, frame_pitch samples apart; moments is
 * [nframes][4] and psnr [nframes][2] (either may be NULL).  Frames are done
 * one after another, each by the single-frame functions above. */
int oracle_frames(const void *ref, const void *dis, int w, int h,
                  ptrdiff_t stride, ptrdiff_t frame_pitch, int nframes,
                  int bpc, double *moments, double *psnr);

/* PSNR in dB from an MSE (true scale) at bit depth bpc: 10 log10(peak^2 /
 * mse), peak = (2^bpc - 1) / 2^(bpc - 8); +infinity for mse 0; NaN for bpc
 * outside [8, 16].  The pages give no formula: this is a reading, parity
 * unpinned against them. */
double oracle_psnr_db(double mse, int bpc);

#ifdef __cplusplus
}
#endif
#endif
