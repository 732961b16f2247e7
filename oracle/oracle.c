/*
 * oracle.c -- plain, slow CPU reference for float_moment and float_psnr.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  It is the definition of the
 * result, written as the loops the pages describe, with no blocking, fusion,
 * reordering or integer tricks:
 *
 *   picture_copy()          codeword -> float x / 2^(bpc-8)
 *                           [Research-2081, Finding: power-of-two
 *                            normalisation makes samples fractional above
 *                            8 bpc]
 *   compute_2nd_moment()    double += (double)(float square), raster order,
 *                           then / (w*h)
 *                           [ADR-1497, Context]
 *   first moment            double += (double)float, raster order, / (w*h)
 *                           [Research-2081, Selected restoration: first
 *                            moments are the per-pixel values over the
 *                            pixel count; ADR-1497, Consequences: all four
 *                            outputs equal the CPU's]
 *   float_psnr extract()    row double += (double)(float square of the
 *                           sample difference); frame double += row double,
 *                           rows in order; mse = noise / (w*h)
 *                           [ADR-1499, Context and Decision]
 *
 * Build: C99, -O2 -fno-fast-math -ffp-contract=off, x86-64 SSE2 arithmetic
 * (FLT_EVAL_METHOD 0: float expressions are evaluated in float, double in
 * double), no -march flags.  IEEE round-to-nearest-even throughout.
 *
 * ORACLE_MUTANT (test builds only): plants one of a list of plausible
 * mistakes so that the pin tests can show each one is caught.  0 = none.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

#if FLT_EVAL_METHOD != 0
#error "the oracle needs float arithmetic evaluated in float (SSE2)"
#endif

#define EINVAL_ 22

static int bad_args(const void *ref, const void *dis, int w, int h,
                    ptrdiff_t stride, int bpc)
{
    if (!ref || !dis) return 1;
    if (w <= 0 || h <= 0) return 1;
    if (stride < w) return 1;
    if (bpc < 8 || bpc > 16) return 1;
    return 0;
}

/* The scaler of the power-of-two normalisation, as a float. */
static float scaler_of(int bpc)
{
#if ORACLE_MUTANT == 12
    return (float)(1u << (bpc - 7)); /* mutant: scaler off by one bit */
#else
    return (float)(1u << (bpc - 8));
#endif
}

/* Row pointer arithmetic, in samples. */
static ptrdiff_t row_offset(int i, int w, ptrdiff_t stride)
{
#if ORACLE_MUTANT == 4
    (void)stride;
    return (ptrdiff_t)i * w; /* mutant: ignores the stride */
#else
    (void)w;
    return (ptrdiff_t)i * stride;
#endif
}

static unsigned sample_at(const void *plane, int bpc, ptrdiff_t idx)
{
    if (bpc == 8) return ((const uint8_t *)plane)[idx];
    return ((const uint16_t *)plane)[idx];
}

/* picture_copy(): one plane of codewords to a w*h float picture. */
static float *picture_copy(const void *plane, int w, int h, ptrdiff_t stride,
                           int bpc)
{
    float *pic = (float *)malloc(sizeof(float) * (size_t)w * (size_t)h);
    if (!pic) return NULL;
    const float s = scaler_of(bpc);
    for (int i = 0; i < h; i++) {
        const ptrdiff_t off = row_offset(i, w, stride);
        for (int j = 0; j < w; j++)
            pic[(size_t)i * w + j] = (float)sample_at(plane, bpc, off + j) / s;
    }
    return pic;
}

float oracle_fsq(unsigned x, int bpc)
{
    const float v = (float)x / scaler_of(bpc);
    const float sq = v * v;
    return sq;
}

static int last_col(int w)
{
#if ORACLE_MUTANT == 3
    return w - 1; /* mutant: drops the last column */
#else
    return w;
#endif
}

/* Sum of the float pixels into a double, raster order. */
static double first_moment_sum(const float *pic, int w, int h)
{
    double acc = 0.0;
    for (int i = 0; i < h; i++)
        for (int j = 0; j < last_col(w); j++) {
#if ORACLE_MUTANT == 8
            acc += (double)pic[(size_t)i * w + j] /
                   (double)scaler_of(8 + 1); /* mutant: extra halving */
#else
            acc += (double)pic[(size_t)i * w + j];
#endif
        }
    return acc;
}

/* compute_2nd_moment(): float square of each pixel into a double,
 * raster order. */
static double second_moment_sum(const float *pic, int w, int h)
{
#if ORACLE_MUTANT == 2
    float acc = 0.0f; /* mutant: float accumulator */
#else
    double acc = 0.0;
#endif
    for (int i = 0; i < h; i++)
        for (int j = 0; j < last_col(w); j++) {
            const float v = pic[(size_t)i * w + j];
#if ORACLE_MUTANT == 1
            acc += (double)v * (double)v; /* mutant: square in double */
#else
            const float sq = v * v;
            acc += (double)sq;
#endif
        }
    return (double)acc;
}

int oracle_moment_sums(const void *ref, const void *dis, int w, int h,
                       ptrdiff_t stride, int bpc, double acc[4])
{
    if (bad_args(ref, dis, w, h, stride, bpc) || !acc) return -EINVAL_;
    float *pr = picture_copy(ref, w, h, stride, bpc);
    float *pd = picture_copy(dis, w, h, stride, bpc);
    if (!pr || !pd) {
        free(pr);
        free(pd);
        return -12;
    }
    double a[4];
    a[0] = first_moment_sum(pr, w, h);
    a[1] = first_moment_sum(pd, w, h);
    a[2] = second_moment_sum(pr, w, h);
    a[3] = second_moment_sum(pd, w, h);
    free(pr);
    free(pd);
#if ORACLE_MUTANT == 5
    acc[0] = a[1]; acc[1] = a[0]; /* mutant: ref and dis swapped */
    acc[2] = a[3]; acc[3] = a[2];
#else
    acc[0] = a[0]; acc[1] = a[1];
    acc[2] = a[2]; acc[3] = a[3];
#endif
    return 0;
}

int oracle_moment_frame(const void *ref, const void *dis, int w, int h,
                        ptrdiff_t stride, int bpc, double out[4])
{
    double acc[4];
    if (!out) return -EINVAL_;
    int rc = oracle_moment_sums(ref, dis, w, h, stride, bpc, acc);
    if (rc) return rc;
    const double n = (double)w * (double)h;
    for (int k = 0; k < 4; k++) out[k] = acc[k] / n;
    return 0;
}

/* noise_line(): one row of float squares of differences into a double. */
static double noise_line(const float *r, const float *d, int w)
{
    double row = 0.0;
    for (int j = 0; j < last_col(w); j++) {
#if ORACLE_MUTANT == 9
        const double e = (double)r[j] - (double)d[j];
        row += e * e; /* mutant: exact double square, no float rounding */
#else
        const float e = r[j] - d[j];
        const float sq = e * e;
        row += (double)sq;
#endif
    }
    return row;
}

int oracle_psnr_sum(const void *ref, const void *dis, int w, int h,
                    ptrdiff_t stride, int bpc, double *noise)
{
    if (bad_args(ref, dis, w, h, stride, bpc) || !noise) return -EINVAL_;
    float *pr = picture_copy(ref, w, h, stride, bpc);
    float *pd = picture_copy(dis, w, h, stride, bpc);
    if (!pr || !pd) {
        free(pr);
        free(pd);
        return -12;
    }
    double acc = 0.0;
#if ORACLE_MUTANT == 6
    for (int i = h - 1; i >= 0; i--) /* mutant: rows in reverse order */
        acc += noise_line(pr + (size_t)i * w, pd + (size_t)i * w, w);
#elif ORACLE_MUTANT == 7
    for (int i = 0; i < h; i++) /* mutant: terms straight into the frame sum */
        for (int j = 0; j < w; j++) {
            const float e = pr[(size_t)i * w + j] - pd[(size_t)i * w + j];
            const float sq = e * e;
            acc += (double)sq;
        }
#else
    for (int i = 0; i < h; i++)
        acc += noise_line(pr + (size_t)i * w, pd + (size_t)i * w, w);
#endif
    free(pr);
    free(pd);
    *noise = acc;
    return 0;
}

int oracle_psnr_noise(const void *ref, const void *dis, int w, int h,
                      ptrdiff_t stride, int bpc, double out[2])
{
    double noise;
    if (!out) return -EINVAL_;
    int rc = oracle_psnr_sum(ref, dis, w, h, stride, bpc, &noise);
    if (rc) return rc;
    out[0] = noise;
#if ORACLE_MUTANT == 10
    out[1] = noise / (double)w; /* mutant: divides by the width only */
#else
    out[1] = noise / ((double)w * (double)h);
#endif
    return 0;
}

/* Batch helper: the extractors run once per frame (ADR-1497, Context;
 * ADR-1499, Context), so a batch is the frames one after another, frame f
 * starting f * frame_pitch samples after the first, each through the
 * single-frame functions above. */
int oracle_frames(const void *ref, const void *dis, int w, int h,
                  ptrdiff_t stride, ptrdiff_t frame_pitch, int nframes,
                  int bpc, double *moments, double *psnr)
{
    if (nframes <= 0 || frame_pitch < 0) return -EINVAL_;
    const size_t bytes = bpc == 8 ? 1 : 2;
    for (int f = 0; f < nframes; f++) {
#if ORACLE_MUTANT == 13
        /* mutant: the pitch taken as bytes (not scaled by the sample size) */
        const size_t off = (size_t)f * frame_pitch + 0 * bytes;
#elif ORACLE_MUTANT == 14
        /* mutant: frames assumed packed, h * stride samples apart */
        const size_t off = (size_t)f * (size_t)h * (size_t)stride * bytes;
#else
        const size_t off = (size_t)f * frame_pitch * bytes;
#endif
        const char *r = (const char *)ref + off;
        const char *d = (const char *)dis + off;
        int rc = 0;
        if (moments) rc = oracle_moment_frame(r, d, w, h, stride, bpc,
                                              moments + 4 * (size_t)f);
        if (!rc && psnr) rc = oracle_psnr_noise(r, d, w, h, stride, bpc,
                                                psnr + 2 * (size_t)f);
        if (rc) return rc;
    }
    return 0;
}

/* PSNR in dB of a plane from its MSE, as this project reads it (the pages
 * name the psnr_y / psnr_cb / psnr_cr features of integer_psnr and a
 * float_psnr score, but print no formula or constant: Metal kernel batch
 * digest, Feature scope).  Reading: the textbook 10 * log10(peak^2 / MSE)
 * with peak the largest normalised sample, (2^bpc - 1) / 2^(bpc - 8); no
 * clamp, so MSE 0 gives +infinity.  PARITY UNPINNED against the pages. */
double oracle_psnr_db(double mse, int bpc)
{
    if (bpc < 8 || bpc > 16) return NAN;
#if ORACLE_MUTANT == 15
    const double peak = 255.0; /* mutant: the peak of 8-bit samples at every depth */
#else
    const double peak = (double)((1u << bpc) - 1u) / (double)(1u << (bpc - 8));
#endif
    return 10.0 * log10(peak * peak / mse);
}

