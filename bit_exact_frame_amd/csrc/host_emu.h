/*
 * host_emu.h -- TEST-ONLY entry points of the host emulation library
 * (libbef_emu.so, built from host_emu.cpp with g++; not part of libbef.so).
 *
 * They run the steps of the device algorithm serially on HOST planes, with
 * the same step header (ordsum.h) and the same decomposition as the kernels:
 * row sums, the per-row plan, row pairs from lane runs of staged segments
 * joined by ordered trees, stretches of rows with one plan, a crossing row
 * as at most three groups of runs, else its runs one by one, else its
 * terms.  The pages' own host test checks their twins' steps against the
 * CPU loop the same way, under correct plans and plans broken on purpose
 * (ADR-1497, Decision).  Arguments as in bef.h, on host pointers; every int function
 * returns 0 or -EINVAL.
 */
#ifndef BEF_HOST_EMU_H
#define BEF_HOST_EMU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The general walk of one plane: out = {S1, S2_exact, S2_cpu} in units,
 * under the test flags dbg_flags (BEF_DBG_* of bef.h). */
int bef_host_plane_units(const void *plane, int w, int h, ptrdiff_t stride,
                         int bpc, unsigned dbg_flags, uint64_t out[3]);
/* The fast path's decisions on one plane: out = {1 if the fast path
 * applies (else 0, and the general walk takes the plane), S_cpu, S_exact}. */
int bef_host_fast_units(const void *plane, int w, int h, ptrdiff_t stride,
                        int bpc, uint64_t out[3]);
/* The fast noise: out = {1 if it applies, bits of the noise double in
 * units, exact sum}. */
int bef_host_fast_noise(const void *ref, const void *dis, int w, int h,
                        ptrdiff_t stride, int bpc, uint64_t out[3]);
/* *bits = bit pattern of the noise double in units; *exact = exact sum. */
int bef_host_noise_units(const void *ref, const void *dis, int w, int h,
                         ptrdiff_t stride, int bpc, uint64_t *bits,
                         uint64_t *exact);
/* The one-term step: fl64(s + t) in units. */
uint64_t bef_host_rne53_add(uint64_t s, uint64_t t);
/* The 16-bit row kernel's load shape for planes at these addresses (only
 * their alignment is used; nothing is read): out = {bytes per load (8, 4,
 * or 0 for sample by sample), load slots per lane per group}. */
int bef_host_load_shape(const void *ref, const void *dis, int w,
                        ptrdiff_t stride, ptrdiff_t frame_pitch, int nframes,
                        int out[2]);
/* Pair of a run of terms inside binade e: out = {inc_even, inc_odd}. */
int bef_host_run_pair(const uint32_t *terms, int n, int e, uint64_t out[2]);

#ifdef __cplusplus
}
#endif
#endif
