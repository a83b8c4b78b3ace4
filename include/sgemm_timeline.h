/*
 * libsgemm_timeline: the timeline build of libsgemm (SGEMM_TIMELINE=1).
 *
 * The DD2360 workbook "Applied GPU Programming", Module 8 (section 8.1),
 * separates two profiling questions: where a program's time goes (a
 * timeline) and why one kernel is slow (per-kernel counters).  rocprofv3
 * answers both at the level of whole kernels; this build answers the first
 * inside the direct-load kernel, per workgroup and per K slice, so that the
 * split between the prologue, the main loop and the stores of C, and the
 * time each wave spends waiting for its own loads, can be measured.
 *
 * The library exports everything include/sgemm.h declares, computing the same
 * results; the functions below are exported by this build only.  Only the
 * direct-load kernel (the variants whose tiles stage operands by direct
 * global-to-LDS loads) records anything: a plan on another kernel leaves the
 * arrays as they were.  Most readings are shader-clock counts (s_memtime):
 * the counters of different compute units are unrelated, so only differences
 * between readings of one workgroup are meaningful.  Two per workgroup come
 * from the device's constant-rate real-time counter (s_memrealtime, at
 * sgemm_f32_timeline_clock_khz), which is one for the whole device: they place
 * the workgroups of a call against each other and give each one's shader-clock
 * rate.
 *
 * Every function returns a hipError_t value as int (0 = hipSuccess); all act
 * on the current device and are synchronous.  The arrays hold the readings of
 * the last call that wrote them (calls write only the workgroups they run):
 * clear them before the call to be measured, and serialise that call.
 */
#ifndef SGEMM_TIMELINE_H
#define SGEMM_TIMELINE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * sgemm_f32_timeline_layout: the array sizes.
 *   *phase_wgs  workgroups with phase readings (ids 0 .. phase_wgs-1 of a
 *               call's first launch);
 *   *slice_wgs  workgroups with per-slice readings (ids 0 .. slice_wgs-1);
 *   *waves      wave slots per workgroup in the slice array;
 *   *slices     slice slots per wave (slices 0 .. slices-1 are recorded).
 * hipErrorInvalidValue if a pointer is NULL.
 */
int sgemm_f32_timeline_layout(int *phase_wgs, int *slice_wgs, int *waves, int *slices);

/*
 * sgemm_f32_timeline_read: copies the readings to host memory.
 *   phase[6*w + i]  workgroup w, shader clock: i = 0 entry, 1 loop start (the
 *                   first slice has landed in LDS), 2 loop end, 3 every
 *                   thread's stores of C done; real-time counter: 4 entry,
 *                   5 stores done;
 *   slice[((w*waves + v)*slices + s)*2 + i]  workgroup w, wave v, slice s:
 *                   i = 0 before the wave waits for its own loads of slice
 *                   s+1, i = 1 after that wait (the workgroup barrier
 *                   follows).  32-bit counts: differences wrap modulo 2^32.
 * Unwritten entries are 0.  phase_bytes and slice_bytes may be smaller than
 * the arrays (a prefix is copied; 0 copies nothing); larger sizes, or a NULL
 * pointer with a non-zero size, give hipErrorInvalidValue.
 */
int sgemm_f32_timeline_read(unsigned long long *phase, size_t phase_bytes, unsigned int *slice,
                            size_t slice_bytes);

/*
 * sgemm_f32_timeline_clock_khz: the real-time counter's rate in kHz
 * (hipDeviceAttributeWallClockRate of the current device).
 */
int sgemm_f32_timeline_clock_khz(int *khz);

/* sgemm_f32_timeline_clear: sets both arrays to 0. */
int sgemm_f32_timeline_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_TIMELINE_H */
