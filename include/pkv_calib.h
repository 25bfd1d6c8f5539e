/*
 * pkv_calib.h -- measurement utilities of the benchmark, built as a library
 * of their own (libpkv_calib.so).  Nothing here is part of the paged KV-cache
 * path: these kernels calibrate the figures the path is judged by.
 *
 *   pkv_calib_clock       the shader clock, read by one wave that spins for
 *                         a given time (run beside the measured kernels, on
 *                         another stream, it reports the clock under their
 *                         load).
 *   pkv_calib_read_runs   a plain read kernel over a list of 4 KB runs,
 *                         one list per wave: the attainable read rate of an
 *                         address stream, such as the K/V runs a decode batch
 *                         reads, with no arithmetic.
 *
 * Conventions: device pointers unless stated; calls only enqueue work on
 * `stream` (a hipStream_t; NULL is the default stream) and return 0 on
 * success, 1 for invalid arguments (nothing enqueued), 2 for a launch error.
 */
#ifndef PKV_CALIB_H
#define PKV_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * One wave reads the shader-clock counter (s_memtime) and the constant
 * 100 MHz counter (s_memrealtime) until `ticks_100mhz` ticks of the latter
 * have passed, then writes out[0] = shader-clock ticks and out[1] =
 * constant-clock ticks elapsed.  The clock in MHz is 100 * out[0] / out[1].
 *   out            2 uint64 (device memory)
 *   ticks_100mhz   host, 1 .. 1e9 (at most 10 s)
 */
int pkv_calib_clock(uint64_t* out, int64_t ticks_100mhz, void* stream);

/*
 * Wave w of the launch reads the runs of run_kib KiB at device addresses
 * run_addr[wave_begin[w]] .. run_addr[wave_begin[w + 1] - 1] in order,
 * 32 KiB in flight (8 runs of 4 KiB, 16 of 2 KiB, 32 of 1 KiB), with
 * non-temporal 16-byte loads (the cache policy
 * the decode kernels use for their K/V stream), and writes the XOR of every
 * 32-bit word it read, per lane, to sink[64 w + lane].
 *   run_addr       uint64 [wave_begin[num_waves]]: each a device address of
 *                  1024 * run_kib readable bytes, 16-byte aligned
 *                  (precondition)
 *   wave_begin     int64 [num_waves + 1], non-decreasing, wave_begin[0] = 0
 *   num_waves      host, >= 1
 *   run_kib        host, 1, 2 or 4 (a 16-bit K or V run of a 16-token block
 *                  is 4 KiB at head_dim 128, an FP8 one 2 KiB)
 *   sink           uint32 [64 * num_waves]
 */
int pkv_calib_read_runs(const uint64_t* run_addr, const int64_t* wave_begin, int64_t num_waves,
                        int32_t run_kib, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_CALIB_H */
