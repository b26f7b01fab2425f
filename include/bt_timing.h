/* Timing build of the library (libbt_timing.so, built beside libbt.so from
 * the same sources with BT_WAVE_TIMESTAMPS defined).  It exports everything
 * bt.h declares, with the same results, and in addition each wave of a
 * streaming grouped launch (bt_gemm_grouped with packed dot products) and
 * of bt_read_probe records the GPU's 100 MHz real-time counter at fixed
 * points of its work, and its hardware position, for the launch that ran
 * last.  It is a measurement tool: the stamps cost a few instructions per
 * wave, and the product library does not contain them.  Not thread-safe:
 * concurrent launches overwrite each other's records. */
#ifndef BT_TIMING_H
#define BT_TIMING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BT_TIMED_WAVES 4096 /* waves recorded (waves past this are not) */
#define BT_TIMED_SLOTS 8    /* uint64 per wave in bt_wave_timestamps */

/* Copies the records of the last streaming grouped launch to host memory:
 * ts [BT_TIMED_WAVES][8] uint64, slots 0 wave entry, 1 range and first
 * problem known, 2 first weight group and activation sums arrived (plans
 * that quantize their own activations: the first segment's rows quantized), 3 end of
 * the last segment's loop, 4 hand-offs done, 5 after the workgroup barrier,
 * 6 exit, 7 segments streamed (a count, not a time); hw [BT_TIMED_WAVES][2]
 * uint32, the wave's HW_ID and XCC_ID registers.  Global wave w is wave
 * w % (waves per workgroup) of workgroup w / (waves per workgroup).
 * Entries of waves that did not run keep what an earlier launch wrote.
 * Synchronizes with the device.  Returns BT_OK, BT_E_NULL or BT_E_HIP. */
int32_t bt_wave_timestamps(uint64_t* ts, uint32_t* hw);

/* The same for the last bt_read_probe launch: ts [BT_TIMED_WAVES][4]
 * uint64, slots 0 entry, 1 first load group arrived, 2 end of the loop
 * (slot 3 unused); hw as above. */
int32_t bt_probe_timestamps(uint64_t* ts, uint32_t* hw);

#ifdef __cplusplus
}
#endif

#endif /* BT_TIMING_H */
