/*
 * oscar_probe.h -- measurement probes of the decode benchmark
 * (liboscar_probe.so).  They are not part of the OScaR path: they measure
 * the hardware bounds the decode kernel is judged against.
 *
 * Return values: 0 on success, 1 for invalid arguments (nothing launched),
 * 4 if the launch failed.  All pointers are device memory owned by the
 * caller; launches are asynchronous on `stream` (a hipStream_t, NULL = the
 * default stream); nothing is allocated.
 */
#ifndef OSCAR_PROBE_H
#define OSCAR_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The decode kernel's cache stream without its compute: grid (splits,
 * num_kv_heads, batch) of 16-wave workgroups with the decode kernel's LDS
 * footprint; in each, two loader waves copy the 9472-byte group blocks
 * split, split + splits, ... of its (sequence, KV head) into an 8-stage LDS
 * ring with direct global -> LDS nontemporal loads, two groups in flight
 * each.  The time per launch is the streaming ceiling of that access
 * pattern (the decode's attainable bound, launch costs included).
 *
 * blocks : the contiguous packed cache, uint8 [batch][num_kv_heads]
 *          [capacity/128][9472], 16-byte aligned (every group is read).
 * sink   : uint32 [batch][num_kv_heads][splits][2], written (one word per
 *          loader wave, the first word its copies brought in).
 */
int32_t oscar_probe_stream(const uint8_t* blocks, int32_t batch, int32_t num_kv_heads, int32_t capacity,
                           int32_t splits, uint32_t* sink, void* stream);

/*
 * num_blocks one-wave workgroups each run `iters` dependent FMAs and write
 * out[3 i] = shader-clock cycles and out[3 i + 1] = wall-clock ticks over
 * that loop (out[3 i + 2] is a dependency sink).  The shader clock in MHz is
 * cycles / ticks * oscar_probe_wall_clock_khz() / 1000.
 * out : uint64 [num_blocks][3].
 */
int32_t oscar_probe_clock(uint64_t* out, int32_t num_blocks, int32_t iters, void* stream);

/* Rate of the wall clock read by oscar_probe_clock on the current device, in
 * kHz (0 if it cannot be queried). */
int32_t oscar_probe_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_PROBE_H */
