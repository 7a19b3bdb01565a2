/*
 * bha_probe.h -- C ABI of libbha_probe.so, the HBM streaming probe that sits
 * beside libbha.so (gfx950).
 *
 * It measures what plain streaming reaches on the device, so the bandwidth of
 * the block-hybrid kernels can be set against a ceiling measured with the same
 * kind of loads: each of the four waves of a work-group streams its own
 * contiguous slice of every trip with 16-byte loads that are contiguous across
 * the wave (1 KiB per load instruction), as the forward streams a pair's state
 * record, and optionally writes a share of output per trip with 16-byte
 * stores, as the forward writes a pair's output rows. It computes nothing of
 * the method and is not used by libbha.so.
 *
 * Trip t reads 4 * loads_per_lane KiB starting at byte 4096 * loads_per_lane * t
 * of src and writes 4 * store_kb_per_wave KiB starting at byte
 * 4096 * store_kb_per_wave * t of dst. A persistent grid of wgs_per_cu
 * work-groups per compute unit takes trips b, b + G, b + 2G, ...; each wave
 * keeps `buffers` trips' slices in flight (the next one is issued as soon as
 * the current one has been consumed).
 *
 * Conventions: device pointers; the caller allocates everything; the call is
 * asynchronous on `stream`; invalid arguments return BHA_PROBE_ERR_ARG and
 * enqueue nothing; a failed launch returns BHA_PROBE_ERR_HIP.
 */
#ifndef BHA_PROBE_H
#define BHA_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { BHA_PROBE_OK = 0, BHA_PROBE_ERR_ARG = -1, BHA_PROBE_ERR_HIP = -2 };

typedef struct {
    int32_t loads_per_lane;    /* 16-byte loads per lane per trip: 8, 16 or 32 */
    int32_t buffers;           /* trips in flight per wave: 1 or 2 */
    int32_t nontemporal;       /* 0: plain loads, 1: non-temporal loads */
    int32_t wgs_per_cu;        /* resident work-groups per compute unit, 1..8 */
    int32_t store_kb_per_wave; /* KiB each wave writes per trip, 0..8 (0: read only) */
    int32_t store_mode;        /* when a trip's share is written:
                                  0: plain stores right after the trip's slice is summed
                                  1: non-temporal stores right after the trip
                                  2: plain stores of all the work-group's trips after its
                                     last read (writes gathered at the end of the launch)
                                  3: plain stores of the last four trips' shares together,
                                     every fourth trip
                                  4: the first half of the work-group's trips as in mode 0,
                                     the second half after its last read */
} bha_probe_cfg;

/* Bytes one trip reads from src and writes to dst (negative: invalid cfg). */
int64_t bha_probe_trip_read_bytes(const bha_probe_cfg* cfg);
int64_t bha_probe_trip_write_bytes(const bha_probe_cfg* cfg);

/* Floats `sink` must hold (one per thread of the grid on the current device). */
int64_t bha_probe_sink_floats(const bha_probe_cfg* cfg);

/*
 * bha_probe_stream -- one launch of `trips` trips.
 *   src  : trips * bha_probe_trip_read_bytes(cfg) readable bytes, 16-byte aligned.
 *   dst  : trips * bha_probe_trip_write_bytes(cfg) writable bytes, 16-byte
 *          aligned (may be NULL when store_kb_per_wave == 0).
 *   sink : bha_probe_sink_floats(cfg) floats; written only if a sum of the
 *          loaded values equals a sentinel (keeps the loads from being dropped).
 */
int bha_probe_stream(const bha_probe_cfg* cfg, const void* src, int64_t trips, void* dst, float* sink,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BHA_PROBE_H */
