// HBM streaming probe (libbha_probe.so): plain streaming reads, optionally
// mixed with writes, shaped like the block-hybrid forward's state stream, as
// a measured ceiling for the library's HBM-bound kernels. The interface is in
// include/bha_probe.h. Nothing here is used by libbha.so.
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "../../include/bha_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// A sum no finite data of the probe's buffers reaches in practice: only then
// is the sink written, so the loads stay live and the sink stays untouched.
constexpr float kSentinel = -3.0e-38f;

template <int NSL, bool NT>
__device__ __forceinline__ void load_slice(const f32x4* src, int64_t trip, int64_t trips, int wv, int lane,
                                           f32x4 (&b)[NSL])
{
    const int64_t tc = trip < trips ? trip : trips - 1;  // past the end: a repeat of the last trip, never consumed
    const f32x4* p = src + (tc * kWaves + wv) * (NSL * 64) + lane;
#pragma unroll
    for (int i = 0; i < NSL; ++i) b[i] = NT ? __builtin_nontemporal_load(p + i * 64) : p[i * 64];
}

template <int NSL>
__device__ __forceinline__ f32x4 consume(const f32x4 (&b)[NSL], f32x4 acc)
{
#pragma unroll
    for (int i = 0; i < NSL; ++i) acc += b[i];
    return acc;
}

// trip's share of dst: wkb KiB per wave
template <bool NTS>
__device__ __forceinline__ void write_share(f32x4* dst, int64_t trip, int wkb, int wv, int lane, f32x4 acc)
{
    f32x4* p = dst + (trip * kWaves + wv) * (static_cast<int64_t>(wkb) * 64) + lane;
    for (int i = 0; i < wkb; ++i) {
        if constexpr (NTS) __builtin_nontemporal_store(acc, p + i * 64);
        else p[i * 64] = acc;
    }
}

// Work-group b takes trips b, b + G, ...; each wave keeps NBUF trips' slices
// in flight and issues the next one as soon as a slice has been summed. SM:
// the store mode of include/bha_probe.h.
template <int NSL, int NBUF, bool NT, int SM>
__global__ __launch_bounds__(kThreads) void stream_probe_kernel(const f32x4* src, int64_t trips, f32x4* dst, int wkb,
                                                                float* sink)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t G = gridDim.x;
    int64_t t = blockIdx.x;
    f32x4 buf[NBUF][NSL];
#pragma unroll
    for (int j = 0; j < NBUF; ++j) load_slice<NSL, NT>(src, t + j * G, trips, wv, lane, buf[j]);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    bool more = t < trips;
    int done = 0;  // trips of this work-group summed so far
    const int64_t per_wg = (trips - blockIdx.x + G - 1) / G;
    while (more) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
            if (more) {
                acc = consume<NSL>(buf[j], acc);
                load_slice<NSL, NT>(src, t + NBUF * G, trips, wv, lane, buf[j]);
                ++done;
                if (wkb > 0 && (SM <= 1 || (SM == 4 && 2 * done <= per_wg)))
                    write_share<SM == 1>(dst, t, wkb, wv, lane, acc);
                t += G;
                more = t < trips;
                if (wkb > 0 && SM == 3 && (done % 4 == 0 || !more)) {
                    // the shares of the last (up to) four trips
                    const int n = done % 4 == 0 ? 4 : done % 4;
                    for (int i = 1; i <= n; ++i) write_share<false>(dst, t - i * G, wkb, wv, lane, acc);
                }
            }
        }
    }
    if (wkb > 0 && SM == 2)
        for (int64_t u = blockIdx.x; u < trips; u += G) write_share<false>(dst, u, wkb, wv, lane, acc);
    if (wkb > 0 && SM == 4)
        for (int64_t j = per_wg / 2; j < per_wg; ++j) write_share<false>(dst, blockIdx.x + j * G, wkb, wv, lane, acc);
    const float s = acc[0] + acc[1] + acc[2] + acc[3];
    if (s == kSentinel) sink[static_cast<int64_t>(blockIdx.x) * kThreads + tid] = s;
}

bool valid(const bha_probe_cfg* c)
{
    return c && (c->loads_per_lane == 8 || c->loads_per_lane == 16 || c->loads_per_lane == 32) &&
           (c->buffers == 1 || c->buffers == 2) && (c->nontemporal == 0 || c->nontemporal == 1) &&
           c->wgs_per_cu >= 1 && c->wgs_per_cu <= 8 && c->store_kb_per_wave >= 0 && c->store_kb_per_wave <= 8 &&
           c->store_mode >= 0 && c->store_mode <= 4;
}

int compute_units()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

template <int NSL, int NBUF, bool NT, int SM>
hipError_t launch(dim3 grid, hipStream_t s, const f32x4* src, int64_t trips, f32x4* dst, int wkb, float* sink)
{
    void* argv[] = {&src, &trips, &dst, &wkb, &sink};
    return hipLaunchKernel(reinterpret_cast<const void*>(stream_probe_kernel<NSL, NBUF, NT, SM>), grid,
                           dim3(kThreads), argv, 0, s);
}

template <int NSL, int NBUF, bool NT>
hipError_t launch_sm(const bha_probe_cfg* c, dim3 grid, hipStream_t s, const f32x4* src, int64_t trips, f32x4* dst,
                     float* sink)
{
    const int w = c->store_kb_per_wave;
    switch (c->store_mode) {
        case 0: return launch<NSL, NBUF, NT, 0>(grid, s, src, trips, dst, w, sink);
        case 1: return launch<NSL, NBUF, NT, 1>(grid, s, src, trips, dst, w, sink);
        case 2: return launch<NSL, NBUF, NT, 2>(grid, s, src, trips, dst, w, sink);
        case 3: return launch<NSL, NBUF, NT, 3>(grid, s, src, trips, dst, w, sink);
        default: return launch<NSL, NBUF, NT, 4>(grid, s, src, trips, dst, w, sink);
    }
}

template <int NSL>
hipError_t launch_nsl(const bha_probe_cfg* c, dim3 grid, hipStream_t s, const f32x4* src, int64_t trips, f32x4* dst,
                      float* sink)
{
    if (c->buffers == 1)
        return c->nontemporal ? launch_sm<NSL, 1, true>(c, grid, s, src, trips, dst, sink)
                              : launch_sm<NSL, 1, false>(c, grid, s, src, trips, dst, sink);
    return c->nontemporal ? launch_sm<NSL, 2, true>(c, grid, s, src, trips, dst, sink)
                          : launch_sm<NSL, 2, false>(c, grid, s, src, trips, dst, sink);
}

}  // namespace

extern "C" int64_t bha_probe_trip_read_bytes(const bha_probe_cfg* cfg)
{
    return valid(cfg) ? static_cast<int64_t>(kWaves) * cfg->loads_per_lane * 1024 : BHA_PROBE_ERR_ARG;
}

extern "C" int64_t bha_probe_trip_write_bytes(const bha_probe_cfg* cfg)
{
    return valid(cfg) ? static_cast<int64_t>(kWaves) * cfg->store_kb_per_wave * 1024 : BHA_PROBE_ERR_ARG;
}

extern "C" int64_t bha_probe_sink_floats(const bha_probe_cfg* cfg)
{
    if (!valid(cfg)) return BHA_PROBE_ERR_ARG;
    const int cus = compute_units();
    if (cus <= 0) return BHA_PROBE_ERR_HIP;
    return static_cast<int64_t>(cus) * cfg->wgs_per_cu * kThreads;
}

extern "C" int bha_probe_stream(const bha_probe_cfg* cfg, const void* src, int64_t trips, void* dst, float* sink,
                                hipStream_t stream)
{
    if (!valid(cfg) || !src || !sink || trips < 1) return BHA_PROBE_ERR_ARG;
    if (cfg->store_kb_per_wave > 0 && !dst) return BHA_PROBE_ERR_ARG;
    if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16 ||
        reinterpret_cast<uintptr_t>(sink) % 4)
        return BHA_PROBE_ERR_ARG;
    const int cus = compute_units();
    if (cus <= 0) return BHA_PROBE_ERR_HIP;
    int64_t g = static_cast<int64_t>(cus) * cfg->wgs_per_cu;
    if (g > trips) g = trips;  // every work-group takes at least one trip
    const dim3 grid(static_cast<uint32_t>(g));
    const f32x4* s = static_cast<const f32x4*>(src);
    f32x4* d = static_cast<f32x4*>(dst);
    hipError_t e;
    switch (cfg->loads_per_lane) {
        case 8: e = launch_nsl<8>(cfg, grid, stream, s, trips, d, sink); break;
        case 16: e = launch_nsl<16>(cfg, grid, stream, s, trips, d, sink); break;
        default: e = launch_nsl<32>(cfg, grid, stream, s, trips, d, sink); break;
    }
    return e == hipSuccess ? BHA_PROBE_OK : BHA_PROBE_ERR_HIP;
}
