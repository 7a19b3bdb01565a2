// Internal declarations shared by the C-ABI layer and the HIP kernels of
// libbha.so. Not part of the public interface (include/bha.h is).
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "../../include/bha.h"

namespace bha {

// Everything a launch needs, already validated on the host.
struct ForwardArgs {
    int R, H, d, FW, B, io;  // H: query heads
    float scale;  // resolved: never 0
    const void *q, *k, *v;
    bha_strides qs;  // q (and out's layout is os)
    bha_strides ks;  // k and v
    int G;           // query heads per K/V head (1: one K/V head per query head)
    const void* w;
    int64_t wh;
    const float* gamma;  // [H]
    const float* state;  // [num_slots][H / G][record]; W: one per K/V head
    int num_slots;
    const int32_t* slot_ids;
    void* out;
    bha_strides os;
};

struct CommitArgs {
    int R, H, d, FW, B, io;
    const void *k, *v;
    bha_strides ks;
    const void* w;
    int64_t wh;
    float* state;
    int num_slots;
    const int32_t* slot_ids;
    // prefill: request r's tokens are packed rows seq_offsets[r] .. seq_offsets[r+1]-1
    // (of total_tokens); nullptr for a commit of B tokens per request
    const int32_t* seq_offsets;
    int64_t total_tokens;
    // requests with commit_mask[r] == 0 are left untouched; nullptr: all commit
    const uint8_t* commit_mask;
};

// Token range of request r in a commit or prefill, clamped as documented.
__device__ __forceinline__ void commit_rows(const CommitArgs& a, int r, int64_t& first_row, int& n)
{
    if (a.commit_mask != nullptr && a.commit_mask[r] == 0) {
        first_row = -1;
        n = 0;
        return;
    }
    if (a.seq_offsets == nullptr) {
        first_row = -1;  // rows r*req + t*tok
        n = a.B;
        return;
    }
    int64_t s0 = a.seq_offsets[r], s1 = a.seq_offsets[r + 1];
    s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
    s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
    first_row = s0;
    const int64_t len = s1 - s0;
    n = len > 0x7fffffff ? 0x7fffffff : static_cast<int>(len);
}

// Work-group order of a ragged prefill (one work-group per request and head,
// each running over its request's whole token range). Work-groups are handed
// out in blockIdx order, so in request order a long request dispatched late
// runs on with the rest of the device idle. Longest first instead, to within
// about 9 %: the token counts (as commit_rows clamps them) are put in 256
// buckets, eight per power of two, the longest in bucket 0; grid position s
// takes the request at offset o of bucket b in request order, where b and o
// place s in the buckets' concatenation. Cost per work-group: a histogram, a
// 256-entry prefix sum in one wave and a prefix sum over contiguous ranges of
// requests -- O(R / NT), about 2 us of latency before the work-group's own
// loads. The tail it removes is a large share of the launch only when the
// work-groups fill the device a few times over, so it applies up to
// kPrefillOrderPairs (request, head) pairs (about 16 rounds of two
// work-groups per CU) and kPrefillOrderMax requests. Measured: 256 x 16
// pairs over 256..8,192-token prompts 1,948 -> 1,721 us; 1,024 x 16 pairs
// over 32..1,024-token prompts 1,255 us in request order, 1,322 us ordered.
// Commits of B rows per request keep request order. `lds` holds
// kPrefillOrderLds ints, free again on return; every thread of the
// work-group calls it.
constexpr int kPrefillOrderMax = 2048;
constexpr int64_t kPrefillOrderPairs = 8192;
constexpr int kPrefillOrderLds = 256 + 16 + 2;

__device__ __forceinline__ int prefill_bucket(int n)
{
    if (n <= 1) return 255;
    const int e = 31 - __builtin_clz(static_cast<uint32_t>(n));  // 1 .. 30
    const int m = e >= 3 ? (n >> (e - 3)) & 7 : (n << (3 - e)) & 7;
    return 255 - (8 * e + m);  // 8 .. 247
}

template <int NT>
__device__ int prefill_request(const CommitArgs& a, int s, int tid, int* lds)
{
    static_assert(NT % 64 == 0 && NT / 64 <= 16, "one partial sum per wave");
    constexpr int PER = (kPrefillOrderMax + NT - 1) / NT;  // requests per thread, at most
    if (a.seq_offsets == nullptr || a.R > kPrefillOrderMax || static_cast<int64_t>(a.R) * a.H > kPrefillOrderPairs)
        return s;
    int* const hist = lds;        // [256]
    int* const wsum = lds + 256;  // [16]
    int* const sel = wsum + 16;   // [2]: bucket and offset, then the request
    const int lane = tid & 63, wave = tid / 64;
    // thread tid: requests r0 .. r0 + per - 1 (clamped to R); their buckets in
    // registers, from one round of loads of the offsets (and mask)
    const int per = (a.R + NT - 1) / NT, r0 = tid * per;
    int bk[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        bk[i] = -1;
        if (i < per && r0 + i < a.R) {
            int64_t f;
            int n;
            commit_rows(a, r0 + i, f, n);
            bk[i] = prefill_bucket(n);
        }
    }
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if (bk[i] >= 0) atomicAdd(&hist[bk[i]], 1);
    __syncthreads();
    if (wave == 0) {
        // lane l: buckets 4l .. 4l + 3
        int h[4], t = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = hist[4 * lane + i];
            t += h[i];
        }
        int x = t;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        int start = x - t;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (s >= start && s < start + h[i]) {
                sel[0] = 4 * lane + i;
                sel[1] = s - start;
            }
            start += h[i];
        }
    }
    __syncthreads();
    const int b = sel[0], o = sel[1];
    int c = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) c += bk[i] == b;
    int x = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int k = x - c;
    for (int w = 0; w < wave; ++w) k += wsum[w];
    if (o >= k && o < k + c) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (bk[i] == b) {
                if (k == o) sel[0] = r0 + i;
                ++k;
            }
    }
    __syncthreads();
    const int pick = sel[0];
    __syncthreads();  // every thread has its pick before the caller reuses lds
    return pick;
}

// Softmax attention of the block's queries over the request's prefix and the
// block: prefix rows seq_offsets[r] .. seq_offsets[r+1]-1 of kp, vp (clamped).
struct PrefixArgs {
    int R, H, d, B, io;
    float scale;  // resolved: never 0
    const void *q, *k, *v;
    bha_strides qs;
    const void *kp, *vp;
    bha_strides ps;  // ps.req unused
    const int32_t* seq_offsets;
    int64_t total_tokens;
    void* out;
    bha_strides os;
    // key-sequence split: with splits > 1 each (request, head) pair is spread
    // over `splits` work-groups that leave fp32 partial results in `part`
    // (splits * R * H records of prefix_part_floats(d) floats), merged by a
    // second launch
    float* part;
    int splits;
};

// Floats of one partial-result record of the split prefix attention: the
// unnormalised output [32][d], then the running maximum and normaliser [32] each.
__host__ __device__ inline int64_t prefix_part_floats(int d) { return 32 * static_cast<int64_t>(d) + 64; }

// Bytes of the static buffer the allocation-free prefix attention keeps its
// split partials in, and its address on the current device (looked up once
// per device).
constexpr int64_t kNoAllocScratchBytes = int64_t(9) << 20;
hipError_t noalloc_scratch(void** ptr);

// Key-sequence splits the matrix-core prefix attention uses for these sizes
// (1 when the pairs alone fill the GPU or the path does not apply).
int prefix_attention_splits(int R, int H, int d, int B, int io, int64_t total_tokens);
// 32-query tiles of a block of B tokens in the matrix-core prefix attention
// (one work-group per pair, query tile and key range).
int prefix_query_tiles(int B);

struct PhiArgs {
    int R, H, d, FW, B, io;
    const void* x;
    bha_strides xs;
    const void* w;
    int64_t wh;
    float* phi;
};

// Enqueues one kernel and returns that launch's own status. The thread's
// sticky last error (hipGetLastError) is neither read nor cleared: it may hold
// an error left by an earlier, unrelated call, which must not decide whether
// this launch happened.
template <typename T>
struct same_type {
    using type = T;
};
template <typename... KA>
inline hipError_t launch_kernel(void (*kernel)(KA...), dim3 grid, dim3 block, hipStream_t s,
                                typename same_type<KA>::type... args)
{
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s);
}

// Kernel choice is made on the host from the arguments alone: each
// *_supported predicate says whether its launcher covers the call; a launcher
// is only called for arguments its predicate accepts, and returns the status
// of the launches it enqueued.

// Softmax prefix attention: matrix-core kernel (bf16, B <= 64, 32-bit row
// offsets) and the fp32-arithmetic kernel for every size and both I/O dtypes.
bool prefix_attention_mfma_supported(const PrefixArgs& a);
hipError_t launch_prefix_attention_mfma(const PrefixArgs& a, hipStream_t s);
hipError_t launch_prefix_attention_generic(const PrefixArgs& a, hipStream_t s);

// Plain fp32-arithmetic kernels: every supported size and both I/O dtypes.
hipError_t launch_forward_generic(const ForwardArgs& a, hipStream_t s);
hipError_t launch_commit_generic(const CommitArgs& a, hipStream_t s);
hipError_t launch_feature_map_generic(const PhiArgs& a, hipStream_t s);

// bf16 MFMA kernels for bf16 I/O.
bool forward_mfma_supported(const ForwardArgs& a);
hipError_t launch_forward_mfma(const ForwardArgs& a, hipStream_t s);
bool commit_mfma_supported(const CommitArgs& a);
hipError_t launch_commit_mfma(const CommitArgs& a, hipStream_t s);
bool prefill_mfma_supported(const CommitArgs& a);
hipError_t launch_prefill_mfma(const CommitArgs& a, hipStream_t s);
// Forward of the block's last denoising step and the commit of its K, V in one
// pass over each pair's state (bf16, B <= 32); c carries the commit mask.
bool forward_commit_mfma_supported(const ForwardArgs& a);
hipError_t launch_forward_commit_mfma(const ForwardArgs& a, const CommitArgs& c, hipStream_t s);
bool feature_map_mfma_supported(const PhiArgs& a);
hipError_t launch_feature_map_mfma(const PhiArgs& a, hipStream_t s);

// Host-side argument checks (no HIP calls); see bha_validate.cpp.
int validate_dims(const bha_dims* d);
int validate_tokens(const void* p, const bha_strides* st, const bha_dims* d, bool is_output);
int validate_w(const void* w, int64_t w_head_stride, const bha_dims* d);
int validate_state(const void* state, int32_t num_slots, const int32_t* slot_ids,
                   const bha_dims* d);

}  // namespace bha
