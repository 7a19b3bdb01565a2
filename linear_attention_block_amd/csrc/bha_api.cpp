// C-ABI entry points of libbha.so: validate on the host, then enqueue the
// kernels on the caller's stream. The interface contract is in include/bha.h.
#include <math.h>
#include <stdint.h>

#include "bha_internal.hpp"

#define BHA_VERSION_NUMBER 10000 /* 1.0.0 */

using namespace bha;

// The status of the launches a call enqueued (each launcher returns its
// launches' own status; the thread's sticky last error is not consulted).
static int launch_status(hipError_t e) { return e == hipSuccess ? BHA_OK : BHA_ERR_HIP; }

// Kernel choice is made on the host before anything is enqueued: one
// launcher per call, picked by its *_supported predicate.
static hipError_t launch_forward_any(const ForwardArgs& a, hipStream_t stream)
{
    return forward_mfma_supported(a) ? launch_forward_mfma(a, stream) : launch_forward_generic(a, stream);
}

// A commit of B tokens per request: the commit kernel (bf16, B <= 32), the
// prefill kernel over each request's B rows (bf16, B <= 64), else the
// fp32-arithmetic commit kernel.
static hipError_t launch_commit_any(const CommitArgs& a, hipStream_t stream)
{
    if (commit_mfma_supported(a)) return launch_commit_mfma(a, stream);
    if (prefill_mfma_supported(a)) return launch_prefill_mfma(a, stream);
    return launch_commit_generic(a, stream);
}

extern "C" int bha_feature_map(const bha_dims* dims, const void* x, const bha_strides* xs,
                               const void* w, int64_t w_head_stride, float* phi,
                               hipStream_t stream)
{
    int st = validate_dims(dims);
    if (st != BHA_OK) return st;
    if (dims->num_requests == 0) return BHA_OK;
    if ((st = validate_tokens(x, xs, dims, false)) != BHA_OK) return st;
    if ((st = validate_w(w, w_head_stride, dims)) != BHA_OK) return st;
    if (!phi) return BHA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(phi) % 4 != 0) return BHA_ERR_ALIGN;
    PhiArgs a;
    a.R = dims->num_requests; a.H = dims->num_heads; a.d = dims->head_dim;
    a.FW = dims->feat_half; a.B = dims->block_size; a.io = dims->io_dtype;
    a.x = x; a.xs = *xs; a.w = w; a.wh = w_head_stride; a.phi = phi;
    return launch_status(feature_map_mfma_supported(a) ? launch_feature_map_mfma(a, stream)
                                                       : launch_feature_map_generic(a, stream));
}

extern "C" int bha_block_forward(const bha_dims* dims, const void* q, const void* k, const void* v,
                                 const bha_strides* qkv, const void* w, int64_t w_head_stride,
                                 const float* gamma, const float* state, int32_t num_slots,
                                 const int32_t* slot_ids, void* out, const bha_strides* outs,
                                 hipStream_t stream)
{
    int st = validate_dims(dims);
    if (st != BHA_OK) return st;
    if (dims->num_requests == 0) return BHA_OK;
    if ((st = validate_tokens(q, qkv, dims, false)) != BHA_OK) return st;
    if ((st = validate_tokens(k, qkv, dims, false)) != BHA_OK) return st;
    if ((st = validate_tokens(v, qkv, dims, false)) != BHA_OK) return st;
    if ((st = validate_w(w, w_head_stride, dims)) != BHA_OK) return st;
    if (!gamma) return BHA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(gamma) % 4 != 0) return BHA_ERR_ALIGN;
    if ((st = validate_state(state, num_slots, slot_ids, dims)) != BHA_OK) return st;
    if ((st = validate_tokens(out, outs, dims, true)) != BHA_OK) return st;
    ForwardArgs a;
    a.R = dims->num_requests; a.H = dims->num_heads; a.d = dims->head_dim;
    a.FW = dims->feat_half; a.B = dims->block_size; a.io = dims->io_dtype;
    a.scale = dims->scale > 0.0f ? dims->scale : 1.0f / sqrtf((float)dims->head_dim);
    a.q = q; a.k = k; a.v = v; a.qs = *qkv; a.ks = *qkv; a.G = 1;
    a.w = w; a.wh = w_head_stride; a.gamma = gamma;
    a.state = state; a.num_slots = num_slots; a.slot_ids = slot_ids; a.out = out; a.os = *outs;
    return launch_status(launch_forward_any(a, stream));
}

extern "C" int bha_block_forward_gqa(const bha_dims* dims, int32_t num_kv_heads, const void* q,
                                     const bha_strides* qs, const void* k, const void* v, const bha_strides* kvs,
                                     const void* w, int64_t w_head_stride, const float* gamma, const float* state,
                                     int32_t num_slots, const int32_t* slot_ids, void* out,
                                     const bha_strides* outs, hipStream_t stream)
{
    int st = validate_dims(dims);
    if (st != BHA_OK) return st;
    if (num_kv_heads < 1 || dims->num_heads % num_kv_heads != 0) return BHA_ERR_DIMS;
    if (dims->num_requests == 0) return BHA_OK;
    // K, V, W and the state have num_kv_heads heads
    bha_dims kvd = *dims;
    kvd.num_heads = num_kv_heads;
    if ((st = validate_tokens(q, qs, dims, false)) != BHA_OK) return st;
    if ((st = validate_tokens(k, kvs, &kvd, false)) != BHA_OK) return st;
    if ((st = validate_tokens(v, kvs, &kvd, false)) != BHA_OK) return st;
    if ((st = validate_w(w, w_head_stride, &kvd)) != BHA_OK) return st;
    if (!gamma) return BHA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(gamma) % 4 != 0) return BHA_ERR_ALIGN;
    if ((st = validate_state(state, num_slots, slot_ids, &kvd)) != BHA_OK) return st;
    if ((st = validate_tokens(out, outs, dims, true)) != BHA_OK) return st;
    ForwardArgs a;
    a.R = dims->num_requests; a.H = dims->num_heads; a.d = dims->head_dim;
    a.FW = dims->feat_half; a.B = dims->block_size; a.io = dims->io_dtype;
    a.scale = dims->scale > 0.0f ? dims->scale : 1.0f / sqrtf((float)dims->head_dim);
    a.q = q; a.k = k; a.v = v; a.qs = *qs; a.ks = *kvs; a.G = dims->num_heads / num_kv_heads;
    a.w = w; a.wh = w_head_stride; a.gamma = gamma;
    a.state = state; a.num_slots = num_slots; a.slot_ids = slot_ids; a.out = out; a.os = *outs;
    return launch_status(launch_forward_any(a, stream));
}

extern "C" int bha_state_commit(const bha_dims* dims, const void* k, const void* v,
                                const bha_strides* kv, const void* w, int64_t w_head_stride,
                                float* state, int32_t num_slots, const int32_t* slot_ids,
                                hipStream_t stream)
{
    int st = validate_dims(dims);
    if (st != BHA_OK) return st;
    if (dims->num_requests == 0) return BHA_OK;
    if ((st = validate_tokens(k, kv, dims, false)) != BHA_OK) return st;
    if ((st = validate_tokens(v, kv, dims, false)) != BHA_OK) return st;
    if ((st = validate_w(w, w_head_stride, dims)) != BHA_OK) return st;
    if ((st = validate_state(state, num_slots, slot_ids, dims)) != BHA_OK) return st;
    CommitArgs a;
    a.R = dims->num_requests; a.H = dims->num_heads; a.d = dims->head_dim;
    a.FW = dims->feat_half; a.B = dims->block_size; a.io = dims->io_dtype;
    a.k = k; a.v = v; a.ks = *kv; a.w = w; a.wh = w_head_stride;
    a.state = state; a.num_slots = num_slots; a.slot_ids = slot_ids;
    a.seq_offsets = nullptr; a.total_tokens = 0; a.commit_mask = nullptr;
    return launch_status(launch_commit_any(a, stream));
}

extern "C" int bha_block_forward_commit(const bha_dims* dims, const void* q, const void* k, const void* v,
                                        const bha_strides* qkv, const void* w, int64_t w_head_stride,
                                        const float* gamma, float* state, int32_t num_slots,
                                        const int32_t* slot_ids, const uint8_t* commit_mask, void* out,
                                        const bha_strides* outs, hipStream_t stream)
{
    int st = validate_dims(dims);
    if (st != BHA_OK) return st;
    if (dims->num_requests == 0) return BHA_OK;
    if ((st = validate_tokens(q, qkv, dims, false)) != BHA_OK) return st;
    if ((st = validate_tokens(k, qkv, dims, false)) != BHA_OK) return st;
    if ((st = validate_tokens(v, qkv, dims, false)) != BHA_OK) return st;
    if ((st = validate_w(w, w_head_stride, dims)) != BHA_OK) return st;
    if (!gamma) return BHA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(gamma) % 4 != 0) return BHA_ERR_ALIGN;
    if ((st = validate_state(state, num_slots, slot_ids, dims)) != BHA_OK) return st;
    if ((st = validate_tokens(out, outs, dims, true)) != BHA_OK) return st;
    ForwardArgs a;
    a.R = dims->num_requests; a.H = dims->num_heads; a.d = dims->head_dim;
    a.FW = dims->feat_half; a.B = dims->block_size; a.io = dims->io_dtype;
    a.scale = dims->scale > 0.0f ? dims->scale : 1.0f / sqrtf((float)dims->head_dim);
    a.q = q; a.k = k; a.v = v; a.qs = *qkv; a.ks = *qkv; a.G = 1;
    a.w = w; a.wh = w_head_stride; a.gamma = gamma;
    a.state = state; a.num_slots = num_slots; a.slot_ids = slot_ids; a.out = out; a.os = *outs;
    CommitArgs c;
    c.R = a.R; c.H = a.H; c.d = a.d; c.FW = a.FW; c.B = a.B; c.io = a.io;
    c.k = k; c.v = v; c.ks = *qkv; c.w = w; c.wh = w_head_stride;
    c.state = state; c.num_slots = num_slots; c.slot_ids = slot_ids;
    c.seq_offsets = nullptr; c.total_tokens = 0; c.commit_mask = commit_mask;
    if (forward_commit_mfma_supported(a)) return launch_status(launch_forward_commit_mfma(a, c, stream));
    // the same result in two launches: the forward reads the state before the
    // commit changes it (both on the caller's stream)
    hipError_t e = launch_forward_any(a, stream);
    if (e == hipSuccess) e = launch_commit_any(c, stream);
    return launch_status(e);
}

extern "C" int bha_state_prefill(const bha_dims* dims, const void* k, const void* v, const bha_strides* kv,
                                 const int32_t* seq_offsets, int64_t total_tokens, const void* w,
                                 int64_t w_head_stride, float* state, int32_t num_slots,
                                 const int32_t* slot_ids, hipStream_t stream)
{
    int st = validate_dims(dims);
    if (st != BHA_OK) return st;
    if (dims->num_requests == 0) return BHA_OK;
    if (total_tokens < 0) return BHA_ERR_DIMS;
    if (!seq_offsets || !kv) return BHA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(seq_offsets) % 4 != 0) return BHA_ERR_ALIGN;
    if (total_tokens == 0) return BHA_OK;
    // the packed tokens, checked as one "request" of total_tokens rows
    bha_dims packed = *dims;
    packed.num_requests = 1;
    if (total_tokens > INT32_MAX) return BHA_ERR_DIMS;
    packed.block_size = static_cast<int32_t>(total_tokens);
    bha_strides ps = *kv;
    ps.req = 0;
    if ((st = validate_tokens(k, &ps, &packed, false)) != BHA_OK) return st;
    if ((st = validate_tokens(v, &ps, &packed, false)) != BHA_OK) return st;
    if ((st = validate_w(w, w_head_stride, dims)) != BHA_OK) return st;
    if ((st = validate_state(state, num_slots, slot_ids, dims)) != BHA_OK) return st;
    CommitArgs a;
    a.R = dims->num_requests; a.H = dims->num_heads; a.d = dims->head_dim;
    a.FW = dims->feat_half; a.B = dims->block_size; a.io = dims->io_dtype;
    a.k = k; a.v = v; a.ks = ps; a.w = w; a.wh = w_head_stride;
    a.state = state; a.num_slots = num_slots; a.slot_ids = slot_ids;
    a.seq_offsets = seq_offsets; a.total_tokens = total_tokens; a.commit_mask = nullptr;
    return launch_status(prefill_mfma_supported(a) ? launch_prefill_mfma(a, stream) : launch_commit_generic(a, stream));
}

static int64_t prefix_workspace_bytes(const bha_dims* d, int splits)
{
    if (splits < 2) return 0;
    return static_cast<int64_t>(d->num_requests) * d->num_heads * prefix_query_tiles(d->block_size) * splits *
           prefix_part_floats(d->head_dim) * 4;
}

extern "C" int64_t bha_prefix_attention_workspace(const bha_dims* dims, int64_t total_tokens)
{
    int st = validate_dims(dims);
    if (st != BHA_OK) return st;
    if (total_tokens < 0 || total_tokens > INT32_MAX) return BHA_ERR_DIMS;
    if (dims->num_requests == 0) return 0;
    return prefix_workspace_bytes(dims, prefix_attention_splits(dims->num_requests, dims->num_heads, dims->head_dim,
                                                                dims->block_size, dims->io_dtype, total_tokens));
}

// Validation and marshalling shared by the two prefix-attention entry points;
// fills everything but the split and its partial-result buffer.
static int prefix_prepare(const bha_dims* dims, const void* q, const void* k, const void* v, const bha_strides* qkv,
                          const void* kp, const void* vp, const bha_strides* kvp, const int32_t* seq_offsets,
                          int64_t total_tokens, void* out, const bha_strides* outs, PrefixArgs& a)
{
    int st;
    if ((st = validate_tokens(q, qkv, dims, false)) != BHA_OK) return st;
    if ((st = validate_tokens(k, qkv, dims, false)) != BHA_OK) return st;
    if ((st = validate_tokens(v, qkv, dims, false)) != BHA_OK) return st;
    if ((st = validate_tokens(out, outs, dims, true)) != BHA_OK) return st;
    if (total_tokens < 0 || total_tokens > INT32_MAX) return BHA_ERR_DIMS;
    if (!seq_offsets || !kvp) return BHA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(seq_offsets) % 4 != 0) return BHA_ERR_ALIGN;
    bha_strides ps = *kvp;
    ps.req = 0;
    if (total_tokens > 0) {
        // the packed prefix, checked as one "request" of total_tokens rows
        bha_dims packed = *dims;
        packed.num_requests = 1;
        packed.block_size = static_cast<int32_t>(total_tokens);
        if ((st = validate_tokens(kp, &ps, &packed, false)) != BHA_OK) return st;
        if ((st = validate_tokens(vp, &ps, &packed, false)) != BHA_OK) return st;
    } else {
        kp = k;  // no prefix rows are read
        vp = v;
        ps.tok = qkv->tok;
        ps.head = qkv->head;
    }
    a.part = nullptr;
    a.splits = 1;
    a.R = dims->num_requests; a.H = dims->num_heads; a.d = dims->head_dim;
    a.B = dims->block_size; a.io = dims->io_dtype;
    a.scale = dims->scale > 0.0f ? dims->scale : 1.0f / sqrtf((float)dims->head_dim);
    a.q = q; a.k = k; a.v = v; a.qs = *qkv; a.kp = kp; a.vp = vp; a.ps = ps;
    a.seq_offsets = seq_offsets; a.total_tokens = total_tokens; a.out = out; a.os = *outs;
    return BHA_OK;
}

static hipError_t launch_prefix_any(const PrefixArgs& a, hipStream_t stream)
{
    return prefix_attention_mfma_supported(a) ? launch_prefix_attention_mfma(a, stream)
                                              : launch_prefix_attention_generic(a, stream);
}

extern "C" int bha_prefix_attention(const bha_dims* dims, const void* q, const void* k, const void* v,
                                    const bha_strides* qkv, const void* kp, const void* vp, const bha_strides* kvp,
                                    const int32_t* seq_offsets, int64_t total_tokens, void* workspace,
                                    int64_t workspace_bytes, void* out, const bha_strides* outs, hipStream_t stream)
{
    int st = validate_dims(dims);
    if (st != BHA_OK) return st;
    if (dims->num_requests == 0) return BHA_OK;
    PrefixArgs a;
    if ((st = prefix_prepare(dims, q, k, v, qkv, kp, vp, kvp, seq_offsets, total_tokens, out, outs, a)) != BHA_OK)
        return st;
    if (workspace_bytes < 0) return BHA_ERR_DIMS;
    if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return BHA_ERR_ALIGN;
    // the split the workspace allows (fewer splits, down to none, when it is short)
    int splits = prefix_attention_splits(dims->num_requests, dims->num_heads, dims->head_dim, dims->block_size,
                                         dims->io_dtype, total_tokens);
    const int64_t per_split = prefix_workspace_bytes(dims, 2) / 2;
    const int64_t fit = workspace ? workspace_bytes / per_split : 0;
    if (splits > fit) splits = static_cast<int>(fit);
    if (splits < 2) splits = 1;
    a.part = splits > 1 ? static_cast<float*>(workspace) : nullptr;
    a.splits = splits;
    return launch_status(launch_prefix_any(a, stream));
}

extern "C" int bha_prefix_attention_noalloc(const bha_dims* dims, const void* q, const void* k, const void* v,
                                            const bha_strides* qkv, const void* kp, const void* vp,
                                            const bha_strides* kvp, const int32_t* seq_offsets,
                                            int64_t total_tokens, void* out, const bha_strides* outs,
                                            hipStream_t stream)
{
    int st = validate_dims(dims);
    if (st != BHA_OK) return st;
    if (dims->num_requests == 0) return BHA_OK;
    PrefixArgs a;
    if ((st = prefix_prepare(dims, q, k, v, qkv, kp, vp, kvp, seq_offsets, total_tokens, out, outs, a)) != BHA_OK)
        return st;
    // the split bha_prefix_attention takes with a full workspace
    const int splits = prefix_attention_splits(dims->num_requests, dims->num_heads, dims->head_dim,
                                               dims->block_size, dims->io_dtype, total_tokens);
    if (prefix_workspace_bytes(dims, splits) > kNoAllocScratchBytes) return BHA_ERR_SCRATCH;
    void* scratch_ptr = nullptr;
    if (noalloc_scratch(&scratch_ptr) != hipSuccess) return BHA_ERR_HIP;
    a.part = splits > 1 ? static_cast<float*>(scratch_ptr) : nullptr;
    a.splits = splits;
    return launch_status(launch_prefix_any(a, stream));
}

extern "C" int64_t bha_prefix_attention_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int64_t bha_state_record_floats(int32_t head_dim, int32_t feat_half)
{
    if (head_dim != 64 && head_dim != 128) return -1;
    if (feat_half != 32 && feat_half != 64 && feat_half != 128) return -1;
    return (int64_t)(head_dim + 1) * 2 * feat_half;
}

extern "C" const char* bha_status_string(int status)
{
    switch (status) {
        case BHA_OK: return "BHA_OK: success";
        case BHA_ERR_NULL: return "BHA_ERR_NULL: a required pointer is NULL";
        case BHA_ERR_DIMS: return "BHA_ERR_DIMS: bad count, scale or size overflow";
        case BHA_ERR_UNSUPPORTED: return "BHA_ERR_UNSUPPORTED: head_dim, feat_half or block_size not supported";
        case BHA_ERR_ALIGN: return "BHA_ERR_ALIGN: pointer not aligned";
        case BHA_ERR_STRIDE: return "BHA_ERR_STRIDE: negative, misaligned or overlapping stride";
        case BHA_ERR_DTYPE: return "BHA_ERR_DTYPE: io_dtype is not a bha_dtype value";
        case BHA_ERR_HIP: return "BHA_ERR_HIP: the HIP runtime reported an error";
        case BHA_ERR_SCRATCH:
            return "BHA_ERR_SCRATCH: the call needs more scratch than the library's static device buffer";
        default: return "unknown bha_status";
    }
}

extern "C" int bha_version(void) { return BHA_VERSION_NUMBER; }

// Set by the build to a hash of the library's source files.
#ifndef BHA_SOURCE_HASH
#define BHA_SOURCE_HASH "unknown"
#endif

extern "C" const char* bha_source_hash(void) { return BHA_SOURCE_HASH; }
