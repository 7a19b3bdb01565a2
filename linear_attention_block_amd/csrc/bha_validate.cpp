// Host-side argument validation for the C ABI. Makes no HIP call, so every
// error path can be exercised without a GPU.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "bha_internal.hpp"

namespace bha {

static bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static int64_t elem_size(int io) { return io == BHA_BF16 ? 2 : 4; }

int validate_dims(const bha_dims* d)
{
    if (!d) return BHA_ERR_NULL;
    if (d->io_dtype != BHA_F32 && d->io_dtype != BHA_BF16) return BHA_ERR_DTYPE;
    if (d->num_requests < 0 || d->num_heads < 1) return BHA_ERR_DIMS;
    if (!(d->scale >= 0.0f) || isinf(d->scale)) return BHA_ERR_DIMS;
    if (d->head_dim != 64 && d->head_dim != 128) return BHA_ERR_UNSUPPORTED;
    if (d->feat_half != 32 && d->feat_half != 64 && d->feat_half != 128) return BHA_ERR_UNSUPPORTED;
    if (d->block_size < 1 || d->block_size > 64) return BHA_ERR_UNSUPPORTED;
    // launch grids have at most R * H * 64 work-groups
    if (static_cast<int64_t>(d->num_requests) * d->num_heads * 64 > INT32_MAX) return BHA_ERR_DIMS;
    return BHA_OK;
}

// A token tensor [R][B][H][d] with element strides *st. Outputs must not have
// two (r, t, h) rows overlapping; inputs may (a zero stride broadcasts).
int validate_tokens(const void* p, const bha_strides* st, const bha_dims* d, bool is_output)
{
    if (!p || !st) return BHA_ERR_NULL;
    if (!aligned(p, 16)) return BHA_ERR_ALIGN;
    const int64_t es = elem_size(d->io_dtype);
    const int64_t s[3] = {st->req, st->tok, st->head};
    const int64_t n[3] = {d->num_requests, d->block_size, d->num_heads};
    int64_t last = d->head_dim;  // one past the largest element offset
    for (int i = 0; i < 3; ++i) {
        if (s[i] < 0 || (s[i] * es) % 16 != 0) return BHA_ERR_STRIDE;
        int64_t span;
        if (__builtin_mul_overflow(s[i], n[i] - 1, &span) || __builtin_add_overflow(last, span, &last))
            return BHA_ERR_DIMS;
    }
    int64_t bytes;
    if (__builtin_mul_overflow(last, es, &bytes)) return BHA_ERR_DIMS;
    if (is_output) {
        // Sort the dimensions that have more than one index by stride; each
        // stride must clear the extent of everything nested inside it.
        int idx[3] = {0, 1, 2};
        std::sort(idx, idx + 3, [&](int a, int b) { return s[a] < s[b]; });
        int64_t extent = d->head_dim;
        for (int i = 0; i < 3; ++i) {
            const int j = idx[i];
            if (n[j] <= 1) continue;
            if (s[j] < extent) return BHA_ERR_STRIDE;
            extent = s[j] * (n[j] - 1) + extent;
        }
    }
    return BHA_OK;
}

int validate_w(const void* w, int64_t w_head_stride, const bha_dims* d)
{
    if (!w) return BHA_ERR_NULL;
    if (!aligned(w, 16)) return BHA_ERR_ALIGN;
    const int64_t es = elem_size(d->io_dtype);
    if (w_head_stride < 0 || (w_head_stride * es) % 16 != 0) return BHA_ERR_STRIDE;
    int64_t span;
    if (__builtin_mul_overflow(w_head_stride, (int64_t)d->num_heads, &span)) return BHA_ERR_DIMS;
    return BHA_OK;
}

int validate_state(const void* state, int32_t num_slots, const int32_t* slot_ids, const bha_dims* d)
{
    if (!state || !slot_ids) return BHA_ERR_NULL;
    if (!aligned(state, 16)) return BHA_ERR_ALIGN;
    if (!aligned(slot_ids, 4)) return BHA_ERR_ALIGN;
    if (num_slots < 1) return BHA_ERR_DIMS;
    const int64_t rec = (int64_t)(d->head_dim + 1) * 2 * d->feat_half;
    int64_t n, bytes;
    if (__builtin_mul_overflow((int64_t)num_slots, (int64_t)d->num_heads, &n) ||
        __builtin_mul_overflow(n, rec, &n) || __builtin_mul_overflow(n, (int64_t)4, &bytes))
        return BHA_ERR_DIMS;
    return BHA_OK;
}

}  // namespace bha
