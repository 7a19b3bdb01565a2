/*
 * bha.h -- C ABI of the block-hybrid attention library (libbha.so, gfx950).
 *
 * Block-hybrid attention, as described for "Retrofitting Linear Attention into
 * Diffusion Language Models" (Kim, Roh, Kim): inside the active denoising
 * block of B tokens every query attends to every key of the block with exact,
 * unmasked softmax; all previously committed blocks are folded into a fixed
 * size recurrent state that the query reads through the Hedgehog feature map
 *     phi(x) = [ softmax(x W), softmax(-x W) ]        (dimension F = 2 FW)
 * with  S = sum_t phi(k_t) v_t^T  (F x d)  and  Z = sum_t phi(k_t)  (F).
 * The two branches share one normaliser and a per-head gate g >= 0:
 *     y_i = ( sum_j e^{s_ij - m_i} v_j + g e^{-m_i} phi(q_i)^T S )
 *         / ( sum_j e^{s_ij - m_i}     + g e^{-m_i} phi(q_i)^T Z ),
 *     s_ij = scale * q_i . k_j,  m_i = max_j s_ij.
 * Where the pages define each piece:
 *   - gist.science explainer, "Technical Summary", "Methodology: Block-Hybrid
 *     Attention", list "Architecture Design": within-block softmax, the
 *     cross-block Hedgehog map, the S_n / Z_n states updated only at a commit,
 *     and the merge under a shared normaliser with a learned scalar gate.
 *   - pith.science review, "The reading", "What carries the argument": the
 *     formulas of phi, S_n and Z_n, one map per head, O(F d) read per query.
 *   - pith.science review, "Circularity Check": the state sizes do not grow
 *     with the number of committed tokens.
 * The pages do not print where the gate and m sit; the form above is this
 * library's definition.
 *
 * Conventions common to every entry point
 *   - All tensor pointers are DEVICE pointers; descriptor structs (bha_dims,
 *     bha_strides) are HOST pointers read during the call only.
 *   - Ownership: the caller allocates and frees every buffer. The library never
 *     allocates, frees or synchronises; it keeps no state between calls and is
 *     reentrant.
 *   - Asynchrony: work is enqueued on `stream` (0 = the null stream) and the
 *     call returns without waiting. Calls on one stream run in order; a commit
 *     must be enqueued after the last forward that should not see its block.
 *   - Errors: arguments are checked on the host before anything is enqueued. A
 *     bad argument returns a negative bha_status and enqueues nothing. A
 *     failed launch returns BHA_ERR_HIP. num_requests == 0 returns BHA_OK
 *     without reading any pointer.
 *   - Device-side preconditions (not checkable on the host): slot ids in
 *     [0, num_slots) -- a request with an out-of-range slot gets NaN outputs
 *     from the forward and is skipped by the commit; slot ids of one commit
 *     call are distinct (duplicates race); gamma >= 0; outputs do not alias
 *     inputs.
 *
 * Layouts (elements, not bytes, in every stride)
 *   Tokens  q, k, v, out : element (r, t, h, c) at  r*req + t*tok + h*head + c
 *                          (r < R requests, t < B tokens, h < H heads, c < d);
 *                          the last dimension is contiguous.
 *   Map     w            : element (h, j, c) at  h*w_head_stride + j*d + c
 *                          holds W_h[c][j], i.e. row j is column j of the
 *                          d x FW matrix (the usual [out][in] weight layout);
 *                          w_head_stride == 0 shares one W across heads.
 *   Gate    gamma        : float32 [H].
 *   State   state        : float32, one record of (d+1)*F floats per
 *                          (slot, head), record (s, h) at (s*H + h)*(d+1)*F.
 *                          Inside a record, S[f][c] (f < F, c < d) is stored in
 *                          32 x 4 tiles so that 128-bit loads are contiguous:
 *                            offset((c/32)*(F/4) + f/4)*128 + (c%32)*4 + f%4,
 *                          and Z[f] sits at offset d*F + f. A zero record is
 *                          the state of a request with nothing committed.
 *   Dtypes: tokens, w and out use dims->io_dtype (float32 or bfloat16);
 *           state, gamma and phi are always float32.
 *   Alignment: every token / w / out pointer, every stride times the element
 *           size, and state must be multiples of 16 bytes; gamma, slot_ids
 *           and phi multiples of 4 bytes.
 *   Supported sizes: d in {64, 128}; FW in {32, 64, 128}; 1 <= B <= 64;
 *           1 <= H; 0 <= R. scale == 0 selects 1/sqrt(d).
 */
#ifndef BHA_H
#define BHA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BHA_OK = 0,
    BHA_ERR_NULL = -1,        /* a required pointer is NULL */
    BHA_ERR_DIMS = -2,        /* negative / zero count, bad scale, size overflow */
    BHA_ERR_UNSUPPORTED = -3, /* d, FW or B outside the supported set */
    BHA_ERR_ALIGN = -4,       /* pointer not aligned as stated above */
    BHA_ERR_STRIDE = -5,      /* negative or misaligned stride, rows overlapping */
    BHA_ERR_DTYPE = -6,       /* io_dtype not a bha_dtype value */
    BHA_ERR_HIP = -7,         /* the HIP runtime reported an error at launch */
    BHA_ERR_SCRATCH = -8      /* more scratch than the static buffer of the allocation-free call */
} bha_status;

typedef enum { BHA_F32 = 0, BHA_BF16 = 1 } bha_dtype;

typedef struct {
    int32_t num_requests; /* R: requests in this call (0 => no-op)            */
    int32_t num_heads;    /* H                                                 */
    int32_t head_dim;     /* d  in {64, 128}                                   */
    int32_t feat_half;    /* FW in {32, 64, 128}: columns of W; F = 2 * FW     */
    int32_t block_size;   /* B  in [1, 64]: tokens of the active block         */
    int32_t io_dtype;     /* bha_dtype of q, k, v, w, out and x                */
    float scale;          /* softmax scale of the block logits; 0 => 1/sqrt(d) */
} bha_dims;

typedef struct {
    int64_t req;  /* between requests */
    int64_t tok;  /* between tokens of a block */
    int64_t head; /* between heads */
} bha_strides;

/*
 * bha_feature_map -- phi(x) = [softmax(x W_h), softmax(-x W_h)] for every
 * token of a [R][B][H][d] batch (gist.science "Architecture Design",
 * cross-block bullet; pith.science "What carries the argument").
 *   x   : tokens, strides xs.
 *   phi : float32 output, contiguous [R][B][H][F].
 */
int bha_feature_map(const bha_dims* dims, const void* x, const bha_strides* xs,
                    const void* w, int64_t w_head_stride, float* phi, hipStream_t stream);

/*
 * bha_block_forward -- one denoising step of block-hybrid attention for every
 * (request, head): the within-block softmax over q, k, v, the linear read
 * phi(q)^T S, phi(q)^T Z of the request's state record, and the gated merge
 * written at the top of this file (gist.science "Architecture Design", all
 * four bullets; pith.science "What carries the argument").
 *   q, k, v      : active block tokens, strides qkv.
 *   gamma        : per-head gate.
 *   state        : num_slots * H records (read only).
 *   slot_ids     : int32 [R], the state slot of each request.
 *   out          : tokens in io_dtype, strides outs.
 */
int bha_block_forward(const bha_dims* dims, const void* q, const void* k, const void* v,
                      const bha_strides* qkv, const void* w, int64_t w_head_stride,
                      const float* gamma, const float* state, int32_t num_slots,
                      const int32_t* slot_ids, void* out, const bha_strides* outs,
                      hipStream_t stream);

/*
 * bha_block_forward_gqa -- bha_block_forward with H query heads sharing
 * num_kv_heads K/V heads (grouped queries, G = H / num_kv_heads query heads
 * per K/V head): query head h attends, within the block, to the keys and
 * values of K/V head h / G and reads that head's state with that head's W,
 * so S and Z are kept once per K/V head. Not on the pages, whose model has
 * one K/V head per query head: a variant for models with grouped K/V heads.
 * The feature map stays one W applied to queries and keys alike; the K/V
 * head's W serves its G query heads.
 *   dims->num_heads : H, query heads; must be a multiple of num_kv_heads.
 *   q, out          : [R][B][H][d] with strides *qs, *outs.
 *   k, v            : [R][B][num_kv_heads][d] with strides *kvs.
 *   w               : num_kv_heads maps (w_head_stride apart, 0 = shared).
 *   gamma           : [H] float32, one gate per query head.
 *   state, slot_ids : as for bha_block_forward with num_kv_heads heads per
 *                     slot; built by bha_state_commit / bha_state_prefill
 *                     called with dims->num_heads = num_kv_heads.
 * num_kv_heads == H is bha_block_forward. Errors as for bha_block_forward;
 * num_kv_heads < 1 or not dividing H: BHA_ERR_DIMS.
 */
int bha_block_forward_gqa(const bha_dims* dims, int32_t num_kv_heads, const void* q, const bha_strides* qs,
                          const void* k, const void* v, const bha_strides* kvs, const void* w,
                          int64_t w_head_stride, const float* gamma, const float* state, int32_t num_slots,
                          const int32_t* slot_ids, void* out, const bha_strides* outs, hipStream_t stream);

/*
 * bha_state_commit -- fold a finished block into the state of every
 * (request, head): S += sum_t phi(k_t) v_t^T and Z += sum_t phi(k_t) over the
 * B tokens (gist.science "Architecture Design", state-compression bullet: the
 * states change only when a block is committed; pith.science "What carries
 * the argument"). A read-modify-write of each touched record; slot ids must
 * be distinct within one call.
 */
int bha_state_commit(const bha_dims* dims, const void* k, const void* v, const bha_strides* kv,
                     const void* w, int64_t w_head_stride, float* state, int32_t num_slots,
                     const int32_t* slot_ids, hipStream_t stream);

/*
 * bha_block_forward_commit -- the last denoising step of a block: the forward
 * of bha_block_forward, from the state as it stands (committed blocks only),
 * and then, for the requests whose commit_mask entry is non-zero, the commit
 * of bha_state_commit with the same k and v (gist.science "Architecture
 * Design": the states change only when a block is committed; "Key
 * Contributions": the state is kept per request so that requests at
 * different points join one continuously batched step). Equal to
 * bha_block_forward followed by bha_state_commit on the committing requests,
 * with each record read once and written once.
 *   commit_mask : uint8 [R] device, or NULL for every request.
 *   state       : read and, for committing requests, updated in place; slot
 *                 ids of committing requests must be distinct.
 * Other arguments as for bha_block_forward.
 */
int bha_block_forward_commit(const bha_dims* dims, const void* q, const void* k, const void* v,
                             const bha_strides* qkv, const void* w, int64_t w_head_stride,
                             const float* gamma, float* state, int32_t num_slots,
                             const int32_t* slot_ids, const uint8_t* commit_mask, void* out,
                             const bha_strides* outs, hipStream_t stream);

/*
 * bha_state_prefill -- fold a whole run of tokens per request into its state
 * in one launch: a prompt of any length, or several finished blocks at once.
 * For request r the tokens are rows seq_offsets[r] .. seq_offsets[r+1]-1 of
 * packed k and v, and S += sum_t phi(k_t) v_t^T, Z += sum_t phi(k_t) over
 * them -- the same sums a commit takes per block (gist.science "Architecture
 * Design", state-compression bullet; pith.science "What carries the
 * argument"), taken over all of them at once.
 *   k, v        : element (t, h, c) at t*kv->tok + h*kv->head + c for
 *                 t < total_tokens (kv->req is not used).
 *   seq_offsets : int32 [R + 1] device; clamped on the device to
 *                 0 <= seq_offsets[r] <= seq_offsets[r+1] <= total_tokens.
 *   dims->block_size must be a supported value but is not used.
 * Slot ids must be distinct (duplicates race). total_tokens == 0 is a no-op.
 */
int bha_state_prefill(const bha_dims* dims, const void* k, const void* v, const bha_strides* kv,
                      const int32_t* seq_offsets, int64_t total_tokens, const void* w,
                      int64_t w_head_stride, float* state, int32_t num_slots,
                      const int32_t* slot_ids, hipStream_t stream);

/*
 * bha_prefix_attention -- exact softmax attention of the active block's
 * queries over the request's whole prefix and the block itself: the attention
 * block-hybrid attention replaces, whose cost grows with the prefix
 * (gist.science "Problem Statement": every denoising step attends to all
 * previous blocks). For query i of request r and head h, over the prefix rows
 * t = seq_offsets[r] .. seq_offsets[r+1]-1 of kp, vp and then the B block
 * tokens (no mask):
 *   out_i = sum_t e^{s_it - m_i} v_t / sum_t e^{s_it - m_i},
 *   s_it = scale q_i . k_t, m_i = max_t s_it.
 *   q, k, v, out : as for bha_block_forward.
 *   kp, vp       : packed prefix tokens, element (t, h, c) at
 *                  t*kvp->tok + h*kvp->head + c for t < total_tokens
 *                  (kvp->req is not used); may be NULL when total_tokens == 0.
 *   seq_offsets  : int32 [R + 1] device, clamped on the device to
 *                  0 <= seq_offsets[r] <= seq_offsets[r+1] <= total_tokens.
 *   workspace    : device scratch of workspace_bytes (16-byte aligned), owned
 *                  by the caller, or NULL. When the (request, head) pairs are
 *                  too few to fill the GPU, each pair's keys are split over
 *                  several work-groups whose partial results go here; with a
 *                  shorter (or no) workspace the call splits less (or not at
 *                  all) and is slower but gives the same result up to rounding.
 *                  bha_prefix_attention_workspace gives the size for the full
 *                  split. Calls that share a workspace must not overlap.
 *   dims->feat_half must be a supported value but is not used.
 * No state is read; nothing is written but out and the workspace.
 */
int bha_prefix_attention(const bha_dims* dims, const void* q, const void* k, const void* v,
                         const bha_strides* qkv, const void* kp, const void* vp, const bha_strides* kvp,
                         const int32_t* seq_offsets, int64_t total_tokens, void* workspace,
                         int64_t workspace_bytes, void* out, const bha_strides* outs, hipStream_t stream);

/* Workspace bytes bha_prefix_attention uses for these dims and total_tokens
 * (0: no split), or a negative bha_status for invalid arguments. */
int64_t bha_prefix_attention_workspace(const bha_dims* dims, int64_t total_tokens);

/*
 * bha_prefix_attention_noalloc -- bha_prefix_attention for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Arguments, layouts and result are
 * those of bha_prefix_attention with a full workspace (the same split, so the
 * same output bit for bit), but the split's partial results go to a static
 * device buffer of bha_prefix_attention_noalloc_scratch_bytes() bytes (9 MiB)
 * that the library holds on every GPU it runs on until the process ends. The
 * call allocates and frees nothing; its first call on a device looks the
 * buffer's address up once (with that device current). It runs on the current
 * device: `stream` must belong to it.
 *   Errors: as bha_prefix_attention; a call whose split would need more than
 *   the buffer returns BHA_ERR_SCRATCH and enqueues nothing (the split rule of
 *   this version needs at most 8,486,400 bytes, so this is never returned).
 *   Concurrency: every call on one GPU uses that GPU's one buffer, which keeps
 *   the last call's contents (nothing in it needs to start at zero). Calls
 *   that overlap in time on one GPU -- on other streams or from other threads
 *   -- race on it; the caller must serialise them.
 */
int bha_prefix_attention_noalloc(const bha_dims* dims, const void* q, const void* k, const void* v,
                                 const bha_strides* qkv, const void* kp, const void* vp, const bha_strides* kvp,
                                 const int32_t* seq_offsets, int64_t total_tokens, void* out,
                                 const bha_strides* outs, hipStream_t stream);

/* Bytes of the static device buffer bha_prefix_attention_noalloc uses. */
int64_t bha_prefix_attention_noalloc_scratch_bytes(void);

/* Floats in one (slot, head) state record: (d + 1) * 2 * FW. Returns -1 for
 * unsupported sizes. Host only; touches no device. */
int64_t bha_state_record_floats(int32_t head_dim, int32_t feat_half);

/* Static description of a status code; never NULL. */
const char* bha_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int bha_version(void);

/* Identity of the build: the first 16 hex digits of a SHA-256 over the source
 * files the library was built from (its csrc sources and headers and this
 * header), fixed when it is compiled; "unknown" for a build that did not set
 * it. Static string, never NULL. The Python binding refuses an in-tree
 * library whose hash differs from that of the sources beside it, so a stale
 * build fails loudly instead of running other code. */
const char* bha_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* BHA_H */
