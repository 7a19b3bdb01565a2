// Exact softmax attention of the active block's queries over the request's
// whole prefix and the block itself -- the attention that block-hybrid
// attention replaces in the converted layers, whose cost grows with the prefix
// (gist.science "Problem Statement": every denoising step attends to all
// previous blocks; pith.science "What carries the argument": full attention is
// kept within the block only). For query i of request r and head h:
//   s_it = c q_i . k_t over the prefix rows t and the block's B tokens,
//   out_i = sum_t e^{s_it - m_i} v_t / sum_t e^{s_it - m_i},  m_i = max_t s_it.
//
// bf16 path (B <= 64): one work-group of four waves per (request, head,
// 32-query tile of the block; every tile attends to all keys). Wave
// w takes the 32-key chunks w, w + 4, ... of the prefix-then-block key
// sequence and keeps its own running maximum, normaliser and 32 x d output
// accumulator per query (online softmax); the four partial results are merged
// through LDS at the end, so the main loop has no work-group barrier. Per
// chunk: s^T = K Q^T with v_mfma_f32_32x32x16_bf16 (lane = query), K fragments
// loaded straight from global memory as one contiguous d/2-element run per
// lane (the contraction over d is fed in the order g, k-step kb -> elements
// g d/2 + 8 kb .. + 7 for both K and the Q fragments held in registers); the
// chunk's V rows go to the wave's own LDS tile and are read transposed
// (ds_read_b64_tr_b16) as the A operand of P V, P coming straight from the
// score accumulators. The next chunk's K and V loads are issued before the
// current chunk's arithmetic.
//
// When the (request, head) pairs alone cannot fill the GPU (a few requests
// with long prefixes), each pair's chunk sequence is cut into `splits`
// contiguous ranges, one work-group each; a work-group then leaves its
// unnormalised output, maximum and normaliser in fp32, and a second launch
// rescales the partial results to their common maximum and sums them.
//
// fp32 path (float32 I/O, and bf16 with token strides too large for the
// kernel above): the same layout and split on the fp32 matrix cores.
#include <mutex>

#include "bha_device.hpp"
#include "bha_internal.hpp"
#include "bha_mfma.hpp"

namespace bha {

namespace {

// Key row t of the key sequence (prefix rows first, then the block).
struct KeySource {
    const uint16_t* prefix;  // row 0 of the request's prefix, this head
    const uint16_t* block;   // token 0 of the block, this head
    int64_t ptok, btok;      // token strides (elements)
    int np, nk;              // prefix rows, keys in all (np + B)

    __device__ __forceinline__ const uint16_t* row(int t) const
    {
        t = t < nk ? t : nk - 1;  // past the end: the last key (masked)
        return t < np ? prefix + t * ptok : block + (t - np) * btok;
    }
};

template <int D>
struct SaCfg {
    static constexpr int NKB = D / 16;         // k-steps of the score contraction
    static constexpr int CT = D / 32;          // 32-column output tiles per wave
    static constexpr int VQ = 32 * (D / 8) / 64;  // 16-byte V chunks per lane per key chunk
    static constexpr int TILE = 32 * D;        // bf16 elements of one wave's K or V tile
    static constexpr int LDS_LOOP = 2 * 4 * TILE * 2;  // K and V tiles of four waves
    static constexpr int LDS_MERGE = 4 * D * 32 * 4 + 2 * 4 * 32 * 4;
    static constexpr int LDS = LDS_LOOP > LDS_MERGE ? LDS_LOOP : LDS_MERGE;
};

// Row-contiguous loads of one 32-key chunk: 16 lanes per 256-byte row (d =
// 128; 8 per row at d = 64), so each load instruction covers whole rows.
template <int D>
__device__ __forceinline__ void sa_load_chunk(const KeySource& ks, int c, int lane, u32x4 (&kr)[SaCfg<D>::VQ],
                                              u32x4 (&vr)[SaCfg<D>::VQ], const uint16_t* vprefix,
                                              const uint16_t* vblock)
{
    constexpr int CH = D / 8;
#pragma unroll
    for (int i = 0; i < SaCfg<D>::VQ; ++i) {
        const int idx = lane + 64 * i, t = idx / CH, ch = idx % CH;
        int tt = 32 * c + t;
        tt = tt < ks.nk ? tt : ks.nk - 1;  // past the end: the last key (masked)
        const int64_t off = tt < ks.np ? tt * ks.ptok : (tt - ks.np) * ks.btok;
        // read once per launch: non-temporal (measured 5.4 -> 5.7 TB/s at decode256)
        kr[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>((tt < ks.np ? ks.prefix : ks.block) + off + ch * 8));
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>((tt < ks.np ? vprefix : vblock) + off + ch * 8));
    }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefix_attn_mfma_kernel(PrefixArgs a)
{
    using C = SaCfg<D>;
    constexpr int CH = D / 8;
    // work-group -> (pair, query tile qt: the block's queries 32 qt .. 32 qt + 31, key range sp)
    const int nqt = (a.B + 31) >> 5;
    const int sp = blockIdx.x % a.splits, pq = blockIdx.x / a.splits;
    const int qt = pq % nqt, pair = pq / nqt;
    const int r = pair / a.H, h = pair % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ln = lane & 31, g = lane >> 5;

    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
    uint16_t* const Vt = reinterpret_cast<uint16_t*>(smem) + wv * C::TILE;
    uint16_t* const Kt = reinterpret_cast<uint16_t*>(smem) + (4 + wv) * C::TILE;

    int64_t s0 = a.seq_offsets[r], s1 = a.seq_offsets[r + 1];
    s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
    s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
    KeySource ks;
    const int64_t hoff = static_cast<int64_t>(h) * a.ps.head;
    const int64_t boff = static_cast<int64_t>(r) * a.qs.req + static_cast<int64_t>(h) * a.qs.head;
    ks.prefix = static_cast<const uint16_t*>(a.kp) + s0 * a.ps.tok + hoff;
    ks.block = static_cast<const uint16_t*>(a.k) + boff;
    ks.ptok = a.ps.tok;
    ks.btok = a.qs.tok;
    ks.np = static_cast<int>(s1 - s0 < 0x7fffff00 ? s1 - s0 : 0x7fffff00);
    ks.nk = ks.np + a.B;
    const uint16_t* vprefix = static_cast<const uint16_t*>(a.vp) + s0 * a.ps.tok + hoff;
    const uint16_t* vblock = static_cast<const uint16_t*>(a.v) + boff;
    // this work-group's chunks: [c_lo, c_hi) of the pair's 32-key chunks
    const int nall = (ks.nk + 31) / 32;
    const int c_lo = static_cast<int>(static_cast<int64_t>(nall) * sp / a.splits);
    const int nch = static_cast<int>(static_cast<int64_t>(nall) * (sp + 1) / a.splits);

    // Q fragments: query ln (rows past B read row B - 1; never stored)
    bf16x8 qf[C::NKB];
    {
        const int qi = 32 * qt + ln < a.B ? 32 * qt + ln : a.B - 1;
        const uint16_t* qr = static_cast<const uint16_t*>(a.q) + boff + qi * a.qs.tok + g * (D / 2);
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) qf[kb] = *reinterpret_cast<const bf16x8*>(qr + 8 * kb);
    }

    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 acc[C::CT];
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) acc[ct] = f32x16{};
    u32x4 kr[C::VQ], vr[C::VQ];
    if (c_lo + wv < nch) sa_load_chunk<D>(ks, c_lo + wv, lane, kr, vr, vprefix, vblock);

    for (int c = c_lo + wv; c < nch; c += 4) {
        // K and V rows of this chunk into the wave's tiles (LDS operations of
        // one wave execute in order, so no barrier is needed)
#pragma unroll
        for (int i = 0; i < C::VQ; ++i) {
            const int idx = lane + 64 * i, t = idx / CH, ch = idx % CH;
            *reinterpret_cast<u32x4*>(Kt + t * D + 8 * k_chunk_pos<D>(t, ch)) = kr[i];
            *reinterpret_cast<u32x4*>(Vt + t * D + (((2 * ch) ^ lds_piece_swizzle<D / 4>(t)) << 2)) = vr[i];
        }
        // s^T = K Q^T: lane (ln, g) feeds key row ln, elements g d/2 + 8 kb .. + 7
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
            sacc = mfma32(lds_frag(Kt + ln * D + 8 * k_chunk_pos<D>(ln, g * (CH / 2) + kb)), qf[kb], sacc);
        if (c + 4 < nch) sa_load_chunk<D>(ks, c + 4, lane, kr, vr, vprefix, vblock);

        // online softmax of query ln over the chunk's keys 8 (v/4) + 4 g + v%4
        float mc = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int j = 32 * c + 8 * (v >> 2) + 4 * g + (v & 3);
            const float sv = j < ks.nk ? sacc[v] * a.scale : -INFINITY;
            sacc[v] = sv;
            mc = fmaxf(mc, sv);
        }
        mc = fmaxf(mc, __shfl_xor(mc, 32, 64));
        const float m_new = fmaxf(m_run, mc);
        const float alpha = __expf(m_run - m_new);
        bf16x8 pp[2];
        float ls = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float p = __expf(sacc[v] - m_new);
            ls += p;
            pp[v >> 3][v & 7] = static_cast<__bf16>(p);
        }
        ls += __shfl_xor(ls, 32, 64);
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[ct][v] *= alpha;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) acc[ct] = mfma32(vt_frag_ps<D / 4>(Vt, 32 * ct, kb, lane), pp[kb], acc[ct]);
        __builtin_amdgcn_wave_barrier();
    }

    // merge the four waves: acc as [w][d][query], then m and l per [w][query]
    __syncthreads();
    float* const Ma = reinterpret_cast<float*>(smem);
    float* const Mm = Ma + 4 * D * 32;
    float* const Ml = Mm + 4 * 32;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int dcol = 32 * ct + 8 * (v >> 2) + 4 * g + (v & 3);
            Ma[(wv * D + dcol) * 32 + ln] = acc[ct][v];
        }
    if (g == 0) {
        Mm[wv * 32 + ln] = m_run;
        Ml[wv * 32 + ln] = l_run;
    }
    __syncthreads();
    // thread -> (query, 8 columns), 16-byte row stores
    for (int idx = tid; idx < 32 * CH; idx += 256) {
        const int qi = idx / CH, c8 = (idx % CH) * 8;  // row qi of the query tile
        if (32 * qt + qi >= a.B) continue;
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = Mm[w * 32 + qi];
            M = fmaxf(M, mw[w]);
        }
        float den = 0.0f, sc[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // a wave (or, split, the whole work-group) with no keys: weight 0
            sc[w] = mw[w] == -INFINITY ? 0.0f : __expf(mw[w] - M);
            den += sc[w] * Ml[w * 32 + qi];
        }
        if (a.splits > 1) {
            float* rec = a.part + (static_cast<int64_t>(pq) * a.splits + sp) * prefix_part_floats(D);
            f32x4 nv[2];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float num = 0.0f;
#pragma unroll
                for (int w = 0; w < 4; ++w) num += sc[w] * Ma[(w * D + c8 + e) * 32 + qi];
                nv[e >> 2][e & 3] = num;
            }
            *reinterpret_cast<f32x4*>(rec + qi * D + c8) = nv[0];
            *reinterpret_cast<f32x4*>(rec + qi * D + c8 + 4) = nv[1];
            if (c8 == 0) {
                rec[32 * D + qi] = M;
                rec[32 * D + 32 + qi] = den;
            }
            continue;
        }
        const float inv = 1.0f / den;
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float y[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int dcol = c8 + 2 * e + u;
                float num = 0.0f;
#pragma unroll
                for (int w = 0; w < 4; ++w) num += sc[w] * Ma[(w * D + dcol) * 32 + qi];
                y[u] = num * inv;
            }
            pk[e] = static_cast<uint32_t>(bf16_bits(y[0])) | (static_cast<uint32_t>(bf16_bits(y[1])) << 16);
        }
        uint16_t* orow = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(r) * a.os.req +
                         static_cast<int64_t>(h) * a.os.head + static_cast<int64_t>(32 * qt + qi) * a.os.tok + c8;
        *reinterpret_cast<u32x4*>(orow) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    }
}

// Merge of the split partial results, one work-group per (request, head,
// query): y = sum_s e^{M_s - M} num_s / sum_s e^{M_s - M} l_s, M = max_s M_s.
// Wave 0 turns the splits' maxima and normalisers into weights; then thread
// (g, c) sums column quad c over the splits g, g + G, ... (all of its loads
// issued together) and the G partial sums of each quad are added through LDS.
constexpr int kSplitMax = 64;

template <typename T, int D>
__global__ __launch_bounds__(256) void prefix_attn_merge_kernel(PrefixArgs a)
{
    constexpr int NQ = D / 4, G = 256 / NQ, PER = kSplitMax / G;
    const int pair = blockIdx.x / a.B, q = blockIdx.x % a.B;
    const int qi = q & 31, pq = pair * ((a.B + 31) >> 5) + (q >> 5);  // row in its query tile; (pair, tile)
    const int r = pair / a.H, h = pair % a.H;
    const int tid = threadIdx.x, cq = tid % NQ, g = tid / NQ;
    constexpr int64_t pf = 32 * D + 64;
    const float* base = a.part + static_cast<int64_t>(pq) * a.splits * pf;
    __shared__ float wsh[kSplitMax];
    __shared__ f32x4 part[256];
    if (tid < 64) {
        const int sc = tid < a.splits ? tid : a.splits - 1;
        const float m = tid < a.splits ? base[sc * pf + 32 * D + qi] : -INFINITY;
        const float l = base[sc * pf + 32 * D + 32 + qi];
        const float M = wave_max(m);
        const float w = m == -INFINITY ? 0.0f : expf(m - M);
        const float den = wave_sum(w * l);
        wsh[tid] = w / den;  // zero past the last split
    }
    __syncthreads();
    f32x4 acc = f32x4{};
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int sp = g + G * i;
        const int sc = sp < a.splits ? sp : a.splits - 1;
        const f32x4 x = *reinterpret_cast<const f32x4*>(base + sc * pf + qi * D + 4 * cq);
        acc += wsh[sp] * x;
    }
    part[tid] = acc;
    __syncthreads();
    if (tid < NQ) {
        f32x4 y = part[tid];
#pragma unroll
        for (int j = 1; j < G; ++j) y += part[j * NQ + tid];
        T* orow = static_cast<T*>(a.out) + static_cast<int64_t>(r) * a.os.req + static_cast<int64_t>(h) * a.os.head +
                  static_cast<int64_t>(q) * a.os.tok + 4 * tid;
        if constexpr (sizeof(T) == 2) {
            const uint32_t lo =
                static_cast<uint32_t>(bf16_bits(y[0])) | (static_cast<uint32_t>(bf16_bits(y[1])) << 16);
            const uint32_t hi =
                static_cast<uint32_t>(bf16_bits(y[2])) | (static_cast<uint32_t>(bf16_bits(y[3])) << 16);
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            *reinterpret_cast<u32x2*>(orow) = u32x2{lo, hi};
        } else {
            *reinterpret_cast<f32x4*>(orow) = y;
        }
    }
}

// fp32 path, for float32 I/O and the bf16 shapes the kernel above does not
// take: the same work-group layout (four waves per (request, head, query
// tile, key range), each wave its own 32-key chunks, online softmax, merge at
// the end), on the fp32 matrix cores (v_mfma_f32_32x32x2_f32: fp32 products
// and sums) with accurate expf. Per chunk: s^T = K Q^T (lane = query; K rows
// loaded straight from memory, Q from LDS; k taken in runs of four per lane),
// then out^T += V^T P^T with P straight from the score accumulators (element v
// of a lane is the key 8 (v/4) + 4 (lane/32) + v%4 of its k order). Output
// column tile ct of lane j holds column CT j + ct, so each V row is one
// contiguous CT-float load per lane. The four waves' results are scaled to a
// common maximum and added into one LDS tile in a fixed order.
template <typename T>
__device__ __forceinline__ f32x4 sa_ld4(const T* p);
template <>
__device__ __forceinline__ f32x4 sa_ld4<float>(const float* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
template <>
__device__ __forceinline__ f32x4 sa_ld4<uint16_t>(const uint16_t* p)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
                 __uint_as_float(u[1] & 0xffff0000u)};
}

template <typename T, int N>
__device__ __forceinline__ void sa_ldn(const T* p, float (&x)[N])
{
    if constexpr (N == 4) {
        const f32x4 y = sa_ld4<T>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = y[i];
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = ld_elem(p, i);
    }
}

__device__ __forceinline__ f32x16 mfma32f(float x, float y, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, c, 0, 0, 0);
}

// Three waves per SIMD (160 VGPRs, no spills): 6.02 -> 4.97 ms on a batch of
// 256 requests x 16 heads over 1.02 M prefix tokens, against two by default.
template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void prefix_attn_f32_kernel(
    PrefixArgs a)
{
    constexpr int CT = D / 32;   // output column tiles per wave
    constexpr int QS = D + 4;    // LDS row stride of the query tile and the merged output (floats)
    const int nqt = (a.B + 31) >> 5;
    const int sp = blockIdx.x % a.splits, pq = blockIdx.x / a.splits;
    const int qt = pq % nqt, pair = pq / nqt;
    const int r = pair / a.H, h = pair % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ln = lane & 31, g = lane >> 5;

    __shared__ __attribute__((aligned(16))) float Qs[32 * QS];  // the query tile, then the merged output
    __shared__ float Mm[4 * 32], Ml[4 * 32], Mx[32], Dn[32];

    int64_t s0 = a.seq_offsets[r], s1 = a.seq_offsets[r + 1];
    s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
    s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
    const int64_t np = s1 - s0, nk = np + a.B;
    const int64_t hoff = static_cast<int64_t>(h) * a.ps.head;
    const int64_t boff = static_cast<int64_t>(r) * a.qs.req + static_cast<int64_t>(h) * a.qs.head;
    const T* kp = static_cast<const T*>(a.kp) + s0 * a.ps.tok + hoff;
    const T* vp = static_cast<const T*>(a.vp) + s0 * a.ps.tok + hoff;
    const T* kb = static_cast<const T*>(a.k) + boff;
    const T* vb = static_cast<const T*>(a.v) + boff;
    // this work-group's chunks: [c_lo, c_hi) of the pair's 32-key chunks
    const int64_t nall = (nk + 31) / 32;
    const int64_t c_lo = nall * sp / a.splits, c_hi = nall * (sp + 1) / a.splits;

    // query rows past B read row B - 1 (never stored)
    for (int idx = tid; idx < 32 * D / 4; idx += 256) {
        const int qi = idx / (D / 4), c4 = idx % (D / 4);
        const int qr = 32 * qt + qi < a.B ? 32 * qt + qi : a.B - 1;
        *reinterpret_cast<f32x4*>(Qs + qi * QS + 4 * c4) =
            sa_ld4<T>(static_cast<const T*>(a.q) + boff + static_cast<int64_t>(qr) * a.qs.tok + 4 * c4);
    }
    __syncthreads();

    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x16{};
    for (int64_t c = c_lo + wv; c < c_hi; c += 4) {
        // key row of lane ln (past the end: the last key, masked)
        int64_t t = 32 * c + ln;
        t = t < nk ? t : nk - 1;
        const T* krow = t < np ? kp + t * a.ps.tok : kb + (t - np) * a.qs.tok;
        f32x16 sacc = f32x16{};
#pragma unroll 4
        for (int gi = 0; gi < D / 8; ++gi) {
            const int k0 = 8 * gi + 4 * g;
            const f32x4 x = sa_ld4<T>(krow + k0);
            const f32x4 y = *reinterpret_cast<const f32x4*>(Qs + ln * QS + k0);
            sacc = mfma32f(x[0], y[0], sacc);
            sacc = mfma32f(x[1], y[1], sacc);
            sacc = mfma32f(x[2], y[2], sacc);
            sacc = mfma32f(x[3], y[3], sacc);
        }
        // online softmax of query ln over the chunk's keys 8 (v/4) + 4 g + v%4
        float mc = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t j = 32 * c + 8 * (v >> 2) + 4 * g + (v & 3);
            const float sv = j < nk ? sacc[v] * a.scale : -INFINITY;
            sacc[v] = sv;
            mc = fmaxf(mc, sv);
        }
        mc = fmaxf(mc, __shfl_xor(mc, 32, 64));
        const float m_new = fmaxf(m_run, mc);  // finite: the chunk has a key
        const float alpha = expf(m_run - m_new);
        float ls = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            sacc[v] = expf(sacc[v] - m_new);
            ls += sacc[v];
        }
        ls += __shfl_xor(ls, 32, 64);
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[ct][v] *= alpha;
        // out^T += V^T P^T: lane (ln, g) gives V[key][CT ln + ct] for the
        // keys 8 b + 4 g + z of its k order
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                int64_t tv = 32 * c + 8 * b + 4 * g + z;
                tv = tv < nk ? tv : nk - 1;  // weight 0
                float vv[CT];
                sa_ldn<T, CT>((tv < np ? vp + tv * a.ps.tok : vb + (tv - np) * a.qs.tok) + CT * ln, vv);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[ct] = mfma32f(vv[ct], sacc[4 * b + z], acc[ct]);
            }
    }

    // merge the four waves: each scales its rows to the common maximum, then
    // they add into Qs (now the output tile [query][column]) in wave order
    if (g == 0) {
        Mm[wv * 32 + ln] = m_run;
        Ml[wv * 32 + ln] = l_run;
    }
    __syncthreads();  // also: every wave is done with the query tile
    {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, Mm[w * 32 + ln]);
        float den = 0.0f, mine = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // a wave (or, split, the whole work-group) with no keys: weight 0
            const float mw = Mm[w * 32 + ln];
            const float sc = mw == -INFINITY ? 0.0f : expf(mw - M);
            den += sc * Ml[w * 32 + ln];
            if (w == wv) mine = sc;
        }
        if (wv == 0 && g == 0) {
            Mx[ln] = M;
            Dn[ln] = den;
        }
        for (int w = 0; w < 4; ++w) {
            if (w == wv) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        float* o = Qs + ln * QS + CT * (8 * (v >> 2) + 4 * g + (v & 3)) + ct;
                        *o = (w == 0 ? 0.0f : *o) + mine * acc[ct][v];
                    }
            }
            __syncthreads();
        }
    }
    // rows of the merged tile: thread -> (query, four columns)
    for (int idx = tid; idx < 32 * D / 4; idx += 256) {
        const int qi = idx / (D / 4), c4 = idx % (D / 4);
        if (32 * qt + qi >= a.B) continue;
        const f32x4 num = *reinterpret_cast<const f32x4*>(Qs + qi * QS + 4 * c4);
        if (a.splits > 1) {
            float* rec = a.part + (static_cast<int64_t>(pq) * a.splits + sp) * prefix_part_floats(D);
            *reinterpret_cast<f32x4*>(rec + qi * D + 4 * c4) = num;
            if (c4 == 0) {
                rec[32 * D + qi] = Mx[qi];
                rec[32 * D + 32 + qi] = Dn[qi];
            }
            continue;
        }
        const float inv = 1.0f / Dn[qi];
        T* orow = static_cast<T*>(a.out) + static_cast<int64_t>(r) * a.os.req + static_cast<int64_t>(h) * a.os.head +
                  static_cast<int64_t>(32 * qt + qi) * a.os.tok + 4 * c4;
#pragma unroll
        for (int e = 0; e < 4; ++e) st_elem(orow, e, num[e] * inv);
    }
}

// Work-groups the split aims for (one per CU of 256: measured faster than two,
// fewer and longer splits spend less on each work-group's first loads and its
// final merge), and the fewest 32-key chunks a split should hold so that its
// partial record (about 16 KiB) stays small beside the keys and values it
// reads (16 chunks: 256 KiB).
constexpr int64_t kSplitTargetWgs = 256;
constexpr int64_t kSplitMinChunks = 16;

}  // namespace

// ---------------------------------------------------------------------------
// Allocation-free split partials (bha_prefix_attention_noalloc)
// ---------------------------------------------------------------------------
// For callers that cannot allocate, the split's partial records go to this
// static buffer instead of a caller workspace. Its size covers the largest
// split prefix_attention_splits picks: a split happens only for fewer than
// kSplitTargetWgs (request, head, query tile) units, each split at most
// ceil(kSplitTargetWgs / units) ways, so at most 2 kSplitTargetWgs - 2 = 510
// records of prefix_part_floats(128) floats (16,640 bytes): 8,486,400 bytes.
// Each GPU the library runs on holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static_assert((2 * kSplitTargetWgs - 2) * 4 * (32 * 128 + 64) <= kNoAllocScratchBytes,
              "the largest split fits the static buffer");

// This device's address of `scratch`, looked up with hipGetSymbolAddress on
// the first call on each device (with that device current) and kept; in host
// code the array's own name is not a device address.
hipError_t noalloc_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static void* addr[kMaxDevices];
    static hipError_t err[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev] { err[dev] = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch)); });
    if (err[dev] != hipSuccess) return err[dev];
    *ptr = addr[dev];
    return hipSuccess;
}

int prefix_query_tiles(int B) { return (B + 31) / 32; }

int prefix_attention_splits(int R, int H, int d, int B, int io, int64_t total_tokens)
{
    if (B > 64 || (d != 64 && d != 128) || R <= 0) return 1;
    const int64_t pairs = static_cast<int64_t>(R) * H * prefix_query_tiles(B);
    const int64_t avg_chunks = (total_tokens / R + B + 31) / 32;
    int64_t sp = (kSplitTargetWgs + pairs - 1) / pairs;
    sp = sp < avg_chunks / kSplitMinChunks ? sp : avg_chunks / kSplitMinChunks;
    sp = sp < kSplitMax ? sp : static_cast<int64_t>(kSplitMax);
    return sp < 2 ? 1 : static_cast<int>(sp);
}

bool prefix_attention_mfma_supported(const PrefixArgs& a)
{
    // per-lane offsets within a block and a chunk are 32-bit
    return a.io == BHA_BF16 && a.B >= 1 && a.B <= 64 && (a.d == 64 || a.d == 128) && a.qs.tok >= 0 &&
           a.qs.tok < (int64_t(1) << 25) && a.ps.tok >= 0 && a.ps.tok < (int64_t(1) << 25);
}

hipError_t launch_prefix_attention_mfma(const PrefixArgs& a, hipStream_t s)
{
    if (a.splits < 1 || a.splits > kSplitMax || (a.splits > 1 && !a.part)) return hipErrorInvalidValue;
    const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.R) * a.H * prefix_query_tiles(a.B) * a.splits)),
        block(256);
    hipError_t e = a.d == 128 ? launch_kernel(prefix_attn_mfma_kernel<128>, grid, block, s, a)
                              : launch_kernel(prefix_attn_mfma_kernel<64>, grid, block, s, a);
    if (e != hipSuccess || a.splits == 1) return e;
    const dim3 mgrid(static_cast<uint32_t>(static_cast<int64_t>(a.R) * a.H * a.B));
    return a.d == 128 ? launch_kernel(prefix_attn_merge_kernel<uint16_t, 128>, mgrid, dim3(256), s, a)
                      : launch_kernel(prefix_attn_merge_kernel<uint16_t, 64>, mgrid, dim3(256), s, a);
}

template <typename T, int D>
static hipError_t prefix_f32_launch(const PrefixArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.R) * a.H * prefix_query_tiles(a.B) * a.splits));
    const hipError_t e = launch_kernel(prefix_attn_f32_kernel<T, D>, grid, dim3(256), s, a);
    if (e != hipSuccess || a.splits == 1) return e;
    const dim3 mgrid(static_cast<uint32_t>(static_cast<int64_t>(a.R) * a.H * a.B));
    return launch_kernel(prefix_attn_merge_kernel<T, D>, mgrid, dim3(256), s, a);
}

hipError_t launch_prefix_attention_generic(const PrefixArgs& a, hipStream_t s)
{
    if (a.splits < 1 || a.splits > kSplitMax || (a.splits > 1 && !a.part)) return hipErrorInvalidValue;
    if (a.io == BHA_BF16) return a.d == 128 ? prefix_f32_launch<uint16_t, 128>(a, s) : prefix_f32_launch<uint16_t, 64>(a, s);
    return a.d == 128 ? prefix_f32_launch<float, 128>(a, s) : prefix_f32_launch<float, 64>(a, s);
}

}  // namespace bha
