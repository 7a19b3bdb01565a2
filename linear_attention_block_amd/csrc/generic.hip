// fp32-arithmetic kernels of block-hybrid attention for gfx950.
//
// They cover every supported size (d in {64,128}, FW in {32,64,128}, B <= 64)
// and both I/O dtypes, with fp32 products and sums throughout (the forward's
// contractions on the fp32 matrix cores, everything else in fp32 vector code
// with accurate expf). They serve float32 I/O (where bf16 matrix-core inputs
// would lose the precision the caller asked for) and the shapes the bf16
// kernels do not tile. The forward and the commit run one work-group per
// (request, head); the feature map one wave per token and head.
#include "bha_device.hpp"
#include "bha_internal.hpp"

namespace bha {

namespace {

constexpr int kThreads = 256;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 32x32 fp32 matrix-core product with two k values per step: lane l gives
// A[l % 32][k = l / 32] and B[k = l / 32][l % 32], and holds D[i][l % 32] for
// i = 8 (v / 4) + 4 (l / 32) + v % 4 in element v. Products and sums are fp32.
__device__ __forceinline__ f32x16 mfma32f(float x, float y, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, c, 0, 0, 0);
}

// Four consecutive elements as floats (16- or 8-byte aligned).
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4(const uint16_t* p)
{
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}

// ---------------------------------------------------------------------------
// Forward: one work-group of four waves per (request, query head), over query
// tiles of 32 rows. With s_ij = scale q_i.k_j, m_i = max_j s_ij,
// p_ij = e^{s_ij - m_i}, l_i = sum_j p_ij and den_i = phi(q_i)^T Z,
//   y_i = (al_i sum_j p_ij v_j + be_i phi(q_i)^T S) / (al_i l_i + be_i den_i)
// (merge_weights), computed as one product Y = P' V + Phi' S with the rows of
// P and phi(Q) scaled by al_i / denominator and be_i / denominator. The three
// products (feature logits U = Q W^T, block logits, Y) run on the fp32 matrix
// cores; the row softmaxes go through LDS, eight threads per row. Operand k
// indices are taken in runs of four per lane (one 16-byte load feeds four
// steps); the state's 32-column panels make its operand loads whole 1 KB rows.
// The record is read once per work-group.
// ---------------------------------------------------------------------------
// Six work-groups per CU where the LDS allows it (FW <= 64: 25.6 KB each, at
// most 80 registers); the state stream of some overlaps the logits and
// softmaxes of others.
template <typename T, int D, int FW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6))) void forward_generic_kernel(ForwardArgs a)
{
    constexpr int F = 2 * FW;
    constexpr int PS = 64 + 4;  // LDS row strides (floats)
    constexpr int FS = F + 4;
    constexpr int US = FS;      // U shares the rows of Phi' (see below)
    constexpr int NU = FW / 32;  // feature-logit column tiles
    constexpr int NQ = FW / 4;   // features per thread in the softmax
    const int pair = blockIdx.x;
    const int h = pair % a.H, r = pair / a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int B = a.B, NK = (B + 31) >> 5;

    __shared__ __attribute__((aligned(16))) float Ps[32 * PS];
    __shared__ __attribute__((aligned(16))) float Phs[32 * FS];
    // U row i lies in Phi' row i: the softmax reads row i of U and then writes
    // row i of Phi' from the eight threads of row i, all of one wave, whose
    // LDS accesses complete in program order
    float* const Us = Phs;

    T* const ob = static_cast<T*>(a.out) + static_cast<int64_t>(r) * a.os.req + static_cast<int64_t>(h) * a.os.head;
    const int slot = a.slot_ids[r];
    if (slot < 0 || slot >= a.num_slots) {
        for (int idx = tid; idx < B * D; idx += kThreads)
            st_elem(ob, static_cast<int64_t>(idx / D) * a.os.tok + idx % D, __builtin_nanf(""));
        return;
    }
    // query head h reads K/V head h / G: its keys, values, W and state
    const int hk = h / a.G, Hk = a.H / a.G;
    const float* rec = a.state + (static_cast<int64_t>(slot) * Hk + hk) * static_cast<int64_t>(D + 1) * F;
    const T* qb = static_cast<const T*>(a.q) + static_cast<int64_t>(r) * a.qs.req + static_cast<int64_t>(h) * a.qs.head;
    const int64_t kvo = static_cast<int64_t>(r) * a.ks.req + static_cast<int64_t>(hk) * a.ks.head;
    const T* kb = static_cast<const T*>(a.k) + kvo;
    const T* vb = static_cast<const T*>(a.v) + kvo;
    const T* W = static_cast<const T*>(a.w) + static_cast<int64_t>(hk) * a.wh;
    const float gam = a.gamma[h];

    for (int i0 = 0; i0 < B; i0 += 32) {
        // U and the block logits, one 32-column tile per wave. Rows past the
        // block are clamped to its last row: computed, never used.
        for (int job = wave; job < NU + NK; job += 4) {
            const bool isu = job < NU;
            const int j0 = 32 * (isu ? job : job - NU);
            const T* arow = qb + static_cast<int64_t>(min(i0 + l32, B - 1)) * a.qs.tok;
            const T* brow = isu ? W + static_cast<int64_t>(j0 + l32) * D
                                : kb + static_cast<int64_t>(min(j0 + l32, B - 1)) * a.ks.tok;
            f32x16 acc = {};
#pragma unroll 4
            for (int g = 0; g < D / 8; ++g) {
                const int k0 = 8 * g + 4 * hf;
                const f32x4 x = ld4(arow + k0), y = ld4(brow + k0);
                acc = mfma32f(x[0], y[0], acc);
                acc = mfma32f(x[1], y[1], acc);
                acc = mfma32f(x[2], y[2], acc);
                acc = mfma32f(x[3], y[3], acc);
            }
            float* dst = isu ? Us + j0 + l32 : Ps + j0 + l32;
            const int ds = isu ? US : PS;
            const float sc = isu ? 1.0f : a.scale;
#pragma unroll
            for (int v = 0; v < 16; ++v) dst[(8 * (v >> 2) + 4 * hf + (v & 3)) * ds] = acc[v] * sc;
        }
        __syncthreads();

        // Row softmaxes: row i = tid / 8; thread p = tid % 8 takes keys p + 8t,
        // and features (sign p / 4, quarter p % 4) of phi.
        {
            const int i = tid >> 3, p = tid & 7, q4 = p & 3, sgn = p >> 2;
            float s[8];
            float m = -INFINITY;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int j = p + 8 * t;
                s[t] = j < B ? Ps[i * PS + j] : -INFINITY;
                m = fmaxf(m, s[t]);
            }
            m = fmaxf(m, __shfl_xor(m, 1, 64));
            m = fmaxf(m, __shfl_xor(m, 2, 64));
            m = fmaxf(m, __shfl_xor(m, 4, 64));
            float l = 0.0f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                s[t] = p + 8 * t < B ? expf(s[t] - m) : 0.0f;
                l += s[t];
            }
            l += __shfl_xor(l, 1, 64);
            l += __shfl_xor(l, 2, 64);
            l += __shfl_xor(l, 4, 64);

            const float sg = sgn ? -1.0f : 1.0f;
            float e[NQ];
            float mu = -INFINITY;
#pragma unroll
            for (int t = 0; t < NQ; t += 4) {
                const f32x4 u4 = *reinterpret_cast<const f32x4*>(Us + i * US + q4 * NQ + t);
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    e[t + z] = sg * u4[z];
                    mu = fmaxf(mu, e[t + z]);
                }
            }
            mu = fmaxf(mu, __shfl_xor(mu, 1, 64));
            mu = fmaxf(mu, __shfl_xor(mu, 2, 64));
            float su = 0.0f;
#pragma unroll
            for (int t = 0; t < NQ; ++t) {
                e[t] = expf(e[t] - mu);
                su += e[t];
            }
            su += __shfl_xor(su, 1, 64);
            su += __shfl_xor(su, 2, 64);
            const float* Z = rec + static_cast<int64_t>(D) * F + sgn * FW + q4 * NQ;
            float dz = 0.0f;
#pragma unroll
            for (int t = 0; t < NQ; t += 4) {
                const f32x4 z4 = ld4(Z + t);
                dz = fmaf(e[t], z4[0], dz);
                dz = fmaf(e[t + 1], z4[1], dz);
                dz = fmaf(e[t + 2], z4[2], dz);
                dz = fmaf(e[t + 3], z4[3], dz);
            }
            dz /= su;
            dz += __shfl_xor(dz, 1, 64);
            dz += __shfl_xor(dz, 2, 64);
            dz += __shfl_xor(dz, 4, 64);

            float al, be;
            merge_weights(gam, m, al, be);
            const float inv = 1.0f / (al * l + be * dz);
            const float ca = al * inv, cb = be * inv / su;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int j = p + 8 * t;
                if (j < 32 * NK) Ps[i * PS + j] = s[t] * ca;
            }
#pragma unroll
            for (int t = 0; t < NQ; t += 4)
                *reinterpret_cast<f32x4*>(Phs + i * FS + sgn * FW + q4 * NQ + t) =
                    f32x4{e[t] * cb, e[t + 1] * cb, e[t + 2] * cb, e[t + 3] * cb};
        }
        __syncthreads();

        // Y = P' V + Phi' S, one 32-column tile per wave.
        for (int ct = wave; ct < D / 32; ct += 4) {
            const int c = 32 * ct + l32;
            f32x16 acc = {};
            for (int g = 0; g < 4 * NK; ++g) {
                const int k0 = 8 * g + 4 * hf;
                const f32x4 x = *reinterpret_cast<const f32x4*>(Ps + l32 * PS + k0);
                float y[4];
#pragma unroll
                for (int z = 0; z < 4; ++z)
                    y[z] = k0 + z < B ? ld_elem(vb, static_cast<int64_t>(k0 + z) * a.ks.tok + c) : 0.0f;
                acc = mfma32f(x[0], y[0], acc);
                acc = mfma32f(x[1], y[1], acc);
                acc = mfma32f(x[2], y[2], acc);
                acc = mfma32f(x[3], y[3], acc);
            }
            // S[f][c] for f = k0 .. k0 + 3 of this column are 16 contiguous
            // bytes; read once: non-temporal (158.7 -> 151.5 us at 256 x 16 pairs)
            const float* sp = rec + static_cast<int64_t>(ct) * (F / 4) * 128 + l32 * 4;
#pragma unroll 4
            for (int g = 0; g < F / 8; ++g) {
                const int k0 = 8 * g + 4 * hf;
                const f32x4 x = *reinterpret_cast<const f32x4*>(Phs + l32 * FS + k0);
                const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + (k0 >> 2) * 128));
                acc = mfma32f(x[0], y[0], acc);
                acc = mfma32f(x[1], y[1], acc);
                acc = mfma32f(x[2], y[2], acc);
                acc = mfma32f(x[3], y[3], acc);
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = i0 + 8 * (v >> 2) + 4 * hf + (v & 3);
                if (i < B) st_elem(ob, static_cast<int64_t>(i) * a.os.tok + c, acc[v]);
            }
        }
        __syncthreads();  // the next tile rewrites Us, Ps and Phs
    }
}

// 16x16 fp32 matrix-core product with four k values per step: lane l gives
// A[l % 16][k = l / 16] and B[k = l / 16][l % 16], and holds
// D[4 (l / 16) + v][l % 16] in element v.
__device__ __forceinline__ f32x4 mfma16f(float x, float y, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c, 0, 0, 0);
}

// Four consecutive elements as loaded (16 bytes of float, 8 of bf16), kept
// raw while the load is in flight and widened when used.
template <typename T>
struct Raw4;
template <>
struct Raw4<float> {
    f32x4 x;
    __device__ __forceinline__ void load(const float* p) { x = *reinterpret_cast<const f32x4*>(p); }
    __device__ __forceinline__ f32x4 f32() const { return x; }
};
template <>
struct Raw4<uint16_t> {
    uint2 x;
    __device__ __forceinline__ void load(const uint16_t* p) { x = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ f32x4 f32() const
    {
        return f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u), __uint_as_float(x.y << 16),
                     __uint_as_float(x.y & 0xffff0000u)};
    }
};

// ---------------------------------------------------------------------------
// Commit and prefill: one work-group of eight waves per (request, head), over
// the request's B block tokens (commit) or its packed token range (prefill),
// 32 tokens at a time. Each wave owns 32x32 tiles of the state (rows f,
// columns c), held in matrix-core accumulators from the first load of the
// record to its single write-back (the record's 32-column panels make both
// whole 1 KB wave accesses; the write-back is non-temporal). Per chunk: its K
// and V rows, loaded into registers during the previous chunk, go to LDS and
// the next chunk's loads are issued; the feature logits U = K W^T on 16x16
// fp32 tiles (W rows from memory, k taken in runs of four per lane, two
// accumulators so consecutive steps do not wait on each other); phi(k) per
// token, 16 threads per token (accurate expf); the Z sums; then
// dS = phi(K)^T V on 32x32 fp32 tiles over the chunk's tokens, the wave's
// tiles interleaved step by step. Rows past the
// range hold copies of the last K row, zero phi and zero V.
// ---------------------------------------------------------------------------
constexpr int kCommitThreads = 512;

template <typename T, int D, int FW>
__global__ __launch_bounds__(kCommitThreads) void commit_generic_kernel(CommitArgs a)
{
    constexpr int F = 2 * FW;
    constexpr int NT = kCommitThreads, NW = NT / 64;
    constexpr int TC = 32;                               // tokens per chunk
    constexpr int US = FW + 4, FS = F + 8, VS = D + 8, KS = D + 4;  // LDS row strides (floats)
    constexpr int LQ = TC * D / 4 / NT;                  // 4-element pieces of K (and V) per thread per chunk
    constexpr int NTILE = (F / 32) * (D / 32);           // 32x32 state tiles
    constexpr int TPW = (NTILE + NW - 1) / NW;           // state tiles per wave
    constexpr int NUT = (TC / 16) * (FW / 16);           // 16x16 logit tiles per chunk
    constexpr int PT = FW / 8;                           // features per thread in the softmax
    const int pair = blockIdx.x;
    const int h = pair % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5, l16 = lane & 15, q = lane >> 4;

    __shared__ __attribute__((aligned(16))) float u[TC * US];
    __shared__ __attribute__((aligned(16))) float ph[TC * FS];
    __shared__ __attribute__((aligned(16))) float xv[TC * VS];
    __shared__ __attribute__((aligned(16))) float xk[TC * KS];
    static_assert(LQ >= 1 && LQ * NT * 4 == TC * D, "whole pieces per thread");
    static_assert(TC * FS >= kPrefillOrderLds, "the ordering scratch fits the phi buffer");
    const int r = prefill_request<NT>(a, pair / a.H, tid, reinterpret_cast<int*>(ph));

    const int slot = a.slot_ids[r];
    if (slot < 0 || slot >= a.num_slots) return;
    int64_t first_row;
    int n;
    commit_rows(a, r, first_row, n);
    if (n == 0) return;
    float* rec = a.state + (static_cast<int64_t>(slot) * a.H + h) * static_cast<int64_t>(D + 1) * F;
    const int64_t base = (first_row < 0 ? static_cast<int64_t>(r) * a.ks.req : first_row * a.ks.tok) +
                         static_cast<int64_t>(h) * a.ks.head;
    const T* kb = static_cast<const T*>(a.k) + base;
    const T* vb = static_cast<const T*>(a.v) + base;
    const T* W = static_cast<const T*>(a.w) + static_cast<int64_t>(h) * a.wh;

    // Element v of tile (ft, ct) is S[32 ft + 8 (v / 4) + 4 hf + v % 4][32 ct + l32]:
    // four consecutive floats of the record per v / 4.
    f32x16 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int ti = wave + NW * i;
        if (ti < NTILE) {
            const int ft = ti / (D / 32), ct = ti % (D / 32);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const f32x4 x = ld4(rec + (static_cast<int64_t>(ct) * (F / 4) + 8 * ft + 2 * b + hf) * 128 + l32 * 4);
#pragma unroll
                for (int z = 0; z < 4; ++z) acc[i][4 * b + z] = x[z];
            }
        } else {
            acc[i] = f32x16{};
        }
    }
    float zacc = 0.0f;

    // piece j of thread tid: row (tid + NT j) / (D / 4), columns 4 ((tid + NT j) % (D / 4)) .. + 3;
    // rows past the range load the last row
    Raw4<T> kr[LQ], vr[LQ];
    auto load_chunk = [&](int tc) {
        const int ntc = n - tc < TC ? n - tc : TC;
#pragma unroll
        for (int j = 0; j < LQ; ++j) {
            const int idx = tid + NT * j, t = idx / (D / 4), c4 = idx % (D / 4);
            const int64_t o = static_cast<int64_t>(tc + (t < ntc ? t : ntc - 1)) * a.ks.tok + 4 * c4;
            kr[j].load(kb + o);
            vr[j].load(vb + o);
        }
    };
    load_chunk(0);

    for (int t0 = 0; t0 < n; t0 += TC) {
        const int nt = n - t0 < TC ? n - t0 : TC;
        __syncthreads();  // the previous chunk's K, phi and V reads are done
#pragma unroll
        for (int j = 0; j < LQ; ++j) {
            const int idx = tid + NT * j, t = idx / (D / 4), c4 = idx % (D / 4);
            *reinterpret_cast<f32x4*>(xk + t * KS + 4 * c4) = kr[j].f32();
            *reinterpret_cast<f32x4*>(xv + t * VS + 4 * c4) = t < nt ? vr[j].f32() : f32x4{};
        }
        if (t0 + TC < n) load_chunk(t0 + TC);
        __syncthreads();
        for (int ut = wave; ut < NUT; ut += NW) {
            const int mt = ut % (TC / 16), jt = ut / (TC / 16);
            const float* krow = xk + (16 * mt + l16) * KS;
            const T* wrow = W + static_cast<int64_t>(16 * jt + l16) * D;
            f32x4 c0 = {}, c1 = {};
#pragma unroll 4
            for (int g = 0; g < D / 16; g += 2) {
                const int k0 = 16 * g + 4 * q;
                const f32x4 x = *reinterpret_cast<const f32x4*>(krow + k0), y = ld4(wrow + k0);
                const f32x4 x1 = *reinterpret_cast<const f32x4*>(krow + k0 + 16), y1 = ld4(wrow + k0 + 16);
                c0 = mfma16f(x[0], y[0], c0);
                c1 = mfma16f(x1[0], y1[0], c1);
                c0 = mfma16f(x[1], y[1], c0);
                c1 = mfma16f(x1[1], y1[1], c1);
                c0 = mfma16f(x[2], y[2], c0);
                c1 = mfma16f(x1[2], y1[2], c1);
                c0 = mfma16f(x[3], y[3], c0);
                c1 = mfma16f(x1[3], y1[3], c1);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) u[(16 * mt + 4 * q + v) * US + 16 * jt + l16] = c0[v] + c1[v];
        }
        __syncthreads();
        {
            // token t = tid / 16; thread p = tid % 16 takes sign p / 8 and the
            // features (p % 8) PT .. + PT - 1 of that half
            const int t = tid >> 4, p = tid & 15, sgn = p >> 3, part = p & 7;
            const float sg = sgn ? -1.0f : 1.0f;
            float e[PT];
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < PT; i += 4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(u + t * US + part * PT + i);
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    e[i + z] = sg * x[z];
                    mx = fmaxf(mx, e[i + z]);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < PT; ++i) {
                e[i] = expf(e[i] - mx);
                sum += e[i];
            }
            sum += __shfl_xor(sum, 1, 64);
            sum += __shfl_xor(sum, 2, 64);
            sum += __shfl_xor(sum, 4, 64);
            const float inv = t < nt ? 1.0f / sum : 0.0f;
#pragma unroll
            for (int i = 0; i < PT; i += 4)
                *reinterpret_cast<f32x4*>(ph + t * FS + sgn * FW + part * PT + i) =
                    f32x4{e[i] * inv, e[i + 1] * inv, e[i + 2] * inv, e[i + 3] * inv};
        }
        __syncthreads();
        if (tid < F)
            for (int t = 0; t < nt; ++t) zacc += ph[t * FS + tid];
#pragma unroll
        for (int g = 0; g < TC / 8; ++g)
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int t = 8 * g + 4 * hf + z;
#pragma unroll
                for (int i = 0; i < TPW; ++i) {
                    const int ti = wave + NW * i;
                    if (ti < NTILE) {
                        const int ft = ti / (D / 32), ct = ti % (D / 32);
                        acc[i] = mfma32f(ph[t * FS + 32 * ft + l32], xv[t * VS + 32 * ct + l32], acc[i]);
                    }
                }
            }
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int ti = wave + NW * i;
        if (ti < NTILE) {
            const int ft = ti / (D / 32), ct = ti % (D / 32);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                __builtin_nontemporal_store(
                    f32x4{acc[i][4 * b], acc[i][4 * b + 1], acc[i][4 * b + 2], acc[i][4 * b + 3]},
                    reinterpret_cast<f32x4*>(rec + (static_cast<int64_t>(ct) * (F / 4) + 8 * ft + 2 * b + hf) * 128 +
                                             l32 * 4));
        }
    }
    if (tid < F) rec[static_cast<int64_t>(D) * F + tid] += zacc;
}

// ---------------------------------------------------------------------------
// Feature map: one wave per (request, token, head).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void feature_map_generic_kernel(PhiArgs a)
{
    const int F = 2 * a.FW;
    const int64_t blk = blockIdx.x;  // ((r * B) + t) * H + h
    const int h = static_cast<int>(blk % a.H);
    const int64_t rt = blk / a.H;
    const int t = static_cast<int>(rt % a.B);
    const int64_t r = rt / a.B;
    const int lane = threadIdx.x;

    __shared__ float xs[128];
    __shared__ float u[128];
    const T* x = static_cast<const T*>(a.x) + r * a.xs.req + static_cast<int64_t>(t) * a.xs.tok +
                 static_cast<int64_t>(h) * a.xs.head;
    const T* W = static_cast<const T*>(a.w) + static_cast<int64_t>(h) * a.wh;
    for (int c = lane; c < a.d; c += 64) xs[c] = ld_elem(x, c);
    __syncthreads();
    for (int j = lane; j < a.FW; j += 64) {
        float s = 0.0f;
        for (int c = 0; c < a.d; ++c) s = fmaf(xs[c], ld_elem(W, static_cast<int64_t>(j) * a.d + c), s);
        u[j] = s;
    }
    __syncthreads();
    float* out = a.phi + blk * F;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const float sg = half == 0 ? 1.0f : -1.0f;
        float mx = -INFINITY;
        for (int j = lane; j < a.FW; j += 64) mx = fmaxf(mx, sg * u[j]);
        mx = wave_max(mx);
        float sum = 0.0f;
        for (int j = lane; j < a.FW; j += 64) sum += expf(sg * u[j] - mx);
        sum = wave_sum(sum);
        for (int j = lane; j < a.FW; j += 64) out[half * a.FW + j] = expf(sg * u[j] - mx) / sum;
    }
}

}  // namespace

template <typename T, int D>
static hipError_t forward_dispatch(const ForwardArgs& a, hipStream_t s, dim3 grid)
{
    switch (a.FW) {
        case 32: return launch_kernel(forward_generic_kernel<T, D, 32>, grid, dim3(kThreads), s, a);
        case 64: return launch_kernel(forward_generic_kernel<T, D, 64>, grid, dim3(kThreads), s, a);
        default: return launch_kernel(forward_generic_kernel<T, D, 128>, grid, dim3(kThreads), s, a);
    }
}

hipError_t launch_forward_generic(const ForwardArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.R) * a.H));
    if (a.io == BHA_BF16)
        return a.d == 128 ? forward_dispatch<uint16_t, 128>(a, s, grid) : forward_dispatch<uint16_t, 64>(a, s, grid);
    return a.d == 128 ? forward_dispatch<float, 128>(a, s, grid) : forward_dispatch<float, 64>(a, s, grid);
}

template <typename T, int D>
static hipError_t commit_dispatch(const CommitArgs& a, hipStream_t s, dim3 grid)
{
    switch (a.FW) {
        case 32: return launch_kernel(commit_generic_kernel<T, D, 32>, grid, dim3(kCommitThreads), s, a);
        case 64: return launch_kernel(commit_generic_kernel<T, D, 64>, grid, dim3(kCommitThreads), s, a);
        default: return launch_kernel(commit_generic_kernel<T, D, 128>, grid, dim3(kCommitThreads), s, a);
    }
}

hipError_t launch_commit_generic(const CommitArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.R) * a.H));
    if (a.io == BHA_BF16)
        return a.d == 128 ? commit_dispatch<uint16_t, 128>(a, s, grid) : commit_dispatch<uint16_t, 64>(a, s, grid);
    return a.d == 128 ? commit_dispatch<float, 128>(a, s, grid) : commit_dispatch<float, 64>(a, s, grid);
}

hipError_t launch_feature_map_generic(const PhiArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.R) * a.B * a.H));
    if (a.io == BHA_BF16) return launch_kernel(feature_map_generic_kernel<uint16_t>, grid, dim3(64), s, a);
    return launch_kernel(feature_map_generic_kernel<float>, grid, dim3(64), s, a);
}

}  // namespace bha
