// Matrix-core (bf16 MFMA, fp32 accumulate) kernels of block-hybrid attention
// for gfx950, used for bf16 I/O with blocks of at most 32 tokens.
//
// One work-group of d/32 waves owns one (request, head) pair; wave w owns the
// 32 value columns [32w, 32w + 32). Every contraction is one
// v_mfma_f32_32x32x16_bf16 tile chain:
//   u^T  = W^T Q^T          (FW x 32)   feature-map logits, lane = token
//   s^T  = K Q^T            (32 x 32)   block logits, lane = query token
//   lin^T = S^T phi(Q)^T    (32 x 32)   per wave: its 32 columns of phi(Q) S
//   sm^T  = V^T P^T         (32 x 32)   per wave: its 32 columns of P V
// The 32x32 accumulator layout puts column n of a tile in lane n % 32 and rows
// 8(v/4) + 4(lane/32) + v%4 in register v. Choosing the order in which each
// lane feeds its eight k-values (any order works if both operands agree) to be
// exactly that row order lets the accumulators of u^T and s^T serve, after the
// softmaxes, directly as the B operands of the next contractions, and lets the
// state tiles (see s_offset) be fed as the A operand straight from 128-bit
// loads, with no LDS round trip for phi, P or S.
//
// The state is the traffic: each wave streams its 16 KiB (F = 128) slice of
// the pair's record with 128-bit loads that are contiguous across the wave
// (1 KiB per instruction), issued before anything else so they overlap the
// staging of Q, K, V and W and the feature-map and softmax arithmetic.
#include "bha_device.hpp"
#include "bha_internal.hpp"

namespace bha {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

template <int D, int FW>
struct Cfg {
    static constexpr int F = 2 * FW;
    static constexpr int NW = D / 32;       // waves per work-group
    static constexpr int NT = 64 * NW;      // threads per work-group
    static constexpr int RS = D + 8;        // padded LDS row (bf16) of Q, K, W
    static constexpr int VS = 32 + 8;       // padded LDS row (bf16) of V^T
    static constexpr int PS = 32 + 4;       // padded LDS row (fp32) of phi(K)^T
    static constexpr int NSL = F / 8;       // 128-bit state loads per lane
    static constexpr int NKB = D / 16;      // k-steps over d
};

// Issue the 128-bit loads of wave w's slice of the S tiles: load t gives lane
// (n, g) = (lane % 32, lane / 32) the features 8t + 4g .. 8t + 4g + 3 of
// column 32w + n.
template <int NSL>
__device__ __forceinline__ void load_state_slice(const float* rec_slice, int lane, f32x4 (&sv)[NSL])
{
    const f32x4* p = reinterpret_cast<const f32x4*>(rec_slice) + lane;
#pragma unroll
    for (int t = 0; t < NSL; ++t) sv[t] = __builtin_nontemporal_load(p + t * 64);
}

// A thread's share of the 16-byte chunks of a 32-row x D bf16 token block,
// held in registers between the global loads and the LDS writes so that all
// global loads of a work-group can be issued back to back. Rows >= nrows are
// zero.
template <int D, int NT>
struct RowChunks {
    static constexpr int CH = D / 8;
    static constexpr int N = 32 * CH / NT;
    uint4 v[N];

    __device__ __forceinline__ void load(const uint16_t* src, int64_t tok, int nrows, int tid)
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, t = idx / CH, ch = idx % CH;
            v[i] = make_uint4(0u, 0u, 0u, 0u);
            if (t < nrows) v[i] = *reinterpret_cast<const uint4*>(src + t * tok + ch * 8);
        }
    }
    // row-major copy, row stride RS
    template <int RS>
    __device__ __forceinline__ void store_rows(uint16_t* dst, int tid) const
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, t = idx / CH, ch = idx % CH;
            *reinterpret_cast<uint4*>(dst + t * RS + ch * 8) = v[i];
        }
    }
    // transposed copy dst[c][t], row stride VS
    template <int VS>
    __device__ __forceinline__ void store_transposed(uint16_t* dst, int tid) const
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, t = idx / CH, ch = idx % CH;
            const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dst[(ch * 8 + 2 * e) * VS + t] = static_cast<uint16_t>(w4[e] & 0xFFFFu);
                dst[(ch * 8 + 2 * e + 1) * VS + t] = static_cast<uint16_t>(w4[e] >> 16);
            }
        }
    }
};

// A thread's share of one head's W (FW rows of D bf16).
template <int D, int FW, int NT>
struct WChunks {
    static constexpr int CH = D / 8;
    static constexpr int N = FW * CH / NT;
    uint4 v[N];

    __device__ __forceinline__ void load(const uint16_t* src, int tid)
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, j = idx / CH, ch = idx % CH;
            v[i] = *reinterpret_cast<const uint4*>(src + j * D + ch * 8);
        }
    }
    template <int RS>
    __device__ __forceinline__ void store_rows(uint16_t* dst, int tid) const
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, j = idx / CH, ch = idx % CH;
            *reinterpret_cast<uint4*>(dst + j * RS + ch * 8) = v[i];
        }
    }
};

// u^T = W^T X^T for the 32 staged token rows X (lane = token).
template <int D, int FW, int RS>
__device__ __forceinline__ void feature_logits(const uint16_t* Ws, const uint16_t* Xs, int ln, int g,
                                               f32x16 (&u)[FW / 32])
{
#pragma unroll
    for (int T = 0; T < FW / 32; ++T) u[T] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
        const bf16x8 bx = lds_frag(Xs + ln * RS + 16 * kb + 8 * g);
#pragma unroll
        for (int T = 0; T < FW / 32; ++T) u[T] = mfma32(lds_frag(Ws + (32 * T + ln) * RS + 16 * kb + 8 * g), bx, u[T]);
    }
}

// Maximum and minimum of one token's FW feature logits, split between lanes
// n and n + 32.
template <int FW>
__device__ __forceinline__ void logit_range(const f32x16 (&u)[FW / 32], float& mx, float& mn)
{
    mx = -INFINITY;
    mn = INFINITY;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            mx = fmaxf(mx, u[T][v]);
            mn = fminf(mn, u[T][v]);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    mn = fminf(mn, __shfl_xor(mn, 32, 64));
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <int D, int FW>
__global__ __launch_bounds__(64 * (D / 32)) __attribute__((amdgpu_waves_per_eu(3, 3))) void forward_mfma_kernel(ForwardArgs a)
{
    using C = Cfg<D, FW>;
    constexpr int F = C::F;
    const int pair = blockIdx.x;
    const int r = pair / a.H, h = pair % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ln = lane & 31, g = lane >> 5;

    __shared__ __attribute__((aligned(16))) uint16_t Qs[32 * C::RS];
    __shared__ __attribute__((aligned(16))) uint16_t Ks[32 * C::RS];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[FW * C::RS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * C::VS];
    __shared__ __attribute__((aligned(16))) float Zs[F];

    const int B = a.B;
    uint16_t* out = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(r) * a.os.req +
                    static_cast<int64_t>(h) * a.os.head;
    const int slot = a.slot_ids[r];
    if (slot < 0 || slot >= a.num_slots) {
        for (int idx = tid; idx < B * D; idx += C::NT)
            out[static_cast<int64_t>(idx / D) * a.os.tok + idx % D] = 0x7FC0u;  // NaN
        return;
    }
    const float* rec = a.state + (static_cast<int64_t>(slot) * a.H + h) * static_cast<int64_t>(D + 1) * F;

    // All global loads first, small operands before the state stream, so that
    // waiting for the operands (the vector-memory counter retires in order)
    // does not wait for the state.
    const int64_t base = static_cast<int64_t>(r) * a.qs.req + static_cast<int64_t>(h) * a.qs.head;
    RowChunks<D, C::NT> qc, kc, vc;
    WChunks<D, FW, C::NT> wc;
    qc.load(static_cast<const uint16_t*>(a.q) + base, a.qs.tok, B, tid);
    kc.load(static_cast<const uint16_t*>(a.k) + base, a.qs.tok, B, tid);
    vc.load(static_cast<const uint16_t*>(a.v) + base, a.qs.tok, B, tid);
    wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh, tid);
    f32x4 zc = f32x4{};
    if (tid < F / 4) zc = reinterpret_cast<const f32x4*>(rec + D * F)[tid];
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sv[C::NSL];
    load_state_slice(rec + wv * F * 32, lane, sv);
    __builtin_amdgcn_sched_barrier(0);
    qc.template store_rows<C::RS>(Qs, tid);
    kc.template store_rows<C::RS>(Ks, tid);
    vc.template store_transposed<C::VS>(Vt, tid);
    wc.template store_rows<C::RS>(Ws, tid);
    if (tid < F / 4) reinterpret_cast<f32x4*>(Zs)[tid] = zc;
    __syncthreads();

    // phi(q) for token ln as bf16 B operands of unnormalised exponentials,
    // e+ = exp(u - max u) and e- = exp(min u - u); the two softmax
    // normalisers sp, sn are applied after the contraction.
    float sp = 0.0f, sn = 0.0f, den = 0.0f;
    bf16x8 pb[F / 16];
    {
        f32x16 u[FW / 32];
        feature_logits<D, FW, C::RS>(Ws, Qs, ln, g, u);
        float mx, mn;
        logit_range<FW>(u, mx, mn);
        float dp = 0.0f, dn = 0.0f;
#pragma unroll
        for (int T = 0; T < FW / 32; ++T)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int fw = 32 * T + 8 * (v >> 2) + 4 * g + (v & 3);
                const float ea = __expf(u[T][v] - mx);
                const float eb = __expf(mn - u[T][v]);
                sp += ea;
                sn += eb;
                dp = fmaf(ea, Zs[fw], dp);
                dn = fmaf(eb, Zs[FW + fw], dn);
                pb[2 * T + (v >> 3)][v & 7] = static_cast<__bf16>(ea);
                pb[FW / 16 + 2 * T + (v >> 3)][v & 7] = static_cast<__bf16>(eb);
            }
        sp += __shfl_xor(sp, 32, 64);
        sn += __shfl_xor(sn, 32, 64);
        dp += __shfl_xor(dp, 32, 64);
        dn += __shfl_xor(dn, 32, 64);
        den = dp / sp + dn / sn;
    }

    // block logits s^T = K Q^T, masked beyond B, exponentials and row sums
    float m = -INFINITY, l = 0.0f;
    bf16x8 pp[2];
    {
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
            sacc = mfma32(lds_frag(Ks + ln * C::RS + 16 * kb + 8 * g), lds_frag(Qs + ln * C::RS + 16 * kb + 8 * g), sacc);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int j = 8 * (v >> 2) + 4 * g + (v & 3);
            const float s = j < B ? sacc[v] * a.scale : -INFINITY;
            sacc[v] = s;
            m = fmaxf(m, s);
        }
        m = fmaxf(m, __shfl_xor(m, 32, 64));
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float p = __expf(sacc[v] - m);
            l += p;
            pp[v >> 3][v & 7] = static_cast<__bf16>(p);
        }
        l += __shfl_xor(l, 32, 64);
    }

    // within-block numerator: sm^T = V^T P^T over this wave's 32 columns
    f32x16 vacc = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const uint16_t* vr = Vt + (32 * wv + ln) * C::VS + 16 * kb + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
        vacc = mfma32(__builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)), pp[kb], vacc);
    }

    // linear read over this wave's 32 columns: lacc = sum_f e_f S_f with the
    // + half rescaled by sn/sp, so that phi(q)^T S = lacc / sn
    f32x16 lacc = f32x16{};
#pragma unroll
    for (int kb = 0; kb < F / 16; ++kb) {
        if (kb == FW / 16) {
            const float rs = sn / sp;
#pragma unroll
            for (int v = 0; v < 16; ++v) lacc[v] *= rs;
        }
        bf16x8 as;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            as[e] = static_cast<__bf16>(sv[2 * kb][e]);
            as[4 + e] = static_cast<__bf16>(sv[2 * kb + 1][e]);
        }
        lacc = mfma32(as, pb[kb], lacc);
    }

    // merge and store this wave's 32 columns of token ln
    if (ln < B) {
        float al, be;
        merge_weights(a.gamma[h], m, al, be);
        const float inv = 1.0f / (al * l + be * den);
        const float bl = be / sn;
        uint16_t* orow = out + static_cast<int64_t>(ln) * a.os.tok + 32 * wv + 4 * g;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            uint32_t pk[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int v0 = 4 * q4 + 2 * e;
                const float y0 = (al * vacc[v0] + bl * lacc[v0]) * inv;
                const float y1 = (al * vacc[v0 + 1] + bl * lacc[v0 + 1]) * inv;
                pk[e] = static_cast<uint32_t>(bf16_bits(y0)) | (static_cast<uint32_t>(bf16_bits(y1)) << 16);
            }
            *reinterpret_cast<uint2*>(orow + 8 * q4) = make_uint2(pk[0], pk[1]);
        }
    }
}

// ---------------------------------------------------------------------------
// Commit
// ---------------------------------------------------------------------------
template <int D, int FW>
__global__ __launch_bounds__(64 * (D / 32)) void commit_mfma_kernel(CommitArgs a)
{
    using C = Cfg<D, FW>;
    constexpr int F = C::F;
    const int pair = blockIdx.x;
    const int r = pair / a.H, h = pair % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ln = lane & 31, g = lane >> 5;

    constexpr int W_BYTES = FW * C::RS * 2;
    constexpr int P_BYTES = F * C::PS * 4;
    constexpr int U_BYTES = W_BYTES > P_BYTES ? W_BYTES : P_BYTES;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[32 * C::RS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * C::VS];
    __shared__ __attribute__((aligned(16))) unsigned char WP[U_BYTES];  // W, then phi(K)^T
    uint16_t* Ws = reinterpret_cast<uint16_t*>(WP);
    float* Pt = reinterpret_cast<float*>(WP);

    const int B = a.B;
    const int slot = a.slot_ids[r];
    if (slot < 0 || slot >= a.num_slots) return;
    float* rec = a.state + (static_cast<int64_t>(slot) * a.H + h) * static_cast<int64_t>(D + 1) * F;

    const int64_t base = static_cast<int64_t>(r) * a.ks.req + static_cast<int64_t>(h) * a.ks.head;
    RowChunks<D, C::NT> kc, vc;
    WChunks<D, FW, C::NT> wc;
    kc.load(static_cast<const uint16_t*>(a.k) + base, a.ks.tok, B, tid);
    vc.load(static_cast<const uint16_t*>(a.v) + base, a.ks.tok, B, tid);
    wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh, tid);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sv[C::NSL];
    load_state_slice(rec + wv * F * 32, lane, sv);
    __builtin_amdgcn_sched_barrier(0);
    kc.template store_rows<C::RS>(Ks, tid);
    vc.template store_transposed<C::VS>(Vt, tid);
    wc.template store_rows<C::RS>(Ws, tid);
    __syncthreads();

    // phi(k_t) for token ln, normalised, fp32
    f32x16 u[FW / 32];
    feature_logits<D, FW, C::RS>(Ws, Ks, ln, g, u);
    float mx, mn;
    logit_range<FW>(u, mx, mn);
    float sp = 0.0f, sn = 0.0f;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            sp += __expf(u[T][v] - mx);
            sn += __expf(mn - u[T][v]);
        }
    sp += __shfl_xor(sp, 32, 64);
    sn += __shfl_xor(sn, 32, 64);
    // padded tokens contribute zero
    const float ip = ln < B ? 1.0f / sp : 0.0f;
    const float in = ln < B ? 1.0f / sn : 0.0f;
    __syncthreads();  // every wave is done reading W before phi(K)^T overwrites it

    // phi(k_t)^T into LDS as fp32 [f][t]
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int fw = 32 * T + 8 * (v >> 2) + 4 * g + (v & 3);
            Pt[fw * C::PS + ln] = __expf(u[T][v] - mx) * ip;
            Pt[(FW + fw) * C::PS + ln] = __expf(mn - u[T][v]) * in;
        }
    __syncthreads();

    // dS = phi(K)^T V: rows f, this wave's 32 columns; fold into the loaded slice
#pragma unroll
    for (int ft = 0; ft < F / 32; ++ft) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const float* pr = Pt + (32 * ft + ln) * C::PS + 16 * kb + 8 * g;
            const f32x4 p0 = *reinterpret_cast<const f32x4*>(pr);
            const f32x4 p1 = *reinterpret_cast<const f32x4*>(pr + 4);
            bf16x8 ap;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ap[e] = static_cast<__bf16>(p0[e]);
                ap[4 + e] = static_cast<__bf16>(p1[e]);
            }
            acc = mfma32(ap, lds_frag(Vt + (32 * wv + ln) * C::VS + 16 * kb + 8 * g), acc);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) sv[4 * ft + (v >> 2)][v & 3] += acc[v];
    }
    f32x4* dst = reinterpret_cast<f32x4*>(rec + wv * F * 32) + lane;
#pragma unroll
    for (int t = 0; t < C::NSL; ++t) __builtin_nontemporal_store(sv[t], dst + t * 64);

    // dZ = sum_t phi(k_t), fp32 from the LDS copy
    for (int f = tid; f < F; f += C::NT) {
        float z = 0.0f;
#pragma unroll
        for (int t = 0; t < 32; ++t) z += Pt[f * C::PS + t];
        rec[D * F + f] += z;
    }
}

template <int D>
static hipError_t forward_by_fw(const ForwardArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(a.R * a.H)), block(64 * (D / 32));
    switch (a.FW) {
        case 32: hipLaunchKernelGGL((forward_mfma_kernel<D, 32>), grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((forward_mfma_kernel<D, 64>), grid, block, 0, s, a); break;
        case 128: hipLaunchKernelGGL((forward_mfma_kernel<D, 128>), grid, block, 0, s, a); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

template <int D>
static hipError_t commit_by_fw(const CommitArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(a.R * a.H)), block(64 * (D / 32));
    switch (a.FW) {
        case 32: hipLaunchKernelGGL((commit_mfma_kernel<D, 32>), grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((commit_mfma_kernel<D, 64>), grid, block, 0, s, a); break;
        case 128: hipLaunchKernelGGL((commit_mfma_kernel<D, 128>), grid, block, 0, s, a); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_mfma(const ForwardArgs& a, hipStream_t s)
{
    if (a.io != BHA_BF16 || a.B > 32) return hipErrorNotSupported;
    if (a.d == 128) return forward_by_fw<128>(a, s);
    if (a.d == 64) return forward_by_fw<64>(a, s);
    return hipErrorNotSupported;
}

hipError_t launch_commit_mfma(const CommitArgs& a, hipStream_t s)
{
    if (a.io != BHA_BF16 || a.B > 32) return hipErrorNotSupported;
    if (a.d == 128) return commit_by_fw<128>(a, s);
    if (a.d == 64) return commit_by_fw<64>(a, s);
    return hipErrorNotSupported;
}

}  // namespace bha
