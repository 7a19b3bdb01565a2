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

// Stage rows [0, 32) x d of a bf16 token tensor into LDS (row stride RS),
// zero-filling rows >= nrows.
template <int D, int NT, int RS>
__device__ __forceinline__ void stage_rows(uint16_t* dst, const uint16_t* src, int64_t tok, int nrows, int tid)
{
    constexpr int CH = D / 8;
    for (int idx = tid; idx < 32 * CH; idx += NT) {
        const int t = idx / CH, ch = idx % CH;
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (t < nrows) x = *reinterpret_cast<const uint4*>(src + t * tok + ch * 8);
        *reinterpret_cast<uint4*>(dst + t * RS + ch * 8) = x;
    }
}

// Stage V transposed: Vt[c][t] (row stride VS), zero for t >= nrows.
template <int D, int NT, int VS>
__device__ __forceinline__ void stage_vt(uint16_t* dst, const uint16_t* src, int64_t tok, int nrows, int tid)
{
    constexpr int CH = D / 8;
    for (int idx = tid; idx < 32 * CH; idx += NT) {
        const int t = idx / CH, ch = idx % CH;
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (t < nrows) x = *reinterpret_cast<const uint4*>(src + t * tok + ch * 8);
        const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dst[(ch * 8 + 2 * e) * VS + t] = static_cast<uint16_t>(w4[e] & 0xFFFFu);
            dst[(ch * 8 + 2 * e + 1) * VS + t] = static_cast<uint16_t>(w4[e] >> 16);
        }
    }
}

// Stage W (FW rows of d bf16) into LDS.
template <int D, int FW, int NT, int RS>
__device__ __forceinline__ void stage_w(uint16_t* dst, const uint16_t* src, int tid)
{
    constexpr int CH = D / 8;
    for (int idx = tid; idx < FW * CH; idx += NT) {
        const int j = idx / CH, ch = idx % CH;
        *reinterpret_cast<uint4*>(dst + j * RS + ch * 8) = *reinterpret_cast<const uint4*>(src + j * D + ch * 8);
    }
}

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

// In place: u -> exp(u - max u) * (1/sum) for the first half, and returns in
// en the second half exp(-u - max(-u)) * (1/sum). The FW values of one token
// are split between lanes n and n + 32.
template <int FW>
__device__ __forceinline__ void hedgehog_softmax(f32x16 (&ep)[FW / 32], f32x16 (&en)[FW / 32])
{
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            mx = fmaxf(mx, ep[T][v]);
            mn = fminf(mn, ep[T][v]);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    mn = fminf(mn, __shfl_xor(mn, 32, 64));
    float sp = 0.0f, sn = 0.0f;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float x = ep[T][v];
            const float a = __expf(x - mx);
            const float b = __expf(mn - x);
            ep[T][v] = a;
            en[T][v] = b;
            sp += a;
            sn += b;
        }
    sp += __shfl_xor(sp, 32, 64);
    sn += __shfl_xor(sn, 32, 64);
    const float ip = 1.0f / sp, in = 1.0f / sn;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            ep[T][v] *= ip;
            en[T][v] *= in;
        }
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <int D, int FW>
__global__ __launch_bounds__(64 * (D / 32)) void forward_mfma_kernel(ForwardArgs a)
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

    f32x4 sv[C::NSL];
    load_state_slice(rec + wv * F * 32, lane, sv);

    const int64_t base = static_cast<int64_t>(r) * a.qs.req + static_cast<int64_t>(h) * a.qs.head;
    stage_rows<D, C::NT, C::RS>(Qs, static_cast<const uint16_t*>(a.q) + base, a.qs.tok, B, tid);
    stage_rows<D, C::NT, C::RS>(Ks, static_cast<const uint16_t*>(a.k) + base, a.qs.tok, B, tid);
    stage_vt<D, C::NT, C::VS>(Vt, static_cast<const uint16_t*>(a.v) + base, a.qs.tok, B, tid);
    stage_w<D, FW, C::NT, C::RS>(Ws, static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh, tid);
    for (int f4 = tid; f4 < F / 4; f4 += C::NT)
        reinterpret_cast<f32x4*>(Zs)[f4] = reinterpret_cast<const f32x4*>(rec + D * F)[f4];
    __syncthreads();

    // phi(q) for token ln: both halves, fp32, in accumulator layout
    f32x16 ep[FW / 32], en[FW / 32];
    feature_logits<D, FW, C::RS>(Ws, Qs, ln, g, ep);
    hedgehog_softmax<FW>(ep, en);

    // den = phi(q) . Z
    float den = 0.0f;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int fw = 32 * T + 8 * (v >> 2) + 4 * g + (v & 3);
            den = fmaf(ep[T][v], Zs[fw], den);
            den = fmaf(en[T][v], Zs[FW + fw], den);
        }
    den += __shfl_xor(den, 32, 64);

    // phi(q) as bf16 B operands, one per 16 features
    bf16x8 pb[F / 16];
#pragma unroll
    for (int kb = 0; kb < F / 16; ++kb) {
        const bool neg = 16 * kb >= FW;
        const int fw0 = 16 * kb - (neg ? FW : 0);
        const int T = fw0 / 32, rb = (fw0 % 32) / 16 * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[kb][e] = static_cast<__bf16>(neg ? en[T][rb + e] : ep[T][rb + e]);
    }

    // block logits s^T = K Q^T, masked beyond B, exponentials and row sums
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
        sacc = mfma32(lds_frag(Ks + ln * C::RS + 16 * kb + 8 * g), lds_frag(Qs + ln * C::RS + 16 * kb + 8 * g), sacc);
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int j = 8 * (v >> 2) + 4 * g + (v & 3);
        const float s = j < B ? sacc[v] * a.scale : -INFINITY;
        sacc[v] = s;
        m = fmaxf(m, s);
    }
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    float l = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const float p = __expf(sacc[v] - m);
        sacc[v] = p;
        l += p;
    }
    l += __shfl_xor(l, 32, 64);
    bf16x8 pp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) pp[kb][e] = static_cast<__bf16>(sacc[8 * kb + e]);

    // linear read: lin^T = S^T phi(q)^T over this wave's 32 columns
    f32x16 lacc = f32x16{};
#pragma unroll
    for (int kb = 0; kb < F / 16; ++kb) {
        bf16x8 as;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            as[e] = static_cast<__bf16>(sv[2 * kb][e]);
            as[4 + e] = static_cast<__bf16>(sv[2 * kb + 1][e]);
        }
        lacc = mfma32(as, pb[kb], lacc);
    }

    // within-block numerator: sm^T = V^T P^T over this wave's 32 columns
    f32x16 vacc = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const uint16_t* vr = Vt + (32 * wv + ln) * C::VS + 16 * kb + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
        const uint4 q4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
        vacc = mfma32(__builtin_bit_cast(bf16x8, q4), pp[kb], vacc);
    }

    // merge and store this wave's 32 columns of token ln
    if (ln < B) {
        float al, be;
        merge_weights(a.gamma[h], m, al, be);
        const float inv = 1.0f / (al * l + be * den);
        uint16_t* orow = out + static_cast<int64_t>(ln) * a.os.tok + 32 * wv + 4 * g;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            uint32_t pk[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int v0 = 4 * q4 + 2 * e;
                const float y0 = (al * vacc[v0] + be * lacc[v0]) * inv;
                const float y1 = (al * vacc[v0 + 1] + be * lacc[v0 + 1]) * inv;
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

    f32x4 sv[C::NSL];
    load_state_slice(rec + wv * F * 32, lane, sv);

    const int64_t base = static_cast<int64_t>(r) * a.ks.req + static_cast<int64_t>(h) * a.ks.head;
    stage_rows<D, C::NT, C::RS>(Ks, static_cast<const uint16_t*>(a.k) + base, a.ks.tok, B, tid);
    stage_vt<D, C::NT, C::VS>(Vt, static_cast<const uint16_t*>(a.v) + base, a.ks.tok, B, tid);
    stage_w<D, FW, C::NT, C::RS>(Ws, static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh, tid);
    __syncthreads();

    f32x16 ep[FW / 32], en[FW / 32];
    feature_logits<D, FW, C::RS>(Ws, Ks, ln, g, ep);
    hedgehog_softmax<FW>(ep, en);
    __syncthreads();  // every wave is done reading W before phi(K)^T overwrites it

    // phi(k_t)^T into LDS as fp32 [f][t]; padded tokens contribute zero
    const bool live = ln < B;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int fw = 32 * T + 8 * (v >> 2) + 4 * g + (v & 3);
            Pt[fw * C::PS + ln] = live ? ep[T][v] : 0.0f;
            Pt[(FW + fw) * C::PS + ln] = live ? en[T][v] : 0.0f;
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
