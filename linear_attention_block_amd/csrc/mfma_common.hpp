// Matrix-core (bf16 MFMA, fp32 accumulate) kernels of block-hybrid attention
// for gfx950, used for bf16 I/O with blocks of at most 64 tokens (the forward
// takes a block of 33 to 64 tokens as two 32-token query tiles over 64 keys;
// commits of more than 32 tokens run through the prefill kernel).
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
//
// This header holds what the kernels share: the tile configuration, the
// operand staging, the feature-map and softmax pieces and the merge. Each
// kernel family has a source file of its own (mfma_forward.hip,
// mfma_gqa.hip, mfma_gqa8.hip, mfma_commit.hip, mfma_fused.hip,
// mfma_prefill.hip, mfma_feature_map.hip), because the compiler optimises the
// helpers over every call in a translation unit: adding the eight-head
// grouped kernel beside the one-head forward changed the forward's
// instruction schedule (LDS reads no longer overlapping its first products)
// and slowed it by 3-5 % (77.3 -> 80.1 us at 256 x 16 pairs, 145.7 -> 153.7
// us at 512 x 16), with the forward's own source unchanged.
#pragma once

#include "bha_device.hpp"
#include "bha_internal.hpp"
#include "bha_mfma.hpp"

namespace bha {

namespace {

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
    // resident waves per SIMD the persistent forward is compiled for (at
    // d = 128, with four-wave work-groups, also work-groups per CU): its
    // register budget (state slice + one pair's working set) allows two,
    // except with F = 256 whose state slice alone takes 128 registers
    static constexpr int WPE = FW >= 128 ? 1 : 2;
};

// Resident waves per SIMD the forward with KT key (and query) tiles is
// compiled for (work-groups per CU at d = 128; the launcher sizes the grid
// from it). At two the query tiles are kept apart by a scheduling barrier,
// so a tile's working set does not overlap the next one's; the second key
// tile's scores and operands do not fit two work-groups' registers at
// FW >= 64 (measured: one work-group per CU, no spills, is as fast as two
// with spills).
// Two query tiles at FW = 64: the next pair's Q, K and V (64 rows each) held
// in registers across the pair leave room for one work-group per CU; loading
// each pair's operands at its start instead (only the state slice runs a
// pair ahead) fits two, the second covering the first's wait. Measured at
// 256 x 16 pairs, d = 128: 120.9 -> 113.9 us at B = 48, 125.6 -> 121.1 us at
// B = 64.
constexpr bool kFwdTwoTileSync = true;

template <int D, int FW, int KT>
constexpr bool fwd_sync_operands()
{
    return kFwdTwoTileSync && KT == 2 && FW == 64;
}

template <int D, int FW, int KT>
constexpr int fwd_wpe()
{
    return KT > 1 && FW >= 64 && !fwd_sync_operands<D, FW, KT>() ? 1 : Cfg<D, FW>::WPE;
}

// Issue the 128-bit loads of wave w's slice of the S tiles: load t gives lane
// (n, g) = (lane % 32, lane / 32) the features 8t + 4g .. 8t + 4g + 3 of
// column 32w + n.
template <int NSL>
__device__ __forceinline__ void load_state_slice(const float* rec_slice, int lane, f32x4 (&sv)[NSL], int live = 1)
{
    const f32x4* p = reinterpret_cast<const f32x4*>(rec_slice) + lane * live;
#pragma unroll
    for (int t = 0; t < NSL; ++t) sv[t] = __builtin_nontemporal_load(p + t * 64 * live);
}

// A thread's share of the 16-byte chunks of a ROWS x D bf16 token block,
// held in registers between the global loads and the LDS writes so that all
// global loads of a work-group can be issued back to back.
template <int D, int NT, int ROWS = 32>
struct RowChunks {
    static constexpr int CH = D / 8;
    static constexpr int N = ROWS * CH / NT;
    u32x4 v[N];

    // tok: token stride in elements; the launcher guarantees ROWS * tok fits
    // in 31 bits. Rows >= nrows read row nrows - 1 (always present): callers
    // give those rows zero weight. Nothing touches the registers until they
    // are stored, so the loads stay in flight until then.
    // live = 0 points every lane at src itself (a placeholder load of one
    // 16-byte location, for loops that keep their load sequence fixed).
    // The rows are read once per launch: non-temporal loads (measured: the
    // forward 84.0 -> 80.7 us at decode256).
    __device__ __forceinline__ void load(const uint16_t* src, int tok, int nrows, int tid, int live = 1)
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, t = idx / CH, ch = idx % CH;
            const int tr = t < nrows ? t : nrows - 1;
            v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (tr * tok + ch * 8) * live));
        }
    }
    // ROWS / RPH heads of RPH rows each, head j at src + j * head
    template <int RPH>
    __device__ __forceinline__ void load_heads(const uint16_t* src, int tok, int64_t head, int nrows, int tid,
                                               int live = 1)
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, t = idx / CH, ch = idx % CH;
            const int j = t / RPH, tr = t % RPH < nrows ? t % RPH : nrows - 1;
            v[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(src + j * head * live + (tr * tok + ch * 8) * live));
        }
    }
    // row-major copy, row stride RS
    template <int RS>
    __device__ __forceinline__ void store_rows(uint16_t* dst, int tid) const
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, t = idx / CH, ch = idx % CH;
            *reinterpret_cast<u32x4*>(dst + t * RS + ch * 8) = v[i];
        }
    }
    // transposed copy dst[c][t], row stride VS
    template <int VS>
    __device__ __forceinline__ void store_transposed(uint16_t* dst, int tid) const
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, t = idx / CH, ch = idx % CH;
            const uint32_t w4[4] = {v[i][0], v[i][1], v[i][2], v[i][3]};
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
    u32x4 v[N];

    __device__ __forceinline__ void load(const uint16_t* src, int tid)
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, j = idx / CH, ch = idx % CH;
            v[i] = *reinterpret_cast<const u32x4*>(src + j * D + ch * 8);
        }
    }
    template <int RS>
    __device__ __forceinline__ void store_rows(uint16_t* dst, int tid) const
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT, j = idx / CH, ch = idx % CH;
            *reinterpret_cast<u32x4*>(dst + j * RS + ch * 8) = v[i];
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
// KT 32-token tiles of the block (KT = 2 for 32 < B <= 64); the queries of
// G query heads (head j at rows 32 KT j ..) that share one K/V head.
template <int D, int FW, int KT = 1, int G = 1>
struct alignas(16) FwdLds {
    using C = Cfg<D, FW>;
    uint16_t Qs[32 * KT * G * C::RS];
    uint16_t Ks[32 * KT * C::RS];
    uint16_t Ws[FW * C::RS];
    uint16_t Vs[32 * KT * C::RS];  // V rows, read transposed by ds_read_b64_tr_b16
    float Zs[C::F];
    uint16_t Os[G == 1 ? 32 * (D + 8) : 8];  // a 32-row output tile, padded (one-head kernels)  // the pair's output rows, padded (one-head, one-tile kernel)
};

// The per-pair operands a thread stages through LDS, held in registers from
// their global loads to the LDS writes.
template <int D, int FW, int KT = 1, int G = 1, int NT = Cfg<D, FW>::NT>
struct PairOperands {
    using C = Cfg<D, FW>;
    RowChunks<D, NT, 32 * KT * G> q;
    RowChunks<D, NT, 32 * KT> k, v;
    f32x4 z;
    const float* rec;  // the state record the slice loads read (slot 0's for an out-of-range slot)
    bool valid;        // the slot id is in range

    // Issues the same loads whatever the pair: the loop's memory operations
    // are then a fixed sequence and every wait covers exactly the loads it
    // needs. p: the pair (request, K/V head); slot: its slot id, read one pair
    // ahead by the caller; live = 0 collapses the loads onto one location (no
    // next pair).
    __device__ __forceinline__ void load(const ForwardArgs& a, int p, int slot, int tid, int live = 1)
    {
        const int HK = a.H / G;
        const int r = p / HK, hk = p % HK;
        const int64_t qbase = static_cast<int64_t>(r) * a.qs.req + static_cast<int64_t>(hk) * G * a.qs.head;
        const int64_t kbase = static_cast<int64_t>(r) * a.ks.req + static_cast<int64_t>(hk) * a.ks.head;
        if constexpr (G == 1)
            q.load(static_cast<const uint16_t*>(a.q) + qbase, static_cast<int>(a.qs.tok), a.B, tid, live);
        else
            q.template load_heads<32 * KT>(static_cast<const uint16_t*>(a.q) + qbase, static_cast<int>(a.qs.tok),
                                           a.qs.head, a.B, tid, live);
        const int ktok = static_cast<int>(a.ks.tok);
        k.load(static_cast<const uint16_t*>(a.k) + kbase, ktok, a.B, tid, live);
        v.load(static_cast<const uint16_t*>(a.v) + kbase, ktok, a.B, tid, live);
        valid = slot >= 0 && slot < a.num_slots;
        rec = a.state + (static_cast<int64_t>(valid ? slot : 0) * HK + hk) * static_cast<int64_t>(D + 1) * C::F;
        z = reinterpret_cast<const f32x4*>(rec + D * C::F)[(tid % (C::F / 4)) * live];
    }

    __device__ __forceinline__ void store_to(uint16_t* Qs, uint16_t* Ks, uint16_t* Vs, float* Zs, int tid) const
    {
        q.template store_rows<C::RS>(Qs, tid);
        k.template store_rows<C::RS>(Ks, tid);
        v.template store_rows<C::RS>(Vs, tid);
        if (tid < C::F / 4) reinterpret_cast<f32x4*>(Zs)[tid] = z;
    }
    __device__ __forceinline__ void store(FwdLds<D, FW, KT, G>& sm, int tid) const
    {
        store_to(sm.Qs, sm.Ks, sm.Vs, sm.Zs, tid);
    }
};

// One (request, head) pair once its operands are in LDS and this wave's slice
// of the state is in sv: phi(q), the block softmax, P V, phi(q)^T S and the
// merge, then the store of this wave's 32 output columns.
// phi(q) for token ln as bf16 B operands of unnormalised exponentials
// e+ = exp(u - max u) and e- = exp(min u - u); returns the two normalisers
// sp, sn and den = phi(q)^T Z.
template <int D, int FW>
__device__ __forceinline__ void phi_operands_at(const uint16_t* Ws, const uint16_t* Qrows, const float* Zs, int ln,
                                                int g, bf16x8 (&pb)[Cfg<D, FW>::F / 16], float& sp, float& sn,
                                                float& den)
{
    using C = Cfg<D, FW>;
    f32x16 u[FW / 32];
    feature_logits<D, FW, C::RS>(Ws, Qrows, ln, g, u);
    constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) u[T][v] *= kLog2e;  // base-2 logits
    float mx, mn;
    logit_range<FW>(u, mx, mn);
    float dp = 0.0f, dn = 0.0f;
    sp = 0.0f;
    sn = 0.0f;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int fw0 = 32 * T + 8 * q4 + 4 * g;
            const f32x4 zp = *reinterpret_cast<const f32x4*>(Zs + fw0);
            const f32x4 zn = *reinterpret_cast<const f32x4*>(Zs + FW + fw0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = 4 * q4 + e;
                const float ea = __builtin_amdgcn_exp2f(u[T][v] - mx);
                const float eb = __builtin_amdgcn_exp2f(mn - u[T][v]);
                sp += ea;
                sn += eb;
                dp = fmaf(ea, zp[e], dp);
                dn = fmaf(eb, zn[e], dn);
                pb[2 * T + (v >> 3)][v & 7] = static_cast<__bf16>(ea);
                pb[FW / 16 + 2 * T + (v >> 3)][v & 7] = static_cast<__bf16>(eb);
            }
        }
    sp += __shfl_xor(sp, 32, 64);
    sn += __shfl_xor(sn, 32, 64);
    dp += __shfl_xor(dp, 32, 64);
    dn += __shfl_xor(dn, 32, 64);
    den = dp / sp + dn / sn;
}

template <int D, int FW, int KT, int G>
__device__ __forceinline__ void phi_operands(const FwdLds<D, FW, KT, G>& sm, int q0, int ln, int g,
                                             bf16x8 (&pb)[Cfg<D, FW>::F / 16], float& sp, float& sn, float& den)
{
    phi_operands_at<D, FW>(sm.Ws, sm.Qs + q0 * Cfg<D, FW>::RS, sm.Zs, ln, g, pb, sp, sn, den);
}

// Linear read of this wave's 32 columns: sum_f e_f S_f with the + half
// rescaled by sn/sp, so that phi(q)^T S = result / sn. Consumes the state slice.
template <int D, int FW>
__device__ __forceinline__ f32x16 linear_read(const f32x4 (&sv)[Cfg<D, FW>::NSL], const bf16x8 (&pb)[Cfg<D, FW>::F / 16],
                                              float sp, float sn)
{
    f32x16 lacc = f32x16{};
#pragma unroll
    for (int kb = 0; kb < Cfg<D, FW>::F / 16; ++kb) {
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
    return lacc;
}

// One half of phi(q) for token ln: h = 0 the exponentials of u - max u,
// h = 1 those of min u - u; the bf16 B operands of that half's linear read,
// its normaliser s and its share dz = e . Z_h (the same sums phi_operands_at
// takes over both halves).
template <int D, int FW>
__device__ __forceinline__ void phi_half_operands(const uint16_t* Ws, const uint16_t* Qrows, const float* Zs, int ln,
                                                  int g, int h, bf16x8 (&pb)[FW / 16], float& s, float& dz)
{
    using C = Cfg<D, FW>;
    f32x16 u[FW / 32];
    feature_logits<D, FW, C::RS>(Ws, Qrows, ln, g, u);
    constexpr float kLog2e = 1.4426950408889634f;
    const float sc = h ? -kLog2e : kLog2e;  // base-2 logits of this half's softmax argument
    float mx = -INFINITY;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            u[T][v] *= sc;
            mx = fmaxf(mx, u[T][v]);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    s = 0.0f;
    dz = 0.0f;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 z = *reinterpret_cast<const f32x4*>(Zs + h * FW + 32 * T + 8 * q4 + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = 4 * q4 + e;
                const float ex = __builtin_amdgcn_exp2f(u[T][v] - mx);
                s += ex;
                dz = fmaf(ex, z[e], dz);
                pb[2 * T + (v >> 3)][v & 7] = static_cast<__bf16>(ex);
            }
        }
    s += __shfl_xor(s, 32, 64);
    dz += __shfl_xor(dz, 32, 64);
}

// The linear read over one feature half, accumulated onto lacc: sv holds
// that half of the wave's state slice (features 8t + 4g .. + 3 of load t), pb
// its phi operands.
template <int FW>
__device__ __forceinline__ f32x16 linear_read_half(const f32x4 (&sv)[FW / 8], const bf16x8 (&pb)[FW / 16],
                                                   f32x16 lacc)
{
#pragma unroll
    for (int kb = 0; kb < FW / 16; ++kb) {
        bf16x8 as;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            as[e] = static_cast<__bf16>(sv[2 * kb][e]);
            as[4 + e] = static_cast<__bf16>(sv[2 * kb + 1][e]);
        }
        lacc = mfma32(as, pb[kb], lacc);
    }
    return lacc;
}

// Block logits s^T = K Q^T over the KT key tiles (masked beyond B), row
// maximum m, exponentials P and row sum l for the query in LDS row q0 + ln,
// then this wave's 32 columns of P V. Key 32 kt + 8(v/4) + 4g + v%4 of tile kt
// lands in P operand 2 kt + v/8, element v%8: the k order vt_frag reads V
// rows in.
template <int D, int FW, int KT, int G>
__device__ __forceinline__ f32x16 block_softmax_pv(const ForwardArgs& a, const FwdLds<D, FW, KT, G>& sm, int q0,
                                                   int wv, int ln, int g, float& m, float& l)
{
    using C = Cfg<D, FW>;
    constexpr int QT = KT;
    bf16x8 pp[2 * QT];
    {
        f32x16 sacc[QT];
#pragma unroll
        for (int kt = 0; kt < QT; ++kt) {
            sacc[kt] = f32x16{};
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
                sacc[kt] = mfma32(lds_frag(sm.Ks + (32 * kt + ln) * C::RS + 16 * kb + 8 * g),
                                  lds_frag(sm.Qs + (q0 + ln) * C::RS + 16 * kb + 8 * g), sacc[kt]);
        }
        m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < QT; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = 32 * kt + 8 * (v >> 2) + 4 * g + (v & 3);
                const float s = j < a.B ? sacc[kt][v] * a.scale : -INFINITY;
                sacc[kt][v] = s;
                m = fmaxf(m, s);
            }
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        l = 0.0f;
#pragma unroll
        for (int kt = 0; kt < QT; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = __expf(sacc[kt][v] - m);
                l += p;
                pp[2 * kt + (v >> 3)][v & 7] = static_cast<__bf16>(p);
            }
        l += __shfl_xor(l, 32, 64);
    }
    f32x16 vacc = f32x16{};
    const int lane = 32 * g + ln;
#pragma unroll
    for (int kb = 0; kb < 2 * QT; ++kb) vacc = mfma32(vt_frag<C::RS>(sm.Vs, 32 * wv, kb, lane), pp[kb], vacc);
    return vacc;
}

// Merge of the two branches for token ln and store of this wave's 32 columns.
__device__ __forceinline__ void merge_store(const ForwardArgs& a, const f32x16& vacc, const f32x16& lacc, float gamma,
                                            float m, float l, float den, float sn, int r, int h, int wv, int qi, int g,
                                            bool valid)
{
    if (qi >= a.B) return;
    float al, be;
    merge_weights(gamma, m, al, be);
    // an out-of-range slot stores NaN rows
    const float inv = valid ? __builtin_amdgcn_rcpf(al * l + be * den) : __builtin_nanf("");
    const float bl = be * __builtin_amdgcn_rcpf(sn);
    uint16_t* orow = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(r) * a.os.req +
                     static_cast<int64_t>(h) * a.os.head + (qi * static_cast<int>(a.os.tok) + 32 * wv + 4 * g);
    uint32_t pk[4][2];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int v0 = 4 * q4 + 2 * e;
            const float y0 = (al * vacc[v0] + bl * lacc[v0]) * inv;
            const float y1 = (al * vacc[v0 + 1] + bl * lacc[v0 + 1]) * inv;
            pk[q4][e] = static_cast<uint32_t>(bf16_bits(y0)) | (static_cast<uint32_t>(bf16_bits(y1)) << 16);
        }
    // Lanes n and n + 32 hold the two 8-byte halves of each 16-byte piece q4
    // of row qi (columns 32 wv + 8 q4 ..): one row swap (v_permlane32_swap)
    // per dword gives lane n pieces 0 and 2 and lane n + 32 pieces 1 and 3,
    // so each store instruction writes 32 contiguous bytes per row with
    // 16-byte lane stores (measured: 81.4 -> 78.3 us per forward at decode256
    // against four 8-byte stores per lane). The partner lane has the same row,
    // so both are active together.
    uint16_t* const rbase = orow - 4 * g;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t send = g ? pk[2 * j][e] : pk[2 * j + 1][e];
            const auto sw = __builtin_amdgcn_permlane32_swap(send, send, false, false);
            const uint32_t recv = g ? sw[0] : sw[1];  // the partner lane's send
            w[e] = g ? recv : pk[2 * j][e];
            w[2 + e] = g ? pk[2 * j + 1][e] : recv;
        }
        *reinterpret_cast<u32x4*>(rbase + 8 * (2 * j + g)) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// Merge for token ln of this wave's 32 columns into the output tile Os
// ([32][D + 8] bf16: a lane writes row qi, and the 16-byte pad moves each row
// by four banks, so the 32 rows a write instruction touches spread over the
// banks instead of all landing on the same two: 32-way bank conflicts on the
// unpadded 2D-byte rows); after a barrier the work-group stores whole 2D-byte rows
// with non-temporal stores, so every line reaches memory complete (a wave's
// own columns are half lines). Measured at decode256 size, interleaved: 74.7
// -> 73.9 us per forward (plain stores of the same rows 74.0 us); the
// one-tile, one-head kernel only.
constexpr bool kFwdStagedOut = true;

template <int D>
__device__ __forceinline__ void merge_to_lds(const ForwardArgs& a, const f32x16& vacc, const f32x16& lacc,
                                             float gamma, float m, float l, float den, float sn, int wv, int qi,
                                             int g, bool valid, uint16_t* Os)
{
    if (qi >= a.B) return;
    float al, be;
    merge_weights(gamma, m, al, be);
    const float inv = valid ? __builtin_amdgcn_rcpf(al * l + be * den) : __builtin_nanf("");
    const float bl = be * __builtin_amdgcn_rcpf(sn);
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
        // columns 32 wv + 8 q4 + 4 g .. + 3 of row qi
        *reinterpret_cast<uint2*>(Os + qi * (D + 8) + 32 * wv + 8 * q4 + 4 * g) = make_uint2(pk[0], pk[1]);
    }
}

// The state slices that the commit and the fused step write back are
// non-temporal stores; on large batches at F <= 128 they also carry device
// scope (the NT and SC1 cache-policy bits), which a plain global store
// cannot, so they are buffer stores. Measured against non-temporal global
// stores, d = 128, same bits, alternated runs on three boxes: commit at
// FW = 64, 256 requests x 16 heads 111.0 -> 109.5 us, 512: 215.0 -> 211.3
// us, 1,024: 423.5 -> 413.2 us, 128: even, 64: 31.2 -> 31.9 us (slower);
// FW = 32, 256: even; FW = 128, 256: 217.4 -> 219.3 us, 2,048: 1,682 ->
// 1,754 us (slower); forward + commit at FW = 64, 256: 130.4 -> 125.5 us.
// Device scope without NT was 5 % slower, NT with SC0 no different. So the
// launchers take device scope when F <= 128 and there are at least
// kDevScopePairsPerCu pairs per CU (eight rounds of the two resident work-
// groups). The loads keep NT alone (the forward with its state slices read
// under the other policies measured the same), and so do the forward's
// output rows (with SC1: 76 -> 80 us at 256 requests).
constexpr int kDevScopePairsPerCu = 16;
template <bool DEV>
constexpr int kStorePolicy = DEV ? (2 | 16) : 2;  // NT (SLC), | SC1 (SCC)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_buffer(void* base, uint32_t bytes);

// A raw buffer resource over `bytes` bytes from `base`, which must be the
// same in every lane of the wave (its halves are read from the first lane,
// as unsigned words: sign-extending the low word would corrupt the address).
// Stores at offsets at or past `bytes` are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_buffer(void* base, uint32_t bytes)
{
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v))));
    const uint32_t hi =
        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v >> 32))));
    void* const p = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo));
    // word 3: 32-bit data format, no index stride, no thread-id addressing
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, static_cast<int>(bytes), 0x00020000);
}

// Store t of lane `lane` of a wave's state slice (NSL 16-byte stores per
// lane, 1 KiB per store across the wave, as load_state_slice reads it):
// non-temporal at device scope with DEV (a buffer store), else a
// non-temporal global store (the buffer form of the same policy measured
// 1.5 % slower at F = 256).
template <bool DEV, int NSL>
__device__ __forceinline__ void store_state(const f32x4& x, float* slice, int lane, int t)
{
    if constexpr (DEV) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), wave_buffer(slice, NSL * 1024),
                                               16 * lane + 1024 * t, 0, kStorePolicy<true>);
    } else {
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(slice) + lane + 64 * t);
    }
}

// Rows row0 .. row0 + 31 of the block's output (those below B) from the
// staged tile, 16 bytes per thread per step, whole rows per store
// instruction (non-temporal: full lines).
template <int D, int NT>
__device__ __forceinline__ void store_out_rows(const ForwardArgs& a, const uint16_t* Os, int r, int h, int tid,
                                               int row0 = 0)
{
    constexpr int CH = D / 8;
#pragma unroll
    for (int i = 0; i < 32 * CH / NT; ++i) {
        const int idx = tid + i * NT, ch = idx % CH, row = row0 + idx / CH;
        if (row < a.B) {
            uint16_t* orow = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(r) * a.os.req +
                             static_cast<int64_t>(h) * a.os.head + (row * static_cast<int>(a.os.tok) + 8 * ch);
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(Os + (row - row0) * (D + 8) + 8 * ch),
                                        reinterpret_cast<u32x4*>(orow));
        }
    }
}

// Block logits s^T = K Q^T for the 32 staged queries at Qrows (masked beyond
// B), row maximum m, exponentials P as bf16 B operands and row sum l.
template <int D>
__device__ __forceinline__ void block_softmax_at(const ForwardArgs& a, const uint16_t* Ks, const uint16_t* Qrows,
                                                 int ln, int g, float& m, float& l, bf16x8 (&pp)[2])
{
    constexpr int RS = D + 8;
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
        sacc = mfma32(lds_frag(Ks + ln * RS + 16 * kb + 8 * g), lds_frag(Qrows + ln * RS + 16 * kb + 8 * g), sacc);
    m = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int j = 8 * (v >> 2) + 4 * g + (v & 3);
        const float s = j < a.B ? sacc[v] * a.scale : -INFINITY;
        sacc[v] = s;
        m = fmaxf(m, s);
    }
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    l = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const float pe = __expf(sacc[v] - m);
        l += pe;
        pp[v >> 3][v & 7] = static_cast<__bf16>(pe);
    }
    l += __shfl_xor(l, 32, 64);
}

// Compute units of the current device (cached per device ordinal).
int compute_units()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// The matrix-core kernels address a block's rows with 32-bit offsets.
bool small_token_stride(int64_t tok) { return tok >= 0 && tok < (int64_t(1) << 25); }

bool mfma_sizes(int d, int FW) { return (d == 64 || d == 128) && (FW == 32 || FW == 64 || FW == 128); }

}  // namespace

// Grouped forwards (mfma_gqa.hip: 2 or 4 query heads per K/V head;
// mfma_gqa8.hip: 8 at FW <= 64), dispatched by launch_forward_mfma.
hipError_t launch_forward_gqa_mfma(const ForwardArgs& a, hipStream_t s);
hipError_t launch_forward_gqa8_mfma(const ForwardArgs& a, hipStream_t s);

}  // namespace bha
