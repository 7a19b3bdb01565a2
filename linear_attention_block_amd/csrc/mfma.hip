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
// staging of Q, K, V and W and the feature-map and softmax arithmetic.
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
    // resident work-groups per CU the persistent forward is built for: its
    // register budget (state slice + one pair's working set) allows two,
    // except with F = 256 whose state slice alone takes 128 registers
    static constexpr int WPE = FW >= 128 ? 1 : 2;
};

// Resident work-groups per CU of the forward with KT key (and query) tiles.
// At two work-groups the query tiles are kept apart by a scheduling barrier,
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
    uint16_t Os[KT == 1 && G == 1 ? 32 * D : 8];  // the pair's output rows (one-head, one-tile kernel)
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
// ([32][D] bf16); after a barrier the work-group stores whole 2D-byte rows
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
        *reinterpret_cast<uint2*>(Os + qi * D + 32 * wv + 8 * q4 + 4 * g) = make_uint2(pk[0], pk[1]);
    }
}

// The B output rows of the tile, 16 bytes per thread per step, whole rows
// per store instruction (non-temporal: full lines).
template <int D, int NT>
__device__ __forceinline__ void store_out_rows(const ForwardArgs& a, const uint16_t* Os, int r, int h, int tid)
{
    constexpr int CH = D / 8;
#pragma unroll
    for (int i = 0; i < 32 * CH / NT; ++i) {
        const int idx = tid + i * NT, row = idx / CH, ch = idx % CH;
        if (row < a.B) {
            uint16_t* orow = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(r) * a.os.req +
                             static_cast<int64_t>(h) * a.os.head + (row * static_cast<int>(a.os.tok) + 8 * ch);
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(Os + row * D + 8 * ch),
                                        reinterpret_cast<u32x4*>(orow));
        }
    }
}

// Persistent forward: WPE work-groups per compute unit, and work-group b
// takes pairs b, b + NG, b + 2 NG, ... (NG = gridDim.x, a multiple of H, so
// every pair of a work-group has the same head: W_h and the gate are loaded
// once). Per pair: the operands arrive in LDS, then per 32-query tile (KT of
// them: two for 32 < B <= 64) phi(q), the block softmax over all KT key
// tiles and P V run while this wave's state slice streams in and the linear
// read reads it; after the last tile the next pair's slice is issued at once,
// and the merge and stores follow. The next pair's Q, K, V, Z loads are issued
// right after the current ones reach LDS. The vector memory counter retires in
// issue order, so every wait only covers loads issued before the ones still
// streaming.
template <int D, int FW, int KT>
__global__ __launch_bounds__(64 * (D / 32))
__attribute__((amdgpu_waves_per_eu(fwd_wpe<D, FW, KT>(), fwd_wpe<D, FW, KT>()))) void forward_mfma_kernel(
    ForwardArgs a, int npairs)
{
    using C = Cfg<D, FW>;
    constexpr int F = C::F;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ln = lane & 31, g = lane >> 5;
    const int NG = gridDim.x;
    int p = blockIdx.x;
    if (p >= npairs) return;
    const int h = p % a.H;
    const float gamma = a.gamma[h];

    __shared__ FwdLds<D, FW, KT> sm;
    {
        WChunks<D, FW, C::NT> wc;
        wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh, tid);
        wc.template store_rows<C::RS>(sm.Ws, tid);
    }

    // slot ids run one pair ahead of the operand loads (index clamped in range)
    auto slot_of = [&](int pp) { return a.slot_ids[(pp < npairs ? pp : npairs - 1) / a.H]; };
    const int count = (npairs - p + NG - 1) / NG;  // pairs of this work-group
    // SYNC: each pair loads its own operands at its start (no registers held
    // across the pair), and only the state slice runs a pair ahead
    constexpr bool SYNC = fwd_sync_operands<D, FW, KT>();
    auto rec_of = [&](int pp, int sl) {
        const bool ok = sl >= 0 && sl < a.num_slots;
        return a.state + (static_cast<int64_t>(ok ? sl : 0) * a.H + pp % a.H) * static_cast<int64_t>(D + 1) * F;
    };
    PairOperands<D, FW, KT> op;
    f32x4 sv[C::NSL];
    // issue order as in the loop (operands, then the slice, then the next
    // slot id), so the waits at the loop head are the same from either side
    if constexpr (!SYNC) op.load(a, p, slot_of(p), tid);
    __builtin_amdgcn_sched_barrier(0);
    load_state_slice((SYNC ? rec_of(p, slot_of(p)) : op.rec) + wv * F * 32, lane, sv);
    __builtin_amdgcn_sched_barrier(0);
    int slot_cur = slot_of(p);
    int slot_next = slot_of(p + NG);
    for (int k = 0; k < count; ++k) {
        // the last pair issues placeholder loads, so every trip runs the same
        // memory operations
        const int live = k + 1 < count ? 1 : 0;
        const int pn = live ? p + NG : p;
        const int r = p / a.H;
        int slot_after = slot_of(pn + NG);
        __syncthreads();  // every wave is done with the previous pair's LDS operands
        if constexpr (SYNC) op.load(a, p, __builtin_amdgcn_readfirstlane(slot_cur), tid);
        const bool valid = op.valid;
        op.store(sm, tid);
        __syncthreads();
        if constexpr (!SYNC) op.load(a, pn, __builtin_amdgcn_readfirstlane(slot_next), tid, live);
        // query tile qt: the block's rows 32 qt ..; all but the last tile, then
        // the last, after whose linear read the state slice registers are free
        // for the next pair's slice
#pragma unroll
        for (int qt = 0; qt + 1 < KT; ++qt) {
            f32x16 lacc, vacc;
            float sp, sn, den, m, l;
            {
                bf16x8 pb[F / 16];
                phi_operands<D, FW, KT, 1>(sm, 32 * qt, ln, g, pb, sp, sn, den);
                vacc = block_softmax_pv<D, FW, KT, 1>(a, sm, 32 * qt, wv, ln, g, m, l);
                lacc = linear_read<D, FW>(sv, pb, sp, sn);
            }
            merge_store(a, vacc, lacc, gamma, m, l, den, sn, r, h, wv, 32 * qt + ln, g, valid);
            // at two work-groups per CU the tiles must not overlap (registers);
            // at one, letting them overlap is faster
            if constexpr (fwd_wpe<D, FW, KT>() > 1) __builtin_amdgcn_sched_barrier(0);
        }
        constexpr int QL = KT - 1;
        f32x16 lacc, vacc;
        float sp, sn, den, m, l;
        {
            bf16x8 pb[F / 16];
            phi_operands<D, FW, KT, 1>(sm, 32 * QL, ln, g, pb, sp, sn, den);
            vacc = block_softmax_pv<D, FW, KT, 1>(a, sm, 32 * QL, wv, ln, g, m, l);
            lacc = linear_read<D, FW>(sv, pb, sp, sn);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
            const float* nrec;
            if constexpr (SYNC) nrec = rec_of(pn, __builtin_amdgcn_readfirstlane(slot_next));
            else nrec = op.rec;  // the next pair's, loaded one pair ahead
            load_state_slice(nrec + wv * F * 32, lane, sv, live);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kFwdStagedOut && KT == 1) {
            merge_to_lds<D>(a, vacc, lacc, gamma, m, l, den, sn, wv, ln, g, valid, sm.Os);
            __syncthreads();
            store_out_rows<D, C::NT>(a, sm.Os, r, h, tid);
        } else {
            merge_store(a, vacc, lacc, gamma, m, l, den, sn, r, h, wv, 32 * QL + ln, g, valid);
        }
        // the slot id read at the top of this trip crosses the loop in a
        // vector register: its wait lands here, a whole trip after the load,
        // and covers no load issued since
        asm volatile("" : "+v"(slot_after));
        slot_cur = slot_next;
        slot_next = slot_after;
        p = pn;
    }
}

// F = 256 with the state slice split by feature half: wave w takes value
// columns 32 (w % NW) and features [FW (w / NW), FW (w / NW) + FW), a
// 64-register slice as at F = 128, so two waves share each SIMD (the whole
// slice, 128 registers, allows one). Both waves of a column slice compute the
// feature logits and their own half's exponentials, normaliser and Z share.
// The + half wave reads its half of the state, runs the block softmax and
// P V, and posts them through LDS; the - half wave scales that accumulator by
// sn / sp and continues it over its own half -- the one-wave kernel's order of
// operations, so the output is the same bit for bit -- then merges and stores.
// Measured at 1,024 x 16 pairs, d = 128, B = 32: 532.4 -> 502.4 us per
// forward (adding the two halves' partial sums instead of continuing one
// accumulator: 490.6 us, but no longer the one-wave kernel's result).
constexpr bool kFwdSplitHalves = true;

template <int D>
__global__ __launch_bounds__(2 * 64 * (D / 32)) __attribute__((amdgpu_waves_per_eu(2, 2))) void forward_split_kernel(
    ForwardArgs a, int npairs)
{
    constexpr int FW = 128;
    using C = Cfg<D, FW>;
    constexpr int F = C::F, NW = C::NW, NT = 2 * C::NT, HS = FW / 8;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ln = lane & 31, g = lane >> 5;
    const int cs = wv % NW, hh = wv / NW;  // column slice, feature half
    const int NG = gridDim.x;
    int p = blockIdx.x;
    if (p >= npairs) return;
    const int h = p % a.H;
    const float gamma = a.gamma[h];

    __shared__ FwdLds<D, FW> sm;
    __shared__ float Xl[NW * 16 * 64];  // the + half's linear read, lane order
    __shared__ float Xv[NW * 16 * 64];  // its P V
    __shared__ __attribute__((aligned(16))) float Xs[NW * 32 * 4];  // per query: m, l, sp, dp
    {
        WChunks<D, FW, NT> wc;
        wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh, tid);
        wc.template store_rows<C::RS>(sm.Ws, tid);
    }

    auto slot_of = [&](int pp) { return a.slot_ids[(pp < npairs ? pp : npairs - 1) / a.H]; };
    const int count = (npairs - p + NG - 1) / NG;
    PairOperands<D, FW, 1, 1, NT> op;
    f32x4 sv[HS];
    const int soff = cs * F * 32 + hh * HS * 256;  // this wave's half slice (floats)
    op.load(a, p, slot_of(p), tid);
    __builtin_amdgcn_sched_barrier(0);
    load_state_slice(op.rec + soff, lane, sv);
    __builtin_amdgcn_sched_barrier(0);
    int slot_next = slot_of(p + NG);
    for (int k = 0; k < count; ++k) {
        const int live = k + 1 < count ? 1 : 0;
        const int pn = live ? p + NG : p;
        const bool valid = op.valid;
        const int r = p / a.H;
        int slot_after = slot_of(pn + NG);
        __syncthreads();  // every wave is done with the previous pair's LDS operands
        op.store(sm, tid);
        __syncthreads();
        op.load(a, pn, __builtin_amdgcn_readfirstlane(slot_next), tid, live);
        bf16x8 pb[FW / 16];
        float s, dz;
        phi_half_operands<D, FW>(sm.Ws, sm.Qs, sm.Zs, ln, g, hh, pb, s, dz);
        if (hh == 0) {
            const f32x16 lacc = linear_read_half<FW>(sv, pb, f32x16{});
            __builtin_amdgcn_sched_barrier(0);
            load_state_slice(op.rec + soff, lane, sv, live);
            __builtin_amdgcn_sched_barrier(0);
            float m, l;
            const f32x16 vacc = block_softmax_pv<D, FW, 1, 1>(a, sm, 0, cs, ln, g, m, l);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                Xl[(cs * 16 + v) * 64 + lane] = lacc[v];
                Xv[(cs * 16 + v) * 64 + lane] = vacc[v];
            }
            if (g == 0) *reinterpret_cast<f32x4*>(Xs + (cs * 32 + ln) * 4) = f32x4{m, l, s, dz};
        }
        __syncthreads();
        if (hh == 1) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(Xs + (cs * 32 + ln) * 4);
            const float m = x[0], l = x[1], sp = x[2], dp = x[3];
            const float rs = s / sp;  // s: sn of this half
            f32x16 lacc, vacc;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                lacc[v] = Xl[(cs * 16 + v) * 64 + lane] * rs;
                vacc[v] = Xv[(cs * 16 + v) * 64 + lane];
            }
            lacc = linear_read_half<FW>(sv, pb, lacc);
            __builtin_amdgcn_sched_barrier(0);
            load_state_slice(op.rec + soff, lane, sv, live);
            __builtin_amdgcn_sched_barrier(0);
            merge_store(a, vacc, lacc, gamma, m, l, dp / sp + dz / s, s, r, h, cs, ln, g, valid);
        }
        asm volatile("" : "+v"(slot_after));
        slot_next = slot_after;
        p = pn;
    }
}

// ---------------------------------------------------------------------------
// Grouped forward with shared per-head operands (G query heads per K/V head,
// blocks of up to 32 tokens). Every wave needs every query head's phi(q) and
// P for its own 32 output columns; instead of each wave computing all of them
// (as the one-head kernel run over G query tiles would), wave w computes phi(q) and the
// block softmax of query heads w, w + NW, ... only, and the results go to LDS
// as the B operands of the linear read and of P V (bf16, in lane order) plus
// the per-query scalars; after a barrier every wave reads each head's operands
// and does its own columns' linear read, P V and merge. The operands reuse the
// LDS of Q and K, which phase one has finished with.
// ---------------------------------------------------------------------------
template <int D, int FW, int G>
struct alignas(16) GqaLds {
    using C = Cfg<D, FW>;
    static constexpr int F = C::F;
    static constexpr int QK_BYTES = (32 * G + 32) * C::RS * 2;  // Q of the G heads, then K
    static constexpr int PB_BYTES = G * (F / 16) * 64 * 16;     // phi(q) operands
    static constexpr int PP_BYTES = G * 2 * 64 * 16;            // P operands
    static constexpr int SC_BYTES = G * 5 * 32 * 4;             // sp, sn, den, m, l per query
    static constexpr int SH_BYTES = PB_BYTES + PP_BYTES + SC_BYTES;
    static constexpr int U_BYTES = QK_BYTES > SH_BYTES ? QK_BYTES : SH_BYTES;
    uint8_t u[U_BYTES];
    uint16_t Ws[FW * C::RS];
    uint16_t Vs[32 * C::RS];
    float Zs[F];
    __device__ uint16_t* qs() { return reinterpret_cast<uint16_t*>(u); }
    __device__ uint16_t* ks() { return reinterpret_cast<uint16_t*>(u) + 32 * G * C::RS; }
    __device__ bf16x8* pb() { return reinterpret_cast<bf16x8*>(u); }
    __device__ bf16x8* pp() { return reinterpret_cast<bf16x8*>(u + PB_BYTES); }
    __device__ float* sc() { return reinterpret_cast<float*>(u + PB_BYTES + PP_BYTES); }
};

// Operand loads one unit ahead (registers held across the unit), except for
// four query heads at FW = 64: there the next unit's four heads of Q would
// not fit beside two work-groups per CU, so each unit loads its own operands
// at its start and the second work-group covers the wait. Measured at 256
// requests x 16 query heads over 4 K/V heads: 41.8 us prefetching at one
// work-group per CU, 34.8 us loading in place at two (in place at one: 46.9;
// for two and eight heads in place is 2-5 % slower at unchanged occupancy).
template <int D, int FW, int G>
constexpr bool gqa_sync_operands()
{
    return D == 128 && G == 4 && FW == 64;
}

// Resident work-groups per CU: two, unless the F = 256 state slice (128
// registers), eight heads' operands, or four heads' prefetched operands at
// FW = 64 leave room for one.
template <int D, int FW, int G>
constexpr int gqa_wpe()
{
    return FW >= 128 || G >= 8 || (G >= 4 && FW >= 64 && !gqa_sync_operands<D, FW, G>()) ? 1 : 2;
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

template <int D, int FW, int G>
__global__ __launch_bounds__(64 * (D / 32))
__attribute__((amdgpu_waves_per_eu(gqa_wpe<D, FW, G>(), gqa_wpe<D, FW, G>()))) void forward_gqa_mfma_kernel(
    ForwardArgs a, int npairs)
{
    using C = Cfg<D, FW>;
    constexpr int F = C::F, NW = C::NW, HPW = (G + NW - 1) / NW;  // phase-one heads per wave
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ln = lane & 31, g = lane >> 5;
    const int NG = gridDim.x, HK = a.H / G;
    int p = blockIdx.x;
    if (p >= npairs) return;
    const int hk = p % HK;
    float gamma[G];
#pragma unroll
    for (int j = 0; j < G; ++j) gamma[j] = a.gamma[hk * G + j];

    __shared__ GqaLds<D, FW, G> sm;
    uint16_t* const Qs = sm.qs();
    uint16_t* const Ks = sm.ks();
    bf16x8* const PB = sm.pb();
    bf16x8* const PP = sm.pp();
    float* const SC = sm.sc();
    {
        WChunks<D, FW, C::NT> wc;
        wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(hk) * a.wh, tid);
        wc.template store_rows<C::RS>(sm.Ws, tid);
    }

    // slot ids run one pair ahead of the operand loads (index clamped in range)
    auto slot_of = [&](int pp) { return a.slot_ids[(pp < npairs ? pp : npairs - 1) / HK]; };
    const int count = (npairs - p + NG - 1) / NG;
    PairOperands<D, FW, 1, G> op;
    f32x4 sv[C::NSL];
    // the state record of unit u with slot id sl (slot 0's for an out-of-range slot)
    auto rec_of = [&](int u, int sl) {
        const bool ok = sl >= 0 && sl < a.num_slots;
        return a.state + (static_cast<int64_t>(ok ? sl : 0) * HK + u % HK) * static_cast<int64_t>(D + 1) * F;
    };
    constexpr bool SYNC = gqa_sync_operands<D, FW, G>();
    if constexpr (!SYNC) op.load(a, p, slot_of(p), tid);
    __builtin_amdgcn_sched_barrier(0);
    load_state_slice((SYNC ? rec_of(p, slot_of(p)) : op.rec) + wv * F * 32, lane, sv);
    __builtin_amdgcn_sched_barrier(0);
    int slot_cur = slot_of(p);
    int slot_next = slot_of(p + NG);
    for (int k = 0; k < count; ++k) {
        const int live = k + 1 < count ? 1 : 0;
        const int pn = live ? p + NG : p;
        const int r = p / HK;
        int slot_after = slot_of(pn + NG);
        __syncthreads();  // every wave is done with the previous pair's LDS operands
        if constexpr (SYNC) op.load(a, p, __builtin_amdgcn_readfirstlane(slot_cur), tid);
        const bool valid = op.valid;
        op.store_to(Qs, Ks, sm.Vs, sm.Zs, tid);
        __syncthreads();
        if constexpr (!SYNC) op.load(a, pn, __builtin_amdgcn_readfirstlane(slot_next), tid, live);

        // lane indices made opaque each trip: the LDS addresses derived from
        // them are computed in the loop, not kept in registers across it
        int tlane = lane;
        asm volatile("" : "+v"(tlane));
        const int tln = tlane & 31, tg = tlane >> 5;
        // phase one: phi(q) and the block softmax of this wave's query heads
        bf16x8 pbo[HPW][F / 16], ppo[HPW][2];
        float sco[HPW][5];
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int j = wv + NW * i;
            if (j < G) {
                const uint16_t* const Qj = Qs + 32 * j * C::RS;
                phi_operands_at<D, FW>(sm.Ws, Qj, sm.Zs, tln, tg, pbo[i], sco[i][0], sco[i][1], sco[i][2]);
                block_softmax_at<D>(a, Ks, Qj, tln, tg, sco[i][3], sco[i][4], ppo[i]);
            }
        }
        __syncthreads();  // Q and K are no longer read: their LDS takes the shared operands
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int j = wv + NW * i;
            if (j < G) {
#pragma unroll
                for (int kb = 0; kb < F / 16; ++kb) PB[(j * (F / 16) + kb) * 64 + tlane] = pbo[i][kb];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) PP[(j * 2 + kb) * 64 + tlane] = ppo[i][kb];
                if (tg == 0) {
#pragma unroll
                    for (int e = 0; e < 5; ++e) SC[(j * 5 + e) * 32 + tln] = sco[i][e];
                }
            }
        }
        __syncthreads();

        // phase two: every query head's linear read, P V and merge for this
        // wave's 32 columns; after the last head's linear read the state slice
        // registers take the next pair's slice
#pragma unroll
        for (int j = 0; j < G; ++j) {
            bf16x8 pb[F / 16], pp[2];
#pragma unroll
            for (int kb = 0; kb < F / 16; ++kb) pb[kb] = PB[(j * (F / 16) + kb) * 64 + tlane];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) pp[kb] = PP[(j * 2 + kb) * 64 + tlane];
            const float sp = SC[(j * 5 + 0) * 32 + tln], sn = SC[(j * 5 + 1) * 32 + tln];
            const float den = SC[(j * 5 + 2) * 32 + tln], m = SC[(j * 5 + 3) * 32 + tln];
            const float l = SC[(j * 5 + 4) * 32 + tln];
            const f32x16 lacc = linear_read<D, FW>(sv, pb, sp, sn);
            if (j == G - 1) {
                __builtin_amdgcn_sched_barrier(0);
                const float* nrec;
                if constexpr (SYNC) nrec = rec_of(pn, __builtin_amdgcn_readfirstlane(slot_next));
                else nrec = op.rec;  // the next unit's, loaded one unit ahead
                load_state_slice(nrec + wv * F * 32, lane, sv, live);
                __builtin_amdgcn_sched_barrier(0);
            }
            f32x16 vacc = f32x16{};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) vacc = mfma32(vt_frag<C::RS>(sm.Vs, 32 * wv, kb, tlane), pp[kb], vacc);
            merge_store(a, vacc, lacc, gamma[j], m, l, den, sn, r, hk * G + j, wv, tln, tg, valid);
            __builtin_amdgcn_sched_barrier(0);  // one head's operands in registers at a time
        }
        asm volatile("" : "+v"(slot_after));
        slot_cur = slot_next;
        slot_next = slot_after;
        p = pn;
    }
}

// Eight query heads per K/V head (FW <= 64) in two passes of four. The unit's
// K, V, Z and state slice are loaded once; each pass stages four heads' Q,
// runs phase one (phi(q) and the block softmax, one head per wave at d = 128)
// into the shared operands and phase two (every head's linear read from the
// slice, P V and merge). K stays in LDS across both passes, so the work-group
// needs 79 KiB of LDS at FW = 64 instead of the 114 KiB of staging all eight
// heads at once, and two work-groups share a CU. Each unit loads its
// operands at its start; only the state slice runs a unit ahead.
template <int D, int FW>
struct alignas(16) Gqa8Lds {
    using C = Cfg<D, FW>;
    static constexpr int F = C::F, GP = 4;  // query heads per pass
    static constexpr int Q_BYTES = 32 * GP * C::RS * 2;
    static constexpr int PB_BYTES = GP * (F / 16) * 64 * 16;  // phi(q) operands
    static constexpr int PP_BYTES = GP * 2 * 64 * 16;         // P operands
    static constexpr int SC_BYTES = GP * 5 * 32 * 4;          // sp, sn, den, m, l per query
    static constexpr int SH_BYTES = PB_BYTES + PP_BYTES + SC_BYTES;
    static constexpr int U_BYTES = Q_BYTES > SH_BYTES ? Q_BYTES : SH_BYTES;
    uint8_t u[U_BYTES];  // the pass's Q, then the shared operands
    uint16_t Ks[32 * C::RS];
    uint16_t Ws[FW * C::RS];
    uint16_t Vs[32 * C::RS];
    float Zs[F];
};

template <int D, int FW>
__global__ __launch_bounds__(64 * (D / 32)) __attribute__((amdgpu_waves_per_eu(2, 2))) void forward_gqa8_kernel(
    ForwardArgs a, int npairs)
{
    using C = Cfg<D, FW>;
    using L = Gqa8Lds<D, FW>;
    constexpr int F = C::F, NW = C::NW, NT = C::NT, G = 8, GP = L::GP;
    constexpr int HPW = (GP + NW - 1) / NW;  // phase-one heads per wave and pass
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int NG = gridDim.x, HK = a.H / G;
    int p = blockIdx.x;
    if (p >= npairs) return;
    const int hk = p % HK;

    __shared__ L sm;
    uint16_t* const Qs = reinterpret_cast<uint16_t*>(sm.u);
    bf16x8* const PB = reinterpret_cast<bf16x8*>(sm.u);
    bf16x8* const PP = reinterpret_cast<bf16x8*>(sm.u + L::PB_BYTES);
    float* const SC = reinterpret_cast<float*>(sm.u + L::PB_BYTES + L::PP_BYTES);
    {
        WChunks<D, FW, NT> wc;
        wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(hk) * a.wh, tid);
        wc.template store_rows<C::RS>(sm.Ws, tid);
    }
    auto slot_of = [&](int pp) { return a.slot_ids[(pp < npairs ? pp : npairs - 1) / HK]; };
    auto rec_of = [&](int u, int sl) {
        const bool ok = sl >= 0 && sl < a.num_slots;
        return a.state + (static_cast<int64_t>(ok ? sl : 0) * HK + u % HK) * static_cast<int64_t>(D + 1) * F;
    };
    const int count = (npairs - p + NG - 1) / NG;
    const int qtok = static_cast<int>(a.qs.tok), ktok = static_cast<int>(a.ks.tok);
    RowChunks<D, NT> kc, vc;
    RowChunks<D, NT, 32 * GP> qc;
    auto load_q = [&](int u, int ps) {
        const int64_t qbase = static_cast<int64_t>(u / HK) * a.qs.req +
                              static_cast<int64_t>(hk * G + ps * GP) * a.qs.head;
        qc.template load_heads<32>(static_cast<const uint16_t*>(a.q) + qbase, qtok, a.qs.head, a.B, tid);
    };
    f32x4 sv[C::NSL];
    load_state_slice(rec_of(p, slot_of(p)) + wv * F * 32, lane, sv);
    int slot_cur = slot_of(p);
    int slot_next = slot_of(p + NG);
    for (int k = 0; k < count; ++k) {
        const int live = k + 1 < count ? 1 : 0;
        const int pn = live ? p + NG : p;
        const int r = p / HK;
        int slot_after = slot_of(pn + NG);
        __syncthreads();  // every wave is done with the previous unit's LDS operands
        {
            const int sl = __builtin_amdgcn_readfirstlane(slot_cur);
            const float* rec = rec_of(p, sl);
            const int64_t kbase = static_cast<int64_t>(r) * a.ks.req + static_cast<int64_t>(hk) * a.ks.head;
            kc.load(static_cast<const uint16_t*>(a.k) + kbase, ktok, a.B, tid);
            vc.load(static_cast<const uint16_t*>(a.v) + kbase, ktok, a.B, tid);
            const f32x4 z = reinterpret_cast<const f32x4*>(rec + D * F)[tid % (F / 4)];
            load_q(p, 0);
            kc.template store_rows<C::RS>(sm.Ks, tid);
            vc.template store_rows<C::RS>(sm.Vs, tid);
            if (tid < F / 4) reinterpret_cast<f32x4*>(sm.Zs)[tid] = z;
            qc.template store_rows<C::RS>(Qs, tid);
        }
        const bool valid = slot_cur >= 0 && slot_cur < a.num_slots;
        __syncthreads();
#pragma unroll
        for (int ps = 0; ps < G / GP; ++ps) {
            if (ps > 0) {
                load_q(p, ps);
                __syncthreads();  // the previous pass's shared operands are read
                qc.template store_rows<C::RS>(Qs, tid);
                __syncthreads();
            }
            int tlane = lane;
            asm volatile("" : "+v"(tlane));
            const int tln = tlane & 31, tg = tlane >> 5;
            bf16x8 pbo[HPW][F / 16], ppo[HPW][2];
            float sco[HPW][5];
#pragma unroll
            for (int i = 0; i < HPW; ++i) {
                const int j = wv + NW * i;
                if (j < GP) {
                    const uint16_t* const Qj = Qs + 32 * j * C::RS;
                    phi_operands_at<D, FW>(sm.Ws, Qj, sm.Zs, tln, tg, pbo[i], sco[i][0], sco[i][1], sco[i][2]);
                    block_softmax_at<D>(a, sm.Ks, Qj, tln, tg, sco[i][3], sco[i][4], ppo[i]);
                }
            }
            __syncthreads();  // the pass's Q is no longer read: its LDS takes the shared operands
#pragma unroll
            for (int i = 0; i < HPW; ++i) {
                const int j = wv + NW * i;
                if (j < GP) {
#pragma unroll
                    for (int kb = 0; kb < F / 16; ++kb) PB[(j * (F / 16) + kb) * 64 + tlane] = pbo[i][kb];
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) PP[(j * 2 + kb) * 64 + tlane] = ppo[i][kb];
                    if (tg == 0) {
#pragma unroll
                        for (int e = 0; e < 5; ++e) SC[(j * 5 + e) * 32 + tln] = sco[i][e];
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < GP; ++j) {
                bf16x8 pb[F / 16], pp[2];
#pragma unroll
                for (int kb = 0; kb < F / 16; ++kb) pb[kb] = PB[(j * (F / 16) + kb) * 64 + tlane];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) pp[kb] = PP[(j * 2 + kb) * 64 + tlane];
                const float sp = SC[(j * 5 + 0) * 32 + tln], sn = SC[(j * 5 + 1) * 32 + tln];
                const float den = SC[(j * 5 + 2) * 32 + tln], m = SC[(j * 5 + 3) * 32 + tln];
                const float l = SC[(j * 5 + 4) * 32 + tln];
                const f32x16 lacc = linear_read<D, FW>(sv, pb, sp, sn);
                if (ps == G / GP - 1 && j == GP - 1) {
                    // the last head's linear read is done: the slice registers
                    // take the next unit's slice
                    __builtin_amdgcn_sched_barrier(0);
                    load_state_slice(rec_of(pn, __builtin_amdgcn_readfirstlane(slot_next)) + wv * F * 32, lane, sv,
                                     live);
                    __builtin_amdgcn_sched_barrier(0);
                }
                f32x16 vacc = f32x16{};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    vacc = mfma32(vt_frag<C::RS>(sm.Vs, 32 * wv, kb, tlane), pp[kb], vacc);
                // the head's gate: a uniform load, read when it is needed
                const float gamma = a.gamma[hk * G + ps * GP + j];
                merge_store(a, vacc, lacc, gamma, m, l, den, sn, r, hk * G + ps * GP + j, wv, tln, tg, valid);
                __builtin_amdgcn_sched_barrier(0);  // one head's operands in registers at a time
            }
        }
        asm volatile("" : "+v"(slot_after));
        slot_cur = slot_next;
        slot_next = slot_after;
        p = pn;
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
    if (a.commit_mask != nullptr && a.commit_mask[r] == 0) return;
    // K, V and W do not depend on the slot: their loads go out first
    const int slot = a.slot_ids[r];
    const int64_t base = static_cast<int64_t>(r) * a.ks.req + static_cast<int64_t>(h) * a.ks.head;
    RowChunks<D, C::NT> kc, vc;
    WChunks<D, FW, C::NT> wc;
    kc.load(static_cast<const uint16_t*>(a.k) + base, static_cast<int>(a.ks.tok), B, tid);
    vc.load(static_cast<const uint16_t*>(a.v) + base, static_cast<int>(a.ks.tok), B, tid);
    wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh, tid);
    if (slot < 0 || slot >= a.num_slots) return;
    float* rec = a.state + (static_cast<int64_t>(slot) * a.H + h) * static_cast<int64_t>(D + 1) * F;
    f32x4 sv[C::NSL];
    load_state_slice(rec + wv * F * 32, lane, sv);
    // Z goes out with the slice (thread tid holds Z[tid + j NT]), so the
    // work-group ends with stores only, not a dependent read of Z after the
    // products
    constexpr int ZPT = (F + C::NT - 1) / C::NT;
    float zold[ZPT];
#pragma unroll
    for (int j = 0; j < ZPT; ++j) zold[j] = tid + j * C::NT < F ? rec[D * F + tid + j * C::NT] : 0.0f;
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
#pragma unroll
    for (int j = 0; j < ZPT; ++j) {
        const int f = tid + j * C::NT;
        if (f < F) {
            float z = 0.0f;
#pragma unroll
            for (int t = 0; t < 32; ++t) z += Pt[f * C::PS + t];
            rec[D * F + f] = zold[j] + z;
        }
    }
}

// ---------------------------------------------------------------------------
// Forward + commit: the last denoising step of a block. One work-group per
// pair computes the step's output from the state as it stands (committed
// blocks only) and then folds the block's K and V into the same state slice,
// which it holds in registers: the record is read once and written once, and
// the separate commit's reads of the record, K and V are saved. Requests with
// commit_mask[r] == 0 only get the forward.
// ---------------------------------------------------------------------------
template <int D, int FW>
struct alignas(16) FusedLds {
    FwdLds<D, FW> f;
    float Pt[Cfg<D, FW>::F * Cfg<D, FW>::PS];  // phi(K)^T, fp32 [f][t]
};

template <int D, int FW>
__global__ __launch_bounds__(64 * (D / 32))
__attribute__((amdgpu_waves_per_eu(Cfg<D, FW>::WPE, Cfg<D, FW>::WPE))) void forward_commit_mfma_kernel(ForwardArgs a, CommitArgs c)
{
    using C = Cfg<D, FW>;
    constexpr int F = C::F;
    const int pair = blockIdx.x;
    const int r = pair / a.H, h = pair % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ln = lane & 31, g = lane >> 5;
    __shared__ FusedLds<D, FW> sm;

    // Q, K, V and W first (they do not depend on the slot), then the slice
    PairOperands<D, FW> op;
    WChunks<D, FW, C::NT> wc;
    wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh, tid);
    op.load(a, pair, a.slot_ids[r], tid);
    f32x4 sv[C::NSL];
    load_state_slice(op.rec + wv * F * 32, lane, sv);
    const bool commit = op.valid && (c.commit_mask == nullptr || c.commit_mask[r] != 0);
    const float gamma = a.gamma[h];
    op.store(sm.f, tid);
    wc.template store_rows<C::RS>(sm.f.Ws, tid);
    __syncthreads();

    // the forward, from the state as loaded
    {
        f32x16 lacc, vacc;
        float sp, sn, den, m, l;
        bf16x8 pb[F / 16];
        phi_operands<D, FW, 1, 1>(sm.f, 0, ln, g, pb, sp, sn, den);
        vacc = block_softmax_pv<D, FW, 1, 1>(a, sm.f, 0, wv, ln, g, m, l);
        lacc = linear_read<D, FW>(sv, pb, sp, sn);
        merge_store(a, vacc, lacc, gamma, m, l, den, sn, r, h, wv, ln, g, op.valid);
    }
    if (!commit) return;
    __builtin_amdgcn_sched_barrier(0);  // keep the commit's work out of the forward's live range

    // phi(k_t) for token ln, normalised, fp32; tokens past B give zero
    {
        f32x16 u[FW / 32];
        feature_logits<D, FW, C::RS>(sm.f.Ws, sm.f.Ks, ln, g, u);
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
        const float ip = ln < a.B ? 1.0f / sp : 0.0f;
        const float in = ln < a.B ? 1.0f / sn : 0.0f;
        // every wave has the logits of all 32 tokens; wave w writes the
        // feature tiles T = w (mod waves) of phi(K)^T
#pragma unroll
        for (int T = 0; T < FW / 32; ++T) {
            if (T % C::NW != wv) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int fw = 32 * T + 8 * (v >> 2) + 4 * g + (v & 3);
                sm.Pt[fw * C::PS + ln] = __expf(u[T][v] - mx) * ip;
                sm.Pt[(FW + fw) * C::PS + ln] = __expf(mn - u[T][v]) * in;
            }
        }
    }
    __syncthreads();

    // dS = phi(K)^T V into the slice: A from phi(K)^T rows with the token
    // order of vt_frag (16 kb + 4 g + {0..3}, 16 kb + 8 + 4 g + {0..3})
#pragma unroll
    for (int ft = 0; ft < F / 32; ++ft) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const float* pr = sm.Pt + (32 * ft + ln) * C::PS + 16 * kb + 4 * g;
            const f32x4 p0 = *reinterpret_cast<const f32x4*>(pr);
            const f32x4 p1 = *reinterpret_cast<const f32x4*>(pr + 8);
            bf16x8 ap;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ap[e] = static_cast<__bf16>(p0[e]);
                ap[4 + e] = static_cast<__bf16>(p1[e]);
            }
            acc = mfma32(ap, vt_frag<C::RS>(sm.f.Vs, 32 * wv, kb, lane), acc);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) sv[4 * ft + (v >> 2)][v & 3] += acc[v];
    }
    float* rec = const_cast<float*>(op.rec);
    f32x4* dst = reinterpret_cast<f32x4*>(rec + wv * F * 32) + lane;
#pragma unroll
    for (int t = 0; t < C::NSL; ++t) __builtin_nontemporal_store(sv[t], dst + t * 64);
    // Z as loaded for the forward (its LDS copy), plus the block's phi sums:
    // the work-group ends with stores only
    for (int f = tid; f < F; f += C::NT) {
        float z = 0.0f;
#pragma unroll
        for (int t = 0; t < 32; ++t) z += sm.Pt[f * C::PS + t];
        rec[D * F + f] = sm.f.Zs[f] + z;
    }
}

// ---------------------------------------------------------------------------
// Prefill: one work-group of four waves per (request, head) folds the
// request's whole packed token range into the state; the record is read once
// and written once, the state staying in registers throughout. Wave w owns the
// state rows [r0, r0 + RW) of the value columns [32 cs, 32 cs + 32): with
// d = 128 one column slice and all F features (cs = w), with d = 64 one column
// slice and one feature half. Tokens go in chunks of CT = 64, 16 per wave:
//   * each wave computes phi(k_t) for its own 16 tokens with 16x16x32 tiles
//     (lane = token n, k-group q: features 16 T + 4 q + {0..3}); the
//     contraction over d is fed in the order q, k-step ks -> elements
//     q d/4 + 8 ks .. + 7, the same for W, so each lane's K fragments are one
//     contiguous d/4-element run of its token's row, loaded straight from
//     global memory into registers; the per-token max, min and sums over the
//     features combine the four k-group lanes;
//   * phi(K) goes to LDS once as bf16 rows and V rows are copied to LDS; both
//     are read back transposed (ds_read_b64_tr_b16) as the A and B operands of
//     dS = phi(K)^T V, accumulated straight into the state tiles. Rows past
//     the end of the request hold copies of its last row, with zero phi;
//   * Z accumulates in fp32 per lane (token slot) and is reduced across slots
//     once, at the end, in a fixed order.
// The loop is software pipelined: phi of chunk c + 1 and dS of chunk c run
// between two barriers, from opposite LDS buffers; the K and V loads of chunk
// c + 2 are issued during chunk c + 1's phi. LDS (80 KiB
// at d = 128, F = 128) and registers are sized so that two work-groups share a
// CU and cover each other's barrier and memory waits.
// ---------------------------------------------------------------------------
template <int D, int FW>
struct PCfg {
    static constexpr int F = 2 * FW;
    static constexpr int NC = D / 32;                   // 32-column slices of the state
    static constexpr int NWV = F * NC > 512 ? 8 : 4;    // waves: at most 128 state rows each
    static constexpr int NT = 64 * NWV;
    static constexpr int CT = 16 * NWV;                 // tokens per chunk, 16 per wave
    static constexpr int RW = F * NC / NWV;             // state rows of one wave
    static constexpr int VC = D / 8;                    // 16-byte chunks per row of V and W
    static constexpr int KS = D / 32;                   // k-steps of the 16x16x32 logits
    static constexpr int PD = 1;                        // chunks whose loads run ahead of phi
    static constexpr int VQ = CT * VC / NT;             // 16-byte V chunks per thread per chunk
    // two LDS buffers of V and phi(K) (pipelined loop) when they fit
    static constexpr int NBUF = 2 * (2 * CT * (D + F) + FW * D) <= 160 * 1024 ? 2 : 1;
    static constexpr int MAIN = 2 * (NBUF * CT * (D + F) + FW * D);
    static constexpr int ZRED = 4 * CT * F;             // fp32 Z partials of every token slot
    static constexpr int LDS = MAIN > ZRED ? MAIN : ZRED;
    // one-buffer loop: each wave's four state tiles are 2 x 2 (two column
    // slices, 64 rows) rather than 4 x 1, so a step of dS reads four operand
    // fragments instead of five
    static constexpr bool SQ = NBUF == 1 && NC % 2 == 0 && RW == 128;
};

// State tile i of wave wv in the prefill: its first row and column slice.
template <int D, int FW>
__device__ __forceinline__ int ptile_row(int wv, int i)
{
    using P = PCfg<D, FW>;
    if constexpr (P::SQ) return (wv / (P::NC / 2)) * 64 + 32 * (i / 2);
    else return (wv / P::NC) * P::RW + 32 * i;
}
template <int D, int FW>
__device__ __forceinline__ int ptile_col(int wv, int i)
{
    using P = PCfg<D, FW>;
    if constexpr (P::SQ) return 2 * (wv % (P::NC / 2)) + i % 2;
    else return wv % P::NC;
}

// All-reductions over the lane pairs (L, L ^ 16) and (L, L ^ 32) with the
// gfx950 row-swap instructions (VALU, no LDS round trip): swapping a value
// with itself leaves each lane holding its own and its partner's.
__device__ __forceinline__ float max_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float min_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float min_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-pair constants of the prefill loop.
template <int D, int FW>
struct PrefillPair {
    const uint16_t* kbase;  // first token row of the request, this head
    const uint16_t* vbase;
    int64_t tok64;          // token stride (elements)
    int tok;
    int n;                  // tokens of the request
    int nchunks;
};

template <int D, int FW>
__device__ __forceinline__ int prefill_chunk_rows(const PrefillPair<D, FW>& pp, int c)
{
    constexpr int CT = PCfg<D, FW>::CT;
    return pp.n - CT * c < CT ? pp.n - CT * c : CT;
}

// V rows of chunk c: thread tid's 16-byte chunks; rows past the end read the
// request's last row (their phi is zero). Nothing consumes the registers until
// they are stored, so the loads stay in flight.
template <int D, int FW>
__device__ __forceinline__ void prefill_load_v(const PrefillPair<D, FW>& pp, int c, int tid,
                                               u32x4 (&vr)[PCfg<D, FW>::VQ])
{
    using P = PCfg<D, FW>;
    const int nc = prefill_chunk_rows(pp, c);
    const uint16_t* src = pp.vbase + static_cast<int64_t>(P::CT) * c * pp.tok64;
#pragma unroll
    for (int i = 0; i < P::VQ; ++i) {
        const int idx = tid + i * P::NT, t = idx / P::VC, ch = idx % P::VC;
        const int tr = t < nc ? t : nc - 1;
        vr[i] = *reinterpret_cast<const u32x4*>(src + (tr * pp.tok + ch * 8));
    }
}

template <int D, int FW>
__device__ __forceinline__ void prefill_store_v(uint16_t* Vb, int tid, const u32x4 (&vr)[PCfg<D, FW>::VQ])
{
    using P = PCfg<D, FW>;
#pragma unroll
    for (int i = 0; i < P::VQ; ++i) {
        const int idx = tid + i * P::NT, t = idx / P::VC, ch = idx % P::VC;
        *reinterpret_cast<u32x4*>(Vb + t * D + (((2 * ch) ^ lds_piece_swizzle<D / 4>(t)) << 2)) = vr[i];
    }
}

// K fragments of wave wv's 16 tokens of chunk c for lane (n16, q): the run
// q d/4 .. q d/4 + d/4 - 1 of the token's row.
template <int D, int FW>
__device__ __forceinline__ void prefill_load_k(const PrefillPair<D, FW>& pp, int c, int wv, int n16, int q,
                                               bf16x8 (&kf)[D / 32])
{
    constexpr int CT = PCfg<D, FW>::CT;
    const int nc = prefill_chunk_rows(pp, c);
    const int t = 16 * wv + n16;
    const int tr = t < nc ? t : nc - 1;
    const uint16_t* src = pp.kbase + static_cast<int64_t>(CT) * c * pp.tok64 + (tr * pp.tok + q * (D / 4));
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) kf[ks] = *reinterpret_cast<const bf16x8*>(src + 8 * ks);
}

// First half of chunk c: V rows to LDS, the loads PD chunks ahead issued,
// phi(K) of this wave's 16 tokens to LDS and into the Z partials. Safe for
// c == nchunks (one past the end): no loads, zero phi, buffers unused.
template <int D, int FW>
__device__ __forceinline__ void prefill_phi(const PrefillPair<D, FW>& pp, int c, int tid, uint16_t* Vs,
                                            uint16_t* Ps, const uint16_t* Ws, u32x4 (&vr)[PCfg<D, FW>::VQ],
                                            bf16x8 (&kf)[D / 32], float (&zl)[FW / 2])
{
    using P = PCfg<D, FW>;
    constexpr int F = P::F, CT = P::CT, KS = P::KS, PD = P::PD;
    constexpr float kLog2e = 1.4426950408889634f;
    const int lane = tid & 63, wv = tid >> 6;
    const int n16 = lane & 15, q = lane >> 4;
    const int nc = prefill_chunk_rows(pp, c);
    uint16_t* const Vb = Vs + (P::NBUF == 2 ? (c & 1) : 0) * (CT * D);
    uint16_t* const Pb = Ps + (P::NBUF == 2 ? (c & 1) : 0) * (CT * F);
    prefill_store_v<D, FW>(Vb, tid, vr);
    if (c + PD < pp.nchunks) prefill_load_v(pp, c + PD, tid, vr);

    // feature logits of this wave's 16 tokens
    f32x4 u[FW / 16];
#pragma unroll
    for (int T = 0; T < FW / 16; ++T) u[T] = f32x4{};
    // W sits in LDS as the logits' A fragments in read order: block
    // ks FW/16 + T (1 KiB) holds, at 16-byte slot lane = n16 + 16 q, the
    // elements q d/4 + 8 ks .. + 7 of row 16 T + n16, so each fragment read is
    // one contiguous, conflict-free 1 KiB. The lane's slot is one address and
    // the blocks are immediate offsets (an opaque lane offset keeps the sum an
    // add that the read can fold)
    int wo = 8 * lane;
    asm volatile("" : "+v"(wo));
    const uint16_t* const Wl = Ws + wo;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int T = 0; T < FW / 16; ++T) u[T] = mfma16(lds_frag(Wl + (ks * (FW / 16) + T) * 512), kf[ks], u[T]);
    if (c + PD < pp.nchunks) prefill_load_k(pp, c + PD, wv, n16, q, kf);
    // per-token extremes and sums over the four k-group lanes (L, L ^ 16,
    // L ^ 32, L ^ 48); the exponentials are base 2 of the scaled differences
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int T = 0; T < FW / 16; ++T)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mx = fmaxf(mx, u[T][e]);
            mn = fminf(mn, u[T][e]);
        }
    mx = max_xor32(max_xor16(mx)) * kLog2e;
    mn = min_xor32(min_xor16(mn)) * kLog2e;
    f32x4 en[FW / 16];
    float sp = 0.0f, sn = 0.0f;
#pragma unroll
    for (int T = 0; T < FW / 16; ++T)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ea = __builtin_amdgcn_exp2f(fmaf(u[T][e], kLog2e, -mx));
            const float eb = __builtin_amdgcn_exp2f(fmaf(u[T][e], -kLog2e, mn));
            u[T][e] = ea;
            en[T][e] = eb;
            sp += ea;
            sn += eb;
        }
    sp = sum_xor32(sum_xor16(sp));
    sn = sum_xor32(sum_xor16(sn));
    const bool valid = 16 * wv + n16 < nc;
    const float ip = valid ? __builtin_amdgcn_rcpf(sp) : 0.0f;
    const float in = valid ? __builtin_amdgcn_rcpf(sn) : 0.0f;
    const int prow_t = 16 * wv + n16;
    uint16_t* const prow = Pb + prow_t * F;
    const int psw = lds_piece_swizzle<F / 4>(prow_t);
#pragma unroll
    for (int T = 0; T < FW / 16; ++T) {
        uint16_t hp[4], hn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float pp_ = u[T][e] * ip, pn = en[T][e] * in;
            zl[4 * T + e] += pp_;
            zl[FW / 4 + 4 * T + e] += pn;
            hp[e] = bf16_bits(pp_);
            hn[e] = bf16_bits(pn);
        }
        // features 16 T + 4 q .. + 3 are piece 4 T + q (+ FW / 4 for the - half)
        const int jp = 4 * T + q, jn = FW / 4 + jp;
        *reinterpret_cast<uint2*>(prow + ((jp ^ psw) << 2)) =
            make_uint2(hp[0] | (uint32_t(hp[1]) << 16), hp[2] | (uint32_t(hp[3]) << 16));
        *reinterpret_cast<uint2*>(prow + ((jn ^ psw) << 2)) =
            make_uint2(hn[0] | (uint32_t(hn[1]) << 16), hn[2] | (uint32_t(hn[3]) << 16));
    }
}

// Element offset, in a piece-swizzled tile of RB pieces per row, of the
// transposed read that vt_frag_ps issues at step 0 for lane lane: row
// 4 g + m / 4 (+ 8 for the upper half), piece c0 / 4 + 4 (q & 1) + m % 4.
template <int RB>
__device__ __forceinline__ int vt_offset_ps(int c0, int row_add, int lane)
{
    const int m = lane & 15, q = lane >> 4, g = lane >> 5;
    const int piece = (c0 >> 2) + 4 * (q & 1) + (m & 3);
    const int row = 4 * g + (m >> 2) + row_add;
    return row * (4 * RB) + ((piece ^ lds_piece_swizzle<RB>(row)) << 2);
}

__device__ __forceinline__ bf16x8 vt_frag_at(const uint16_t* Xs, int lo_off, int hi_off)
{
    const i16x4 lo = lds_read_tr(Xs + lo_off);
    const i16x4 hi = lds_read_tr(Xs + hi_off);
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Second half of chunk c: dS = phi(K)^T V over the chunk, this wave's state
// rows and value columns, accumulated into its state tiles.
template <int D, int FW>
__device__ __forceinline__ void prefill_ds(int c, int tid, const uint16_t* Vs, const uint16_t* Ps,
                                           f32x16 (&st)[PCfg<D, FW>::RW / 32])
{
    using P = PCfg<D, FW>;
    constexpr int F = P::F, NC = P::NC, CT = P::CT, RW = P::RW;
    const int lane = tid & 63, wv = tid >> 6;
    const int cs = wv % NC, r0 = (wv / NC) * RW;
    const uint16_t* const Vb = Vs + (P::NBUF == 2 ? (c & 1) : 0) * (CT * D);
    const uint16_t* const Pb = Ps + (P::NBUF == 2 ? (c & 1) : 0) * (CT * F);
    if constexpr (P::NBUF == 2) {
#pragma unroll
        for (int kb = 0; kb < CT / 16; ++kb) {
            const bf16x8 bv = vt_frag_ps<D / 4>(Vb, 32 * cs, kb, lane);
#pragma unroll
            for (int ft = 0; ft < RW / 32; ++ft)
                st[ft] = mfma32(vt_frag_ps<F / 4>(Pb, r0 + 32 * ft, kb, lane), bv, st[ft]);
        }
    } else {
        // one work-group per CU: no other work-group's waves hide the LDS
        // latency, so the fragments of step kb + 1 are read before step kb's
        // products are issued. The read offsets are formed once: the swizzle
        // depends on the low four bits of the row only, so step kb is the same
        // offsets 16 kb rows further on (an immediate offset of the read).
        // operand fragments of one step: V of the wave's NV column slices, phi(K)
        // of its NP row tiles; tile i takes row operand i / NV and column i % NV
        constexpr int NV = P::SQ ? 2 : 1, NP = RW / 32 / NV;
        int vlo[NV], vhi[NV], plo[NP], phi_[NP];
#pragma unroll
        for (int b = 0; b < NV; ++b) {
            vlo[b] = vt_offset_ps<D / 4>(32 * ptile_col<D, FW>(wv, b), 0, lane);
            vhi[b] = vt_offset_ps<D / 4>(32 * ptile_col<D, FW>(wv, b), 8, lane);
        }
#pragma unroll
        for (int a = 0; a < NP; ++a) {
            plo[a] = vt_offset_ps<F / 4>(ptile_row<D, FW>(wv, NV * a), 0, lane);
            phi_[a] = vt_offset_ps<F / 4>(ptile_row<D, FW>(wv, NV * a), 8, lane);
        }
        bf16x8 bv[NV], pa[NP];
#pragma unroll
        for (int b = 0; b < NV; ++b) bv[b] = vt_frag_at(Vb, vlo[b], vhi[b]);
#pragma unroll
        for (int a = 0; a < NP; ++a) pa[a] = vt_frag_at(Pb, plo[a], phi_[a]);
#pragma unroll
        for (int kb = 0; kb < CT / 16; ++kb) {
            bf16x8 bn[NV], pn[NP];
#pragma unroll
            for (int b = 0; b < NV; ++b) bn[b] = bv[b];
#pragma unroll
            for (int a = 0; a < NP; ++a) pn[a] = pa[a];
            if (kb + 1 < CT / 16) {
                const uint16_t* const vk = Vb + 16 * (kb + 1) * D;
                const uint16_t* const pk = Pb + 16 * (kb + 1) * F;
#pragma unroll
                for (int b = 0; b < NV; ++b) bn[b] = vt_frag_at(vk, vlo[b], vhi[b]);
#pragma unroll
                for (int a = 0; a < NP; ++a) pn[a] = vt_frag_at(pk, plo[a], phi_[a]);
            }
#pragma unroll
            for (int t = 0; t < RW / 32; ++t) st[t] = mfma32(pa[t / NV], bv[t % NV], st[t]);
#pragma unroll
            for (int b = 0; b < NV; ++b) bv[b] = bn[b];
#pragma unroll
            for (int a = 0; a < NP; ++a) pa[a] = pn[a];
        }
    }
}

template <int D, int FW>
__global__ __launch_bounds__(64 * (2 * FW * (D / 32) > 512 ? 8 : 4)) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_mfma_kernel(CommitArgs a)
{
    using P = PCfg<D, FW>;
    constexpr int F = P::F, NC = P::NC, NT = P::NT, CT = P::CT, RW = P::RW, KS = P::KS, VQ = P::VQ;
    const int pair = blockIdx.x;
    const int h = pair % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n16 = lane & 15, q = lane >> 4;

    __shared__ __attribute__((aligned(16))) uint8_t smem[P::LDS];
    static_assert(P::LDS >= 4 * kPrefillOrderLds, "the ordering scratch fits the LDS");
    const int r = prefill_request<NT>(a, pair / a.H, tid, reinterpret_cast<int*>(smem));
    uint16_t* const Vs = reinterpret_cast<uint16_t*>(smem);
    uint16_t* const Ps = Vs + P::NBUF * CT * D;
    uint16_t* const Ws = Ps + P::NBUF * CT * F;
    float* const Zr = reinterpret_cast<float*>(smem);

    const int slot = a.slot_ids[r];
    if (slot < 0 || slot >= a.num_slots) return;
    int64_t first_row;
    int n;
    commit_rows(a, r, first_row, n);
    if (n == 0) return;
    float* rec = a.state + (static_cast<int64_t>(slot) * a.H + h) * static_cast<int64_t>(D + 1) * F;
    // a packed token range, or (a commit of B tokens) the request's block rows
    const int64_t base = (first_row >= 0 ? first_row * a.ks.tok : static_cast<int64_t>(r) * a.ks.req) +
                         static_cast<int64_t>(h) * a.ks.head;
    PrefillPair<D, FW> pp;
    pp.kbase = static_cast<const uint16_t*>(a.k) + base;
    pp.vbase = static_cast<const uint16_t*>(a.v) + base;
    pp.tok64 = a.ks.tok;
    pp.tok = static_cast<int>(a.ks.tok);
    pp.n = n;
    pp.nchunks = (n + CT - 1) / CT;

    {
        const uint16_t* w = static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh;
        constexpr int NWC = FW * P::VC / NT;  // 16-byte chunks of W per thread
        u32x4 wr[NWC];
#pragma unroll
        for (int i = 0; i < NWC; ++i) {
            const int idx = tid + i * NT, row = idx / P::VC, ch = idx % P::VC;
            wr[i] = *reinterpret_cast<const u32x4*>(w + row * D + ch * 8);
        }
#pragma unroll
        for (int i = 0; i < NWC; ++i) {
            // chunk ch of row 16 T + n16 is k-group q = ch / KS, k-step ks = ch % KS
            const int idx = tid + i * NT, row = idx / P::VC, ch = idx % P::VC;
            const int blk = (ch % KS) * (FW / 16) + row / 16, slot = (ch / KS) * 16 + row % 16;
            *reinterpret_cast<u32x4*>(Ws + (blk * 64 + slot) * 8) = wr[i];
        }
    }

    // state tile ft: rows ptile_row + (C layout), columns 32 ptile_col + lane % 32
    f32x16 st[RW / 32];
    // (tiles of one column slice: one base, the tiles at fixed offsets)
    const f32x4* const sp0 = reinterpret_cast<const f32x4*>(
                                 rec + 32 * (ptile_col<D, FW>(wv, 0) * F + ptile_row<D, FW>(wv, 0))) + lane;
#pragma unroll
    for (int ft = 0; ft < RW / 32; ++ft) {
        const f32x4* const sp4 =
            P::SQ ? reinterpret_cast<const f32x4*>(
                        rec + 32 * (ptile_col<D, FW>(wv, ft) * F + ptile_row<D, FW>(wv, ft))) + lane
                  : sp0 + 4 * ft * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 x = __builtin_nontemporal_load(sp4 + i * 64);
#pragma unroll
            for (int e = 0; e < 4; ++e) st[ft][4 * i + e] = x[e];
        }
    }
    float zl[FW / 2];  // this lane's token slot: features 16 T + 4 q + e of the + half, then the - half
#pragma unroll
    for (int i = 0; i < FW / 2; ++i) zl[i] = 0.0f;

    // one register set: chunk c's loads are issued while chunk c - 1's phi is
    // computed, and consumed by chunk c's
    u32x4 vr[VQ];
    bf16x8 kf[KS];
    prefill_load_v(pp, 0, tid, vr);
    prefill_load_k(pp, 0, wv, n16, q, kf);
    if constexpr (P::NBUF == 2) {
        // chunk c lives in LDS buffer c % 2
        __syncthreads();  // W rows visible to every wave
        prefill_phi(pp, 0, tid, Vs, Ps, Ws, vr, kf, zl);
        __syncthreads();
        for (int c = 0; c < pp.nchunks; ++c) {
            prefill_phi(pp, c + 1, tid, Vs, Ps, Ws, vr, kf, zl);
            prefill_ds<D, FW>(c, tid, Vs, Ps, st);
            __syncthreads();
        }
    } else {
        // one buffer: phi and dS of a chunk between barriers. The thread index
        // is made opaque each trip, so the swizzled LDS addresses derived from
        // it are computed in the loop rather than hoisted out of it: hoisted,
        // they do not fit the registers beside the F = 256 state tiles, and
        // their scratch reloads (each waiting for every load in flight) drain
        // the K/V prefetch
        for (int c = 0; c < pp.nchunks; ++c) {
            int tl = tid;
            asm volatile("" : "+v"(tl));
            tl &= NT - 1;  // known in range: index arithmetic stays unsigned shifts
            __syncthreads();  // W rows staged; every wave is done with the previous chunk
            prefill_phi(pp, c, tl, Vs, Ps, Ws, vr, kf, zl);
            __syncthreads();
            prefill_ds<D, FW>(c, tl, Vs, Ps, st);
        }
        __syncthreads();
    }

    f32x4* const dst0 = reinterpret_cast<f32x4*>(rec + 32 * (ptile_col<D, FW>(wv, 0) * F + ptile_row<D, FW>(wv, 0))) + lane;
#pragma unroll
    for (int ft = 0; ft < RW / 32; ++ft) {
        f32x4* const dst =
            P::SQ ? reinterpret_cast<f32x4*>(rec + 32 * (ptile_col<D, FW>(wv, ft) * F + ptile_row<D, FW>(wv, ft))) + lane
                  : dst0 + 4 * ft * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 x = {st[ft][4 * i], st[ft][4 * i + 1], st[ft][4 * i + 2], st[ft][4 * i + 3]};
            __builtin_nontemporal_store(x, dst + i * 64);
        }
    }

    // Z: the token slots' fp32 partials, reduced in a fixed order
    float* const zrow = Zr + (16 * wv + n16) * F + 4 * q;
#pragma unroll
    for (int T = 0; T < FW / 16; ++T) {
        *reinterpret_cast<f32x4*>(zrow + 16 * T) = f32x4{zl[4 * T], zl[4 * T + 1], zl[4 * T + 2], zl[4 * T + 3]};
        *reinterpret_cast<f32x4*>(zrow + FW + 16 * T) =
            f32x4{zl[FW / 4 + 4 * T], zl[FW / 4 + 4 * T + 1], zl[FW / 4 + 4 * T + 2], zl[FW / 4 + 4 * T + 3]};
    }
    __syncthreads();
    for (int f = tid; f < F; f += NT) {
        float z = 0.0f;
        for (int sl = 0; sl < CT; ++sl) z += Zr[sl * F + f];
        rec[D * F + f] += z;
    }
}

// ---------------------------------------------------------------------------
// Feature map (bha_feature_map, bf16 tokens)
// ---------------------------------------------------------------------------
// One work-group of D/32 waves per (head, 32 D/32 consecutive tokens of the
// [R][B] batch). W_h and the tokens' rows go to LDS; each wave then takes 32
// tokens: u^T = W^T X^T on the matrix cores (lane = token, as in the
// forward) and both softmaxes of each token in fp32 (lanes n and n + 32 hold
// halves of token n's logits). phi leaves through the wave's own 32 rows of
// the X tile, which the logits no longer need: a piece of CW features of
// every token at a time is written there from the accumulator layout and read
// back row by row, so each store instruction writes whole CW * 4-byte runs of
// phi rows (the accumulator layout writes 32-byte pieces of 32 rows per
// instruction; measured at 256 x 32 tokens x 16 heads, FW = 64: 40.7 us).
// Roofline: HBM. Algorithmic bytes per (token, head): the row read (2 d) and
// phi written (4 F); W once per head per launch.
template <int D, int FW>
__global__ __launch_bounds__(64 * (D / 32)) void feature_map_mfma_kernel(PhiArgs a, int tiles)
{
    using C = Cfg<D, FW>;
    constexpr int NT = C::NT, TOK = 32 * C::NW, CH = D / 8, F = C::F;
    // features per staged piece (32 rows x CW floats fit the wave's 32 X rows)
    constexpr int CW = (D == 128 ? 64 : 32) < FW ? (D == 128 ? 64 : 32) : FW;
    constexpr int CS = CW + 4;              // padded LDS row (floats) of a staged piece
    static_assert(32 * CS * 4 <= 32 * C::RS * 2, "a staged piece fits the wave's X rows");
    __shared__ alignas(16) uint16_t Ws[FW * C::RS];
    __shared__ alignas(16) uint16_t Xs[TOK * C::RS];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ln = lane & 31, g = lane >> 5;
    const int h = blockIdx.x / tiles;
    const int64_t ntok = static_cast<int64_t>(a.R) * a.B;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x % tiles) * TOK;
    {
        WChunks<D, FW, NT> wc;
        wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh, tid);
        wc.template store_rows<C::RS>(Ws, tid);
    }
    // the tile's rows, 16 bytes per thread per step (rows past the batch read
    // its last row and are not stored)
    u32x4 xv[TOK * CH / NT];
#pragma unroll
    for (int i = 0; i < TOK * CH / NT; ++i) {
        const int idx = tid + i * NT, row = idx / CH, ch = idx % CH;
        const int64_t tk = t0 + row < ntok ? t0 + row : ntok - 1;
        const int64_t r = tk / a.B, t = tk % a.B;
        const uint16_t* src = static_cast<const uint16_t*>(a.x) + r * a.xs.req + t * a.xs.tok +
                              static_cast<int64_t>(h) * a.xs.head + 8 * ch;
        xv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
    }
#pragma unroll
    for (int i = 0; i < TOK * CH / NT; ++i) {
        const int idx = tid + i * NT, row = idx / CH, ch = idx % CH;
        *reinterpret_cast<u32x4*>(Xs + row * C::RS + 8 * ch) = xv[i];
    }
    __syncthreads();
    f32x16 u[FW / 32];
    feature_logits<D, FW, C::RS>(Ws, Xs + 32 * wv * C::RS, ln, g, u);
    constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) u[T][v] *= kLog2e;  // base-2 logits
    float mx, mn;
    logit_range<FW>(u, mx, mn);
    float sp = 0.0f, sn = 0.0f;
    f32x16 en[FW / 32];
#pragma unroll
    for (int T = 0; T < FW / 32; ++T)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float x = u[T][v];
            u[T][v] = __builtin_amdgcn_exp2f(x - mx);
            en[T][v] = __builtin_amdgcn_exp2f(mn - x);
            sp += u[T][v];
            sn += en[T][v];
        }
    sp += __shfl_xor(sp, 32, 64);
    sn += __shfl_xor(sn, 32, 64);
    const float ip = 1.0f / sp, in = 1.0f / sn;
    float* const stage = reinterpret_cast<float*>(Xs + 32 * wv * C::RS);  // this wave's X rows
    const int64_t tw = t0 + 32 * wv;  // the wave's first token
    // piece (half hf, features c0 .. c0 + CW - 1 of that half)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int c0 = 0; c0 < FW; c0 += CW) {
            __syncthreads();  // the previous piece's reads (or the logits' reads of X) are done
#pragma unroll
            for (int T = c0 / 32; T < (c0 + CW) / 32; ++T)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    f32x4 pv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) pv[e] = hf ? en[T][4 * q4 + e] * in : u[T][4 * q4 + e] * ip;
                    *reinterpret_cast<f32x4*>(stage + ln * CS + 32 * T - c0 + 8 * q4 + 4 * g) = pv;
                }
            __syncthreads();
            // rows of CW floats, CW / 4 lanes per row
#pragma unroll
            for (int i = 0; i < 32 * CW / 4 / 64; ++i) {
                const int idx = lane + 64 * i, row = idx / (CW / 4), c4 = idx % (CW / 4);
                const int64_t tk = tw + row;
                if (tk < ntok)
                    *reinterpret_cast<f32x4*>(a.phi + (tk * a.H + h) * F + hf * FW + c0 + 4 * c4) =
                        *reinterpret_cast<const f32x4*>(stage + row * CS + 4 * c4);
            }
        }
}

// Compute units of the current device (cached per device ordinal).
static int compute_units()
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

// Persistent grid: as many work-groups as can be resident (WPE per CU),
// rounded down to a multiple of H so that each keeps one head, and no more
// than there are pairs. With at least kFwdOneGroupPairs pairs per CU the
// one-tile forward runs one work-group per CU instead of two: the memory
// system streams more with half the state slices in flight (measured at
// d = 128, FW = 64, B = 32, six rotating state pools: 512 requests x 16 heads
// 151.3 -> 141.2 us, 1,024 requests 295.1 -> 276.9 us), while below that the
// one work-group's first and last pairs cost more than they save (256
// requests: 77.8 -> 79.5 us).
constexpr int kFwdOneGroupPairs = 32;

template <int D, int FW, int KT>
static hipError_t launch_forward_kt(const ForwardArgs& a, hipStream_t s)
{
    const int npairs = a.R * a.H;
    const int cus = compute_units();
    int wpe = fwd_wpe<D, FW, KT>();
    if (KT == 1 && wpe == 2 && npairs >= static_cast<int64_t>(kFwdOneGroupPairs) * cus) wpe = 1;
    int64_t NG = static_cast<int64_t>(cus) * wpe;
    NG = (NG / a.H) * a.H;
    if (NG < a.H) NG = a.H;
    if (NG > npairs) NG = npairs;
    return launch_kernel(forward_mfma_kernel<D, FW, KT>, dim3(static_cast<uint32_t>(NG)), dim3(64 * (D / 32)), s, a,
                         npairs);
}

// The split-slice F = 256 forward: one work-group of 2 NW waves per CU.
template <int D>
static hipError_t launch_forward_split(const ForwardArgs& a, hipStream_t s)
{
    const int npairs = a.R * a.H;
    int64_t NG = static_cast<int64_t>(compute_units());
    NG = (NG / a.H) * a.H;
    if (NG < a.H) NG = a.H;
    if (NG > npairs) NG = npairs;
    return launch_kernel(forward_split_kernel<D>, dim3(static_cast<uint32_t>(NG)), dim3(2 * 64 * (D / 32)), s, a,
                         npairs);
}

template <int D, int FW, int G>
static hipError_t launch_forward_gqa(const ForwardArgs& a, hipStream_t s)
{
    const int hk = a.H / G, npairs = a.R * hk;
    int64_t NG = static_cast<int64_t>(compute_units()) * gqa_wpe<D, FW, G>();
    NG = (NG / hk) * hk;
    if (NG < hk) NG = hk;
    if (NG > npairs) NG = npairs;
    return launch_kernel(forward_gqa_mfma_kernel<D, FW, G>, dim3(static_cast<uint32_t>(NG)), dim3(64 * (D / 32)), s,
                         a, npairs);
}

// Blocks of up to 64 tokens with one query head per K/V head; up to 32 tokens
// with 2, 4 (or, at FW <= 64, 8) query heads per K/V head.
template <int D, int FW>
static hipError_t launch_forward(const ForwardArgs& a, hipStream_t s)
{
    if (a.G == 1) {
        if constexpr (kFwdSplitHalves && D == 128 && FW == 128)
            if (a.B <= 32) return launch_forward_split<D>(a, s);
        return a.B <= 32 ? launch_forward_kt<D, FW, 1>(a, s) : launch_forward_kt<D, FW, 2>(a, s);
    }
    if (a.G == 2) return launch_forward_gqa<D, FW, 2>(a, s);
    if (a.G == 4) return launch_forward_gqa<D, FW, 4>(a, s);
    if constexpr (FW <= 64) {
        const int hk = a.H / 8, npairs = a.R * hk;
        int64_t NG = static_cast<int64_t>(compute_units()) * 2;
        NG = (NG / hk) * hk;
        if (NG < hk) NG = hk;
        if (NG > npairs) NG = npairs;
        return launch_kernel(forward_gqa8_kernel<D, FW>, dim3(static_cast<uint32_t>(NG)), dim3(64 * (D / 32)), s,
                             a, npairs);
    }
    return hipErrorInvalidValue;  // excluded by forward_mfma_supported
}

template <int D>
static hipError_t forward_by_fw(const ForwardArgs& a, hipStream_t s)
{
    switch (a.FW) {
        case 32: return launch_forward<D, 32>(a, s);
        case 64: return launch_forward<D, 64>(a, s);
        default: return launch_forward<D, 128>(a, s);
    }
}

template <int D>
static hipError_t prefill_by_fw(const CommitArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(a.R * a.H));
    switch (a.FW) {
        case 32: return launch_kernel(prefill_mfma_kernel<D, 32>, grid, dim3(PCfg<D, 32>::NT), s, a);
        case 64: return launch_kernel(prefill_mfma_kernel<D, 64>, grid, dim3(PCfg<D, 64>::NT), s, a);
        default: return launch_kernel(prefill_mfma_kernel<D, 128>, grid, dim3(PCfg<D, 128>::NT), s, a);
    }
}

// Blocks of 33..64 rows are not taken here but by the prefill kernel over
// each request's B rows (at FW = 128 a kernel folding two 32-token tiles into
// the register slice in turn measured 357.6 / 360.4 us against 274.1 / 276.9
// us for the prefill kernel at B = 48 / 64, 256 x 16 pairs, d = 128).
template <int D>
static hipError_t commit_by_fw(const CommitArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(a.R * a.H)), block(64 * (D / 32));
    switch (a.FW) {
        case 32: return launch_kernel(commit_mfma_kernel<D, 32>, grid, block, s, a);
        case 64: return launch_kernel(commit_mfma_kernel<D, 64>, grid, block, s, a);
        default: return launch_kernel(commit_mfma_kernel<D, 128>, grid, block, s, a);
    }
}

template <int D>
static hipError_t forward_commit_by_fw(const ForwardArgs& a, const CommitArgs& c, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(a.R * a.H)), block(64 * (D / 32));
    switch (a.FW) {
        case 32: return launch_kernel(forward_commit_mfma_kernel<D, 32>, grid, block, s, a, c);
        case 64: return launch_kernel(forward_commit_mfma_kernel<D, 64>, grid, block, s, a, c);
        default: return launch_kernel(forward_commit_mfma_kernel<D, 128>, grid, block, s, a, c);
    }
}

template <int D>
static hipError_t feature_map_by_fw(const PhiArgs& a, hipStream_t s)
{
    constexpr int TOK = 32 * (D / 32);
    const int64_t tiles = (static_cast<int64_t>(a.R) * a.B + TOK - 1) / TOK;
    const dim3 grid(static_cast<uint32_t>(tiles * a.H)), block(64 * (D / 32));
    const int nt = static_cast<int>(tiles);
    switch (a.FW) {
        case 32: return launch_kernel(feature_map_mfma_kernel<D, 32>, grid, block, s, a, nt);
        case 64: return launch_kernel(feature_map_mfma_kernel<D, 64>, grid, block, s, a, nt);
        default: return launch_kernel(feature_map_mfma_kernel<D, 128>, grid, block, s, a, nt);
    }
}

}  // namespace

// The matrix-core kernels address a block's rows with 32-bit offsets.
static bool small_token_stride(int64_t tok) { return tok >= 0 && tok < (int64_t(1) << 25); }

static bool mfma_sizes(int d, int FW) { return (d == 64 || d == 128) && (FW == 32 || FW == 64 || FW == 128); }

bool forward_mfma_supported(const ForwardArgs& a)
{
    if (a.io != BHA_BF16 || a.B < 1 || a.B > 64 || !mfma_sizes(a.d, a.FW)) return false;
    if (!small_token_stride(a.qs.tok) || !small_token_stride(a.ks.tok) || !small_token_stride(a.os.tok)) return false;
    if (a.G == 1) return true;
    // grouped K/V heads: one 32-token tile, 2 or 4 query heads per K/V head,
    // or 8 at FW <= 64
    return a.B <= 32 && (a.G == 2 || a.G == 4 || (a.G == 8 && a.FW <= 64));
}

hipError_t launch_forward_mfma(const ForwardArgs& a, hipStream_t s)
{
    return a.d == 128 ? forward_by_fw<128>(a, s) : forward_by_fw<64>(a, s);
}

bool prefill_mfma_supported(const CommitArgs& a)
{
    // packed ranges (seq_offsets), or blocks of B <= 64 rows per request;
    // in-chunk offsets (up to 128 rows) are 32-bit
    if (a.io != BHA_BF16 || !mfma_sizes(a.d, a.FW)) return false;
    if (a.seq_offsets == nullptr && (a.B < 1 || a.B > 64)) return false;
    return a.ks.tok >= 0 && a.ks.tok < (int64_t(1) << 23);
}

hipError_t launch_prefill_mfma(const CommitArgs& a, hipStream_t s)
{
    return a.d == 128 ? prefill_by_fw<128>(a, s) : prefill_by_fw<64>(a, s);
}

bool forward_commit_mfma_supported(const ForwardArgs& a)
{
    if (a.io != BHA_BF16 || a.B < 1 || a.B > 32 || a.G != 1 || !mfma_sizes(a.d, a.FW)) return false;
    return small_token_stride(a.qs.tok) && small_token_stride(a.ks.tok) && small_token_stride(a.os.tok);
}

hipError_t launch_forward_commit_mfma(const ForwardArgs& a, const CommitArgs& c, hipStream_t s)
{
    return a.d == 128 ? forward_commit_by_fw<128>(a, c, s) : forward_commit_by_fw<64>(a, c, s);
}

bool commit_mfma_supported(const CommitArgs& a)
{
    if (a.io != BHA_BF16 || a.seq_offsets != nullptr || a.B < 1 || a.B > 32 || !mfma_sizes(a.d, a.FW)) return false;
    return small_token_stride(a.ks.tok);
}

hipError_t launch_commit_mfma(const CommitArgs& a, hipStream_t s)
{
    return a.d == 128 ? commit_by_fw<128>(a, s) : commit_by_fw<64>(a, s);
}

// phi is stored with 16-byte stores: its base must be 16-byte aligned (the
// ABI asks for 4; other pointers take the fp32-arithmetic kernel)
bool feature_map_mfma_supported(const PhiArgs& a)
{
    return a.io == BHA_BF16 && a.B >= 1 && mfma_sizes(a.d, a.FW) && a.xs.req >= 0 && a.xs.tok >= 0 &&
           a.xs.head >= 0 && reinterpret_cast<uintptr_t>(a.phi) % 16 == 0;
}

hipError_t launch_feature_map_mfma(const PhiArgs& a, hipStream_t s)
{
    return a.d == 128 ? feature_map_by_fw<128>(a, s) : feature_map_by_fw<64>(a, s);
}

}  // namespace bha
