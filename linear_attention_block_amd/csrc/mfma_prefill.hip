// Matrix-core prefill (bha_state_prefill, and commits of 33 to 64 tokens).
#include "mfma_common.hpp"

namespace bha {

namespace {

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
// BUF: the LDS buffer of chunk c when the caller knows it at compile time
// (c % 2 with two buffers), so that the buffer's base folds into the LDS
// instructions' offsets; -1: chosen at run time.
template <int D, int FW, int BUF = -1>
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
    const int buf = P::NBUF == 2 ? (BUF >= 0 ? BUF : (c & 1)) : 0;
    uint16_t* const Vb = Vs + buf * (CT * D);
    uint16_t* const Pb = Ps + buf * (CT * F);
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
            // Z takes the unrounded products (one rounding, whatever the
            // compiler would contract)
            zl[4 * T + e] = __builtin_fmaf(u[T][e], ip, zl[4 * T + e]);
            zl[FW / 4 + 4 * T + e] = __builtin_fmaf(en[T][e], in, zl[FW / 4 + 4 * T + e]);
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
template <int D, int FW, int BUF = -1>
__device__ __forceinline__ void prefill_ds(int c, int tid, const uint16_t* Vs, const uint16_t* Ps,
                                           f32x16 (&st)[PCfg<D, FW>::RW / 32])
{
    using P = PCfg<D, FW>;
    constexpr int F = P::F, NC = P::NC, CT = P::CT, RW = P::RW;
    const int lane = tid & 63, wv = tid >> 6;
    const int cs = wv % NC, r0 = (wv / NC) * RW;
    const int buf = P::NBUF == 2 ? (BUF >= 0 ? BUF : (c & 1)) : 0;
    const uint16_t* const Vb = Vs + buf * (CT * D);
    const uint16_t* const Pb = Ps + buf * (CT * F);
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
        // chunk c lives in LDS buffer c % 2; two chunks per trip, so every
        // buffer index is a constant and folds into the LDS offsets
        __syncthreads();  // W rows visible to every wave
        prefill_phi<D, FW, 0>(pp, 0, tid, Vs, Ps, Ws, vr, kf, zl);
        __syncthreads();
        int c = 0;
        for (; c + 1 < pp.nchunks; c += 2) {
            prefill_phi<D, FW, 1>(pp, c + 1, tid, Vs, Ps, Ws, vr, kf, zl);
            prefill_ds<D, FW, 0>(c, tid, Vs, Ps, st);
            __syncthreads();
            prefill_phi<D, FW, 0>(pp, c + 2, tid, Vs, Ps, Ws, vr, kf, zl);
            prefill_ds<D, FW, 1>(c + 1, tid, Vs, Ps, st);
            __syncthreads();
        }
        if (c < pp.nchunks) {
            prefill_phi<D, FW, 1>(pp, c + 1, tid, Vs, Ps, Ws, vr, kf, zl);
            prefill_ds<D, FW, 0>(c, tid, Vs, Ps, st);
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

template <int D>
hipError_t prefill_by_fw(const CommitArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(a.R * a.H));
    switch (a.FW) {
        case 32: return launch_kernel(prefill_mfma_kernel<D, 32>, grid, dim3(PCfg<D, 32>::NT), s, a);
        case 64: return launch_kernel(prefill_mfma_kernel<D, 64>, grid, dim3(PCfg<D, 64>::NT), s, a);
        default: return launch_kernel(prefill_mfma_kernel<D, 128>, grid, dim3(PCfg<D, 128>::NT), s, a);
    }
}

}  // namespace

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

}  // namespace bha
