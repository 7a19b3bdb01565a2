// Matrix-core forward, one query head per K/V head (bha_block_forward):
// the persistent one- and two-tile kernels and the split-slice F = 256
// kernel.
#include "mfma_common.hpp"

namespace bha {

namespace {

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
// streaming. ONE: compiled for one resident wave per SIMD (the register
// budget of a whole SIMD) instead of fwd_wpe.
template <int D, int FW, int KT, bool ONE>
__global__ __launch_bounds__(64 * (D / 32))
__attribute__((amdgpu_waves_per_eu(ONE ? 1 : fwd_wpe<D, FW, KT>(), ONE ? 1 : fwd_wpe<D, FW, KT>()))) void
forward_mfma_kernel(ForwardArgs a, int npairs)
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
            merge_to_lds<D>(a, vacc, lacc, gamma, m, l, den, sn, wv, ln, g, valid, sm.Os);
            __syncthreads();
            // each query tile's rows go out whole from LDS (two-tile blocks of
            // 48 / 64 tokens at FW = 64: 121.8-124.9 -> 120.5-122.1 us and
            // 130.6-132.1 -> 128.0-129.1 us against 32-byte row pieces stored
            // from the merge, same bits)
            store_out_rows<D, C::NT>(a, sm.Os, r, h, tid, 32 * qt);
            __syncthreads();  // the tile is read before the next tile's merge writes it
            // compiled for two waves per SIMD the tiles must not overlap
            // (registers); for one, letting them overlap is faster
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
        if constexpr (kFwdStagedOut) {
            merge_to_lds<D>(a, vacc, lacc, gamma, m, l, den, sn, wv, ln, g, valid, sm.Os);
            __syncthreads();
            store_out_rows<D, C::NT>(a, sm.Os, r, h, tid, 32 * QL);
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
            merge_to_lds<D>(a, vacc, lacc, gamma, m, l, dp / sp + dz / s, s, cs, ln, g, valid, sm.Os);
        }
        // the output rows go out whole from LDS, non-temporal, as in the
        // one-wave kernel (measured at FW = 128, same bits: 512 x 16 pairs
        // 253.6-254.9 -> 249.0-250.2 us, 256 x 16: 134.5-135.5 -> 130.5-132.7
        // us against 32-byte row pieces stored from the merge)
        __syncthreads();
        store_out_rows<D, NT>(a, sm.Os, r, h, tid);
        asm volatile("" : "+v"(slot_after));
        slot_next = slot_after;
        p = pn;
    }
}

// Persistent grid, sized in waves per SIMD: fwd_wpe resident waves per SIMD
// (what the kernel's registers allow), that is fwd_wpe * 4 / (D / 32)
// work-groups of D / 32 waves per CU, rounded down to a multiple of H so that
// each work-group keeps one head, and no more than there are pairs. With at
// least kFwdOneWavePairs pairs per CU and blocks of more than kFwdOneWaveRows
// tokens the one-tile forward runs one wave per SIMD instead of two: each
// pair's chain of loads, products and stores then has its SIMD to itself and
// the memory system streams more with half the state slices in flight. Measured at FW = 64, B = 32, six rotating state
// pools, d = 128 (one work-group per CU against two): 128 requests x 16
// heads 38.6 -> 37.9 us, 192: 54.4 -> 51.3 us, 256: 72.7-72.9 -> 67.1-70.0
// us, 384: 110.2 -> 100.3 us, 512: 149.3 -> 133.3 us; FW = 32, 256 requests
// 50.3 -> 46.8 us; below 8 pairs per CU no difference. At d = 64 (two-wave
// work-groups) one wave per SIMD means two work-groups per CU: 512 requests
// 88.2 -> 79.9 us (FW = 64) and 65.9 -> 52.4 us (FW = 32) against one. The
// two-tile forward, the commit, the fused step, the grouped forwards and the
// prefill are each slower at one wave per SIMD (at 256 requests, d = 128).
// At one wave per SIMD the d = 64 kernel is also compiled for that register
// budget (256 VGPRs instead of 238): 39.2 -> 37.5 us at FW = 64, 256 requests,
// and 51.7 -> 48.4 us at FW = 32, 512 requests; the d = 128 kernel so
// compiled (272 VGPRs) was 1-2 % slower and keeps the two-wave budget.
constexpr int kFwdOneWavePairs = 8;
// Smaller blocks keep two waves per SIMD, where each pair's chain is short
// and a second wave covers its latency (256 requests, FW = 32: B = 8
// 41.0 -> 37.7 us and B = 16 43.4 -> 41.1 us at two; FW = 64: B = 8 61.6 ->
// 59.8 us, B = 16 even, B = 24 even, B = 32 69.7 -> 73.4 us).
constexpr int kFwdOneWaveRows = 16;

template <int D, int FW, int KT>
hipError_t launch_forward_kt(const ForwardArgs& a, hipStream_t s)
{
    const int npairs = a.R * a.H;
    const int cus = compute_units();
    int wps = fwd_wpe<D, FW, KT>();  // resident waves per SIMD
    if (KT == 1 && a.B > kFwdOneWaveRows && npairs >= static_cast<int64_t>(kFwdOneWavePairs) * cus) wps = 1;
    int64_t NG = static_cast<int64_t>(cus) * wps * 4 / (D / 32);
    NG = (NG / a.H) * a.H;
    if (NG < a.H) NG = a.H;
    if (NG > npairs) NG = npairs;
    const dim3 grid(static_cast<uint32_t>(NG)), block(64 * (D / 32));
    if constexpr (D == 64 && KT == 1 && Cfg<D, FW>::WPE == 2)
        if (wps == 1) return launch_kernel(forward_mfma_kernel<D, FW, KT, true>, grid, block, s, a, npairs);
    return launch_kernel(forward_mfma_kernel<D, FW, KT, false>, grid, block, s, a, npairs);
}

// The split-slice F = 256 forward: one work-group of 2 NW waves per CU.
template <int D>
hipError_t launch_forward_split(const ForwardArgs& a, hipStream_t s)
{
    const int npairs = a.R * a.H;
    int64_t NG = static_cast<int64_t>(compute_units());
    NG = (NG / a.H) * a.H;
    if (NG < a.H) NG = a.H;
    if (NG > npairs) NG = npairs;
    return launch_kernel(forward_split_kernel<D>, dim3(static_cast<uint32_t>(NG)), dim3(2 * 64 * (D / 32)), s, a,
                         npairs);
}

// Blocks of up to 64 tokens, one query head per K/V head.
template <int D, int FW>
hipError_t launch_forward(const ForwardArgs& a, hipStream_t s)
{
    if constexpr (kFwdSplitHalves && D == 128 && FW == 128)
        if (a.B <= 32) return launch_forward_split<D>(a, s);
    return a.B <= 32 ? launch_forward_kt<D, FW, 1>(a, s) : launch_forward_kt<D, FW, 2>(a, s);
}

template <int D>
hipError_t forward_by_fw(const ForwardArgs& a, hipStream_t s)
{
    switch (a.FW) {
        case 32: return launch_forward<D, 32>(a, s);
        case 64: return launch_forward<D, 64>(a, s);
        default: return launch_forward<D, 128>(a, s);
    }
}

}  // namespace

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
    if (a.G == 8) return launch_forward_gqa8_mfma(a, s);
    if (a.G != 1) return launch_forward_gqa_mfma(a, s);
    return a.d == 128 ? forward_by_fw<128>(a, s) : forward_by_fw<64>(a, s);
}

}  // namespace bha
