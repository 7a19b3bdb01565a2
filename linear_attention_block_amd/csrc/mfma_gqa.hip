// Matrix-core grouped forward (bha_block_forward_gqa) with 2 or 4 query
// heads per K/V head.
#include "mfma_common.hpp"

namespace bha {

namespace {

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
    // one query head's output tile (merge_to_lds layout), staged at FW <= 64
    uint16_t Os[FW <= 64 ? 32 * (D + 8) : 8];
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
    if constexpr (!SYNC) {
        op.load(a, p, slot_of(p), tid);
        __builtin_amdgcn_sched_barrier(0);
        load_state_slice(op.rec + wv * F * 32, lane, sv);
        __builtin_amdgcn_sched_barrier(0);
    }
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
        // SYNC: the first unit's slice goes out once its operands are in, so
        // that phase one runs while it arrives (later units' slices are
        // issued a unit ahead)
        if (SYNC && k == 0) load_state_slice(rec_of(p, __builtin_amdgcn_readfirstlane(slot_cur)) + wv * F * 32, lane, sv);
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
            // at FW <= 64 the head's output rows go through LDS and out as whole
            // rows with non-temporal stores, as in the one-head forward
            // (measured at 16 query heads, same bits: 256 requests over 8 K/V
            // heads 49.5 -> 47.6 us, over 4: 37.3 -> 37.0 us; 512 over 4: 68.0
            // -> 67.1 us); at FW = 128 the tile's registers would spill
            if constexpr (FW <= 64) {
                merge_to_lds<D>(a, vacc, lacc, gamma[j], m, l, den, sn, wv, tln, tg, valid, sm.Os);
                __syncthreads();
                store_out_rows<D, C::NT>(a, sm.Os, r, hk * G + j, tid);
                __syncthreads();  // the tile is read before the next head's merge writes it
            } else {
                merge_store(a, vacc, lacc, gamma[j], m, l, den, sn, r, hk * G + j, wv, tln, tg, valid);
            }
            __builtin_amdgcn_sched_barrier(0);  // one head's operands in registers at a time
        }
        asm volatile("" : "+v"(slot_after));
        slot_cur = slot_next;
        slot_next = slot_after;
        p = pn;
    }
}

template <int D, int FW, int G>
hipError_t launch_forward_gqa(const ForwardArgs& a, hipStream_t s)
{
    const int hk = a.H / G, npairs = a.R * hk;
    int64_t NG = static_cast<int64_t>(compute_units()) * gqa_wpe<D, FW, G>();
    NG = (NG / hk) * hk;
    if (NG < hk) NG = hk;
    if (NG > npairs) NG = npairs;
    return launch_kernel(forward_gqa_mfma_kernel<D, FW, G>, dim3(static_cast<uint32_t>(NG)), dim3(64 * (D / 32)), s,
                         a, npairs);
}

template <int D, int FW>
hipError_t gqa_by_g(const ForwardArgs& a, hipStream_t s)
{
    return a.G == 2 ? launch_forward_gqa<D, FW, 2>(a, s) : launch_forward_gqa<D, FW, 4>(a, s);
}

template <int D>
hipError_t gqa_by_fw(const ForwardArgs& a, hipStream_t s)
{
    switch (a.FW) {
        case 32: return gqa_by_g<D, 32>(a, s);
        case 64: return gqa_by_g<D, 64>(a, s);
        default: return gqa_by_g<D, 128>(a, s);
    }
}

}  // namespace

// 2 or 4 query heads per K/V head (the caller has checked
// forward_mfma_supported)
hipError_t launch_forward_gqa_mfma(const ForwardArgs& a, hipStream_t s)
{
    if (a.G != 2 && a.G != 4) return hipErrorInvalidValue;
    return a.d == 128 ? gqa_by_fw<128>(a, s) : gqa_by_fw<64>(a, s);
}

}  // namespace bha
