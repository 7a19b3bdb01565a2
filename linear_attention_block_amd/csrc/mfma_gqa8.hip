// Matrix-core grouped forward (bha_block_forward_gqa) with 8 query heads per
// K/V head.
#include "mfma_common.hpp"

namespace bha {

namespace {

// Eight query heads per K/V head (FW <= 64) in two passes of four. The unit's
// K, V, Z and state slice are loaded once; each pass stages four heads' Q,
// runs phase one (phi(q) and the block softmax, one head per wave at d = 128)
// into the shared operands and phase two (every head's linear read from the
// slice, P V and merge). K stays in LDS across both passes, so the work-group
// needs 79 KiB of LDS at FW = 64 instead of the 114 KiB of staging all eight
// heads at once, and two work-groups share a CU. Each unit loads its
// operands at its start; only the state slice runs a unit ahead. When every
// work-group has exactly one unit (ONE), nothing runs ahead: W, K, V, Z and
// the first pass's Q are issued before the state slice, so phase one runs
// while the slice arrives (it is first read by phase two's linear reads).
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

template <int D, int FW, bool ONE>
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
    WChunks<D, FW, NT> wc;
    wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(hk) * a.wh, tid);
    if constexpr (!ONE) wc.template store_rows<C::RS>(sm.Ws, tid);
    auto slot_of = [&](int pp) { return a.slot_ids[(pp < npairs ? pp : npairs - 1) / HK]; };
    auto rec_of = [&](int u, int sl) {
        const bool ok = sl >= 0 && sl < a.num_slots;
        return a.state + (static_cast<int64_t>(ok ? sl : 0) * HK + u % HK) * static_cast<int64_t>(D + 1) * F;
    };
    const int count = ONE ? 1 : (npairs - p + NG - 1) / NG;
    const int qtok = static_cast<int>(a.qs.tok), ktok = static_cast<int>(a.ks.tok);
    RowChunks<D, NT> kc, vc;
    RowChunks<D, NT, 32 * GP> qc;
    auto load_q = [&](int u, int ps) {
        const int64_t qbase = static_cast<int64_t>(u / HK) * a.qs.req +
                              static_cast<int64_t>(hk * G + ps * GP) * a.qs.head;
        qc.template load_heads<32>(static_cast<const uint16_t*>(a.q) + qbase, qtok, a.qs.head, a.B, tid);
    };
    f32x4 sv[C::NSL];
    if constexpr (!ONE) load_state_slice(rec_of(p, slot_of(p)) + wv * F * 32, lane, sv);
    int slot_cur = slot_of(p);
    int slot_next = ONE ? 0 : slot_of(p + NG);
    for (int k = 0; k < count; ++k) {
        const int live = k + 1 < count ? 1 : 0;
        const int pn = live ? p + NG : p;
        const int r = p / HK;
        int slot_after = ONE ? 0 : slot_of(pn + NG);
        __syncthreads();  // every wave is done with the previous unit's LDS operands
        {
            const int sl = __builtin_amdgcn_readfirstlane(slot_cur);
            const float* rec = rec_of(p, sl);
            const int64_t kbase = static_cast<int64_t>(r) * a.ks.req + static_cast<int64_t>(hk) * a.ks.head;
            kc.load(static_cast<const uint16_t*>(a.k) + kbase, ktok, a.B, tid);
            vc.load(static_cast<const uint16_t*>(a.v) + kbase, ktok, a.B, tid);
            const f32x4 z = reinterpret_cast<const f32x4*>(rec + D * F)[tid % (F / 4)];
            load_q(p, 0);
            if constexpr (ONE) {
                load_state_slice(rec + wv * F * 32, lane, sv);
                wc.template store_rows<C::RS>(sm.Ws, tid);
            }
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
                // this pass's Q was loaded during the previous pass's phase two
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
            // the next pass's Q streams in while this pass's heads are merged
            // (phase two holds fewer registers than phase one)
            if (ps + 1 < G / GP) load_q(p, ps + 1);
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
                if (!ONE && ps == G / GP - 1 && j == GP - 1) {
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

template <int D, int FW>
hipError_t launch_forward_gqa8(const ForwardArgs& a, hipStream_t s)
{
    const int hk = a.H / 8, npairs = a.R * hk;
    int64_t NG = static_cast<int64_t>(compute_units()) * 2;
    NG = (NG / hk) * hk;
    if (NG < hk) NG = hk;
    if (NG >= npairs)
        return launch_kernel(forward_gqa8_kernel<D, FW, true>, dim3(static_cast<uint32_t>(npairs)),
                             dim3(64 * (D / 32)), s, a, npairs);
    return launch_kernel(forward_gqa8_kernel<D, FW, false>, dim3(static_cast<uint32_t>(NG)), dim3(64 * (D / 32)), s,
                         a, npairs);
}

template <int D>
hipError_t gqa8_by_fw(const ForwardArgs& a, hipStream_t s)
{
    return a.FW == 32 ? launch_forward_gqa8<D, 32>(a, s) : launch_forward_gqa8<D, 64>(a, s);
}

}  // namespace

// 8 query heads per K/V head, FW <= 64 (the caller has checked
// forward_mfma_supported)
hipError_t launch_forward_gqa8_mfma(const ForwardArgs& a, hipStream_t s)
{
    if (a.G != 8 || a.FW > 64) return hipErrorInvalidValue;
    return a.d == 128 ? gqa8_by_fw<128>(a, s) : gqa8_by_fw<64>(a, s);
}

}  // namespace bha
