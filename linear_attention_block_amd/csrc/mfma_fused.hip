// Matrix-core forward + commit (bha_block_forward_commit).
#include "mfma_common.hpp"

namespace bha {

namespace {

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

template <int D, int FW, bool DEV>
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

    float* rec = const_cast<float*>(op.rec);
    float* const slice = rec + wv * F * 32;  // this wave's slice
    // dS = phi(K)^T V into the slice: A from phi(K)^T rows with the token
    // order of vt_frag (16 kb + 4 g + {0..3}, 16 kb + 8 + 4 g + {0..3}); each
    // 32-row tile is stored as soon as its dS is added
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
#pragma unroll
        for (int i = 0; i < 4; ++i) store_state<DEV, C::NSL>(sv[4 * ft + i], slice, lane, 4 * ft + i);
    }
    // Z as loaded for the forward (its LDS copy), plus the block's phi sums:
    // the work-group ends with stores only
    for (int f = tid; f < F; f += C::NT) {
        float z = 0.0f;
#pragma unroll
        for (int t = 0; t < 32; ++t) z += sm.Pt[f * C::PS + t];
        rec[D * F + f] = sm.f.Zs[f] + z;
    }
}

template <int D>
hipError_t forward_commit_by_fw(const ForwardArgs& a, const CommitArgs& c, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(a.R * a.H)), block(64 * (D / 32));
    // the state write-back policy of the commit kernel (same rule)
    const bool dev = static_cast<int64_t>(a.R) * a.H >= static_cast<int64_t>(kDevScopePairsPerCu) * compute_units();
    switch (a.FW) {
        case 32:
            return dev ? launch_kernel(forward_commit_mfma_kernel<D, 32, true>, grid, block, s, a, c)
                       : launch_kernel(forward_commit_mfma_kernel<D, 32, false>, grid, block, s, a, c);
        case 64:
            return dev ? launch_kernel(forward_commit_mfma_kernel<D, 64, true>, grid, block, s, a, c)
                       : launch_kernel(forward_commit_mfma_kernel<D, 64, false>, grid, block, s, a, c);
        default: return launch_kernel(forward_commit_mfma_kernel<D, 128, false>, grid, block, s, a, c);
    }
}

}  // namespace

bool forward_commit_mfma_supported(const ForwardArgs& a)
{
    if (a.io != BHA_BF16 || a.B < 1 || a.B > 32 || a.G != 1 || !mfma_sizes(a.d, a.FW)) return false;
    return small_token_stride(a.qs.tok) && small_token_stride(a.ks.tok) && small_token_stride(a.os.tok);
}

hipError_t launch_forward_commit_mfma(const ForwardArgs& a, const CommitArgs& c, hipStream_t s)
{
    return a.d == 128 ? forward_commit_by_fw<128>(a, c, s) : forward_commit_by_fw<64>(a, c, s);
}

}  // namespace bha
