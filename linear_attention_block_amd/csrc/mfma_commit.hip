// Matrix-core commit (bha_state_commit, blocks of up to 32 tokens).
#include "mfma_common.hpp"

namespace bha {

namespace {

// ---------------------------------------------------------------------------
// Commit
// ---------------------------------------------------------------------------
template <int D, int FW, bool DEV>
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

    float* const slice = rec + wv * F * 32;  // this wave's slice
    // dS = phi(K)^T V: rows f, this wave's 32 columns; fold into the loaded
    // slice. Each 32-row tile is stored as soon as its dS is added, so the
    // first tiles' stores overlap the later tiles' products
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
#pragma unroll
        for (int i = 0; i < 4; ++i) store_state<DEV, C::NSL>(sv[4 * ft + i], slice, lane, 4 * ft + i);
    }

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

// Blocks of 33..64 rows are not taken here but by the prefill kernel over
// each request's B rows (at FW = 128 a kernel folding two 32-token tiles into
// the register slice in turn measured 357.6 / 360.4 us against 274.1 / 276.9
// us for the prefill kernel at B = 48 / 64, 256 x 16 pairs, d = 128).
template <int D>
hipError_t commit_by_fw(const CommitArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(a.R * a.H)), block(64 * (D / 32));
    const bool dev = static_cast<int64_t>(a.R) * a.H >= static_cast<int64_t>(kDevScopePairsPerCu) * compute_units();
    switch (a.FW) {
        case 32:
            return dev ? launch_kernel(commit_mfma_kernel<D, 32, true>, grid, block, s, a)
                       : launch_kernel(commit_mfma_kernel<D, 32, false>, grid, block, s, a);
        case 64:
            return dev ? launch_kernel(commit_mfma_kernel<D, 64, true>, grid, block, s, a)
                       : launch_kernel(commit_mfma_kernel<D, 64, false>, grid, block, s, a);
        default: return launch_kernel(commit_mfma_kernel<D, 128, false>, grid, block, s, a);
    }
}

}  // namespace

bool commit_mfma_supported(const CommitArgs& a)
{
    if (a.io != BHA_BF16 || a.seq_offsets != nullptr || a.B < 1 || a.B > 32 || !mfma_sizes(a.d, a.FW)) return false;
    return small_token_stride(a.ks.tok);
}

hipError_t launch_commit_mfma(const CommitArgs& a, hipStream_t s)
{
    return a.d == 128 ? commit_by_fw<128>(a, s) : commit_by_fw<64>(a, s);
}

}  // namespace bha
