// Plain fp32-arithmetic kernels of block-hybrid attention for gfx950.
//
// They cover every supported size (d in {64,128}, FW in {32,64,128}, B <= 64)
// and both I/O dtypes, with float32 loads, FMAs and accurate expf. They serve
// float32 I/O (where bf16 matrix-core inputs would lose the precision the
// caller asked for) and the block sizes the MFMA kernels do not tile. Each
// work-group handles one token (forward, feature map) or one 32-column slice
// of one state record (commit), staging its operands in LDS.
#include "bha_device.hpp"
#include "bha_internal.hpp"

namespace bha {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Forward: one work-group per (request, head, token i). Computes
//   s_j = scale q_i.k_j, m = max_j s_j, p_j = e^{s_j - m}, l = sum_j p_j,
//   phi(q_i), lin = phi(q_i)^T S, den = phi(q_i)^T Z,
//   y = (al sum_j p_j v_j + be lin) / (al l + be den)  (merge_weights).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void forward_generic_kernel(ForwardArgs a)
{
    const int F = 2 * a.FW;
    const int64_t blk = blockIdx.x;
    const int i = static_cast<int>(blk % a.B);
    const int64_t pair = blk / a.B;
    const int h = static_cast<int>(pair % a.H);
    const int64_t r = pair / a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    __shared__ float xq[128];
    __shared__ float u[128];
    __shared__ float ph[256];
    __shared__ float pl[64];
    __shared__ float scal[4];

    T* out = static_cast<T*>(a.out) + r * a.os.req + static_cast<int64_t>(i) * a.os.tok +
             static_cast<int64_t>(h) * a.os.head;
    const int slot = a.slot_ids[r];
    if (slot < 0 || slot >= a.num_slots) {
        for (int c = tid; c < a.d; c += kThreads) st_elem(out, c, __builtin_nanf(""));
        return;
    }
    // query head h reads K/V head h / G: its keys, values, W and state
    const int hk = h / a.G, Hk = a.H / a.G;
    const float* rec = a.state + (static_cast<int64_t>(slot) * Hk + hk) * static_cast<int64_t>(a.d + 1) * F;
    const int64_t kbase = r * a.ks.req + static_cast<int64_t>(hk) * a.ks.head;
    const T* q = static_cast<const T*>(a.q) + r * a.qs.req + static_cast<int64_t>(h) * a.qs.head +
                 static_cast<int64_t>(i) * a.qs.tok;
    const T* kb = static_cast<const T*>(a.k) + kbase;
    const T* vb = static_cast<const T*>(a.v) + kbase;
    const T* W = static_cast<const T*>(a.w) + static_cast<int64_t>(hk) * a.wh;

    for (int c = tid; c < a.d; c += kThreads) xq[c] = ld_elem(q, c);
    __syncthreads();

    // xW (one column j per thread) and the block logits (one key j per thread)
    for (int j = tid; j < a.FW; j += kThreads) {
        float acc = 0.0f;
        for (int c = 0; c < a.d; ++c) acc = fmaf(xq[c], ld_elem(W, static_cast<int64_t>(j) * a.d + c), acc);
        u[j] = acc;
    }
    for (int j = tid; j < a.B; j += kThreads) {
        float acc = 0.0f;
        for (int c = 0; c < a.d; ++c) acc = fmaf(xq[c], ld_elem(kb, static_cast<int64_t>(j) * a.ks.tok + c), acc);
        pl[j] = acc * a.scale;
    }
    __syncthreads();

    if (wave < 2) {
        // wave 0: softmax(u) into ph[0, FW); wave 1: softmax(-u) into ph[FW, F)
        const float sg = wave == 0 ? 1.0f : -1.0f;
        float mx = -INFINITY;
        for (int j = lane; j < a.FW; j += 64) mx = fmaxf(mx, sg * u[j]);
        mx = wave_max(mx);
        float sum = 0.0f;
        for (int j = lane; j < a.FW; j += 64) sum += expf(sg * u[j] - mx);
        sum = wave_sum(sum);
        for (int j = lane; j < a.FW; j += 64) ph[wave * a.FW + j] = expf(sg * u[j] - mx) / sum;
    } else if (wave == 2) {
        // row maximum, exponentials and their sum for the block logits
        float m = -INFINITY;
        for (int j = lane; j < a.B; j += 64) m = fmaxf(m, pl[j]);
        m = wave_max(m);
        float l = 0.0f;
        for (int j = lane; j < a.B; j += 64) {
            const float p = expf(pl[j] - m);
            pl[j] = p;
            l += p;
        }
        l = wave_sum(l);
        if (lane == 0) { scal[0] = m; scal[1] = l; }
    }
    __syncthreads();
    if (wave == 0) {
        float den = 0.0f;
        for (int f = lane; f < F; f += 64) den = fmaf(ph[f], rec[static_cast<int64_t>(a.d) * F + f], den);
        den = wave_sum(den);
        if (lane == 0) scal[2] = den;
    }
    __syncthreads();

    float al, be;
    merge_weights(a.gamma[h], scal[0], al, be);
    const float inv = 1.0f / (al * scal[1] + be * scal[2]);
    for (int c = tid; c < a.d; c += kThreads) {
        float num = 0.0f;
        for (int j = 0; j < a.B; ++j) num = fmaf(pl[j], ld_elem(vb, static_cast<int64_t>(j) * a.ks.tok + c), num);
        float lin = 0.0f;
        for (int f = 0; f < F; ++f) lin = fmaf(ph[f], rec[s_offset(f, c, F)], lin);
        st_elem(out, c, (al * num + be * lin) * inv);
    }
}

// ---------------------------------------------------------------------------
// Commit and prefill: one work-group per (request, head, 32-column slice cs of
// S), over the request's B block tokens (commit) or its packed token range
// (prefill). Tokens are taken 16 at a time: phi(k_t) for the chunk into LDS, then each thread
// accumulates its (f, c) entries of sum_t phi(k_t) v_t^T. The slice cs == 0
// work-group also folds sum_t phi(k_t) into Z. Finally a read-modify-write.
// ---------------------------------------------------------------------------
template <typename T, int FW>
__global__ __launch_bounds__(kThreads) void commit_generic_kernel(CommitArgs a)
{
    constexpr int F = 2 * FW;
    constexpr int KPT = F / 8;  // accumulators per thread: f = fg + 8 k
    constexpr int TC = 16;      // tokens per chunk
    const int nslice = a.d / 32;
    const int64_t blk = blockIdx.x;
    const int cs = static_cast<int>(blk % nslice);
    const int64_t pair = blk / nslice;
    const int h = static_cast<int>(pair % a.H);
    const int64_t r = pair / a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = tid & 31, fg = tid >> 5;

    __shared__ float xk[TC][128];
    __shared__ float u[TC][FW];
    __shared__ float ph[TC][F];
    __shared__ float vv[TC][32];

    const int slot = a.slot_ids[r];
    if (slot < 0 || slot >= a.num_slots) return;
    float* rec = a.state + (static_cast<int64_t>(slot) * a.H + h) * static_cast<int64_t>(a.d + 1) * F;
    int64_t first_row;
    int n;
    commit_rows(a, static_cast<int>(r), first_row, n);
    if (n == 0) return;
    const int64_t base = (first_row < 0 ? r * a.ks.req : first_row * a.ks.tok) + static_cast<int64_t>(h) * a.ks.head;
    const T* kb = static_cast<const T*>(a.k) + base;
    const T* vb = static_cast<const T*>(a.v) + base;
    const T* W = static_cast<const T*>(a.w) + static_cast<int64_t>(h) * a.wh;

    float acc[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) acc[k] = 0.0f;
    float zacc = 0.0f;

    for (int t0 = 0; t0 < n; t0 += TC) {
        const int nt = min(TC, n - t0);
        for (int idx = tid; idx < nt * a.d; idx += kThreads) {
            const int tt = idx / a.d, cc = idx % a.d;
            xk[tt][cc] = ld_elem(kb, static_cast<int64_t>(t0 + tt) * a.ks.tok + cc);
        }
        for (int idx = tid; idx < nt * 32; idx += kThreads) {
            const int tt = idx >> 5, cc = idx & 31;
            vv[tt][cc] = ld_elem(vb, static_cast<int64_t>(t0 + tt) * a.ks.tok + cs * 32 + cc);
        }
        __syncthreads();
        for (int idx = tid; idx < nt * FW; idx += kThreads) {
            const int tt = idx / FW, j = idx % FW;
            float s = 0.0f;
            for (int cc = 0; cc < a.d; ++cc) s = fmaf(xk[tt][cc], ld_elem(W, static_cast<int64_t>(j) * a.d + cc), s);
            u[tt][j] = s;
        }
        __syncthreads();
        for (int tt = wave; tt < nt; tt += kThreads / 64) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const float sg = half == 0 ? 1.0f : -1.0f;
                float mx = -INFINITY;
                for (int j = lane; j < FW; j += 64) mx = fmaxf(mx, sg * u[tt][j]);
                mx = wave_max(mx);
                float sum = 0.0f;
                for (int j = lane; j < FW; j += 64) sum += expf(sg * u[tt][j] - mx);
                sum = wave_sum(sum);
                for (int j = lane; j < FW; j += 64) ph[tt][half * FW + j] = expf(sg * u[tt][j] - mx) / sum;
            }
        }
        __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            const float vc = vv[tt][c];
#pragma unroll
            for (int k = 0; k < KPT; ++k) acc[k] = fmaf(ph[tt][fg + 8 * k], vc, acc[k]);
        }
        if (cs == 0) {
            for (int f = tid; f < F; f += kThreads)
                for (int tt = 0; tt < nt; ++tt) zacc += ph[tt][f];
        }
        __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        const int64_t o = s_offset(fg + 8 * k, cs * 32 + c, F);
        rec[o] += acc[k];
    }
    if (cs == 0 && tid < F) rec[static_cast<int64_t>(a.d) * F + tid] += zacc;
}

// ---------------------------------------------------------------------------
// Feature map: one wave per (request, token, head).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void feature_map_generic_kernel(PhiArgs a)
{
    const int F = 2 * a.FW;
    const int64_t blk = blockIdx.x;  // ((r * B) + t) * H + h
    const int h = static_cast<int>(blk % a.H);
    const int64_t rt = blk / a.H;
    const int t = static_cast<int>(rt % a.B);
    const int64_t r = rt / a.B;
    const int lane = threadIdx.x;

    __shared__ float xs[128];
    __shared__ float u[128];
    const T* x = static_cast<const T*>(a.x) + r * a.xs.req + static_cast<int64_t>(t) * a.xs.tok +
                 static_cast<int64_t>(h) * a.xs.head;
    const T* W = static_cast<const T*>(a.w) + static_cast<int64_t>(h) * a.wh;
    for (int c = lane; c < a.d; c += 64) xs[c] = ld_elem(x, c);
    __syncthreads();
    for (int j = lane; j < a.FW; j += 64) {
        float s = 0.0f;
        for (int c = 0; c < a.d; ++c) s = fmaf(xs[c], ld_elem(W, static_cast<int64_t>(j) * a.d + c), s);
        u[j] = s;
    }
    __syncthreads();
    float* out = a.phi + blk * F;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const float sg = half == 0 ? 1.0f : -1.0f;
        float mx = -INFINITY;
        for (int j = lane; j < a.FW; j += 64) mx = fmaxf(mx, sg * u[j]);
        mx = wave_max(mx);
        float sum = 0.0f;
        for (int j = lane; j < a.FW; j += 64) sum += expf(sg * u[j] - mx);
        sum = wave_sum(sum);
        for (int j = lane; j < a.FW; j += 64) out[half * a.FW + j] = expf(sg * u[j] - mx) / sum;
    }
}

}  // namespace

hipError_t launch_forward_generic(const ForwardArgs& a, hipStream_t s)
{
    const int64_t nblk = static_cast<int64_t>(a.R) * a.H * a.B;
    if (a.io == BHA_BF16)
        hipLaunchKernelGGL(forward_generic_kernel<uint16_t>, dim3(static_cast<uint32_t>(nblk)), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(forward_generic_kernel<float>, dim3(static_cast<uint32_t>(nblk)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename T>
static void commit_dispatch(const CommitArgs& a, hipStream_t s, dim3 grid)
{
    switch (a.FW) {
        case 32: hipLaunchKernelGGL((commit_generic_kernel<T, 32>), grid, dim3(kThreads), 0, s, a); break;
        case 64: hipLaunchKernelGGL((commit_generic_kernel<T, 64>), grid, dim3(kThreads), 0, s, a); break;
        default: hipLaunchKernelGGL((commit_generic_kernel<T, 128>), grid, dim3(kThreads), 0, s, a); break;
    }
}

hipError_t launch_commit_generic(const CommitArgs& a, hipStream_t s)
{
    const int64_t nblk = static_cast<int64_t>(a.R) * a.H * (a.d / 32);
    const dim3 grid(static_cast<uint32_t>(nblk));
    if (a.io == BHA_BF16)
        commit_dispatch<uint16_t>(a, s, grid);
    else
        commit_dispatch<float>(a, s, grid);
    return hipGetLastError();
}

hipError_t launch_feature_map_generic(const PhiArgs& a, hipStream_t s)
{
    const int64_t nblk = static_cast<int64_t>(a.R) * a.B * a.H;
    if (a.io == BHA_BF16)
        hipLaunchKernelGGL(feature_map_generic_kernel<uint16_t>, dim3(static_cast<uint32_t>(nblk)), dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL(feature_map_generic_kernel<float>, dim3(static_cast<uint32_t>(nblk)), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace bha
