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
// Commit and prefill: one work-group of 512 threads per (request, head), over
// the request's B block tokens (commit) or its packed token range (prefill),
// 16 tokens at a time. W is staged once in LDS (rows padded by one float, so
// the 64 rows a wave reads at one column fall in distinct banks). Per chunk:
// the K and V rows to LDS, the feature logits u = k W^T (a wave takes one
// token's logits), phi(k) per token (a wave per token and half), then thread
// (column c, feature group fg) adds phi(k_t)[f] v_t[c] for its contiguous run
// of features f and, for f < F, the Z sums. Finally one read-modify-write of
// the record.
// ---------------------------------------------------------------------------
constexpr int kCommitThreads = 512;

template <typename T, int D, int FW>
__global__ __launch_bounds__(kCommitThreads) void commit_generic_kernel(CommitArgs a)
{
    constexpr int F = 2 * FW;
    constexpr int NT = kCommitThreads;
    constexpr int TC = 16;        // tokens per chunk
    constexpr int WS = D + 1;     // padded W row (floats)
    constexpr int NG = NT / D;    // feature groups: 4 at d = 128, 8 at d = 64
    constexpr int KPT = F / NG;   // accumulators per thread: f = fg KPT .. + KPT - 1
    const int pair = blockIdx.x;
    const int h = pair % a.H, r = pair / a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = tid % D, fg = tid / D;

    __shared__ float Ws[FW * WS];
    __shared__ float xk[TC * D];
    __shared__ float xv[TC * D];
    __shared__ float u[TC * FW];
    __shared__ __attribute__((aligned(16))) float ph[TC * F];

    const int slot = a.slot_ids[r];
    if (slot < 0 || slot >= a.num_slots) return;
    int64_t first_row;
    int n;
    commit_rows(a, r, first_row, n);
    if (n == 0) return;
    float* rec = a.state + (static_cast<int64_t>(slot) * a.H + h) * static_cast<int64_t>(D + 1) * F;
    const int64_t base = (first_row < 0 ? static_cast<int64_t>(r) * a.ks.req : first_row * a.ks.tok) +
                         static_cast<int64_t>(h) * a.ks.head;
    const T* kb = static_cast<const T*>(a.k) + base;
    const T* vb = static_cast<const T*>(a.v) + base;
    const T* W = static_cast<const T*>(a.w) + static_cast<int64_t>(h) * a.wh;
    for (int idx = tid; idx < FW * D; idx += NT) Ws[(idx / D) * WS + idx % D] = ld_elem(W, idx);

    float acc[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) acc[k] = 0.0f;
    float zacc = 0.0f;

    for (int t0 = 0; t0 < n; t0 += TC) {
        const int nt = n - t0 < TC ? n - t0 : TC;
        __syncthreads();  // W staged; every thread is done with the previous chunk
        for (int idx = tid; idx < nt * D; idx += NT) {
            const int tt = idx / D, cc = idx % D;
            const int64_t o = static_cast<int64_t>(t0 + tt) * a.ks.tok + cc;
            xk[idx] = ld_elem(kb, o);
            xv[idx] = ld_elem(vb, o);
        }
        __syncthreads();
        for (int idx = tid; idx < nt * FW; idx += NT) {
            const int tt = idx / FW, j = idx % FW;
            const float* kr = xk + tt * D;
            const float* wr = Ws + j * WS;
            float sdot = 0.0f;
#pragma unroll 8
            for (int cc = 0; cc < D; ++cc) sdot = fmaf(kr[cc], wr[cc], sdot);
            u[idx] = sdot;
        }
        __syncthreads();
        for (int th = wave; th < 2 * nt; th += NT / 64) {
            const int tt = th >> 1, half = th & 1;
            const float sg = half == 0 ? 1.0f : -1.0f;
            float mx = -INFINITY;
            for (int j = lane; j < FW; j += 64) mx = fmaxf(mx, sg * u[tt * FW + j]);
            mx = wave_max(mx);
            float sum = 0.0f;
            for (int j = lane; j < FW; j += 64) sum += expf(sg * u[tt * FW + j] - mx);
            sum = wave_sum(sum);
            for (int j = lane; j < FW; j += 64) ph[tt * F + half * FW + j] = expf(sg * u[tt * FW + j] - mx) / sum;
        }
        __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            const float vc = xv[tt * D + c];
            const float4* pr = reinterpret_cast<const float4*>(ph + tt * F + fg * KPT);
#pragma unroll
            for (int k4 = 0; k4 < KPT / 4; ++k4) {
                const float4 p4 = pr[k4];
                acc[4 * k4] = fmaf(p4.x, vc, acc[4 * k4]);
                acc[4 * k4 + 1] = fmaf(p4.y, vc, acc[4 * k4 + 1]);
                acc[4 * k4 + 2] = fmaf(p4.z, vc, acc[4 * k4 + 2]);
                acc[4 * k4 + 3] = fmaf(p4.w, vc, acc[4 * k4 + 3]);
            }
        }
        if (tid < F)
            for (int tt = 0; tt < nt; ++tt) zacc += ph[tt * F + tid];
    }
#pragma unroll
    for (int k = 0; k < KPT; ++k) rec[s_offset(fg * KPT + k, c, F)] += acc[k];
    if (tid < F) rec[static_cast<int64_t>(D) * F + tid] += zacc;
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

template <typename T, int D>
static void commit_dispatch(const CommitArgs& a, hipStream_t s, dim3 grid)
{
    switch (a.FW) {
        case 32: hipLaunchKernelGGL((commit_generic_kernel<T, D, 32>), grid, dim3(kCommitThreads), 0, s, a); break;
        case 64: hipLaunchKernelGGL((commit_generic_kernel<T, D, 64>), grid, dim3(kCommitThreads), 0, s, a); break;
        default: hipLaunchKernelGGL((commit_generic_kernel<T, D, 128>), grid, dim3(kCommitThreads), 0, s, a); break;
    }
}

hipError_t launch_commit_generic(const CommitArgs& a, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.R) * a.H));
    if (a.io == BHA_BF16) {
        if (a.d == 128) commit_dispatch<uint16_t, 128>(a, s, grid);
        else commit_dispatch<uint16_t, 64>(a, s, grid);
    } else {
        if (a.d == 128) commit_dispatch<float, 128>(a, s, grid);
        else commit_dispatch<float, 64>(a, s, grid);
    }
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
