// Matrix-core feature map (bha_feature_map, bf16 tokens).
#include "mfma_common.hpp"

namespace bha {

namespace {

// ---------------------------------------------------------------------------
// Feature map (bha_feature_map, bf16 tokens)
// ---------------------------------------------------------------------------
// Persistent: units are (tile of 32 D/32 consecutive tokens of the [R][B]
// batch, head), unit u = tile u / H of head u % H, and work-group b takes
// units b, b + NG, ... (NG a multiple of H, so W_h is loaded once). The next
// unit's rows are loaded into registers while the current one is computed.
// A unit's rows go to LDS beside W_h; each wave then takes 32 tokens:
// u^T = W^T X^T on the matrix cores (lane = token, as in the forward) and
// both softmaxes of each token in fp32 (lanes n and n + 32 hold
// halves of token n's logits). phi leaves through the wave's own 32 rows of
// the X tile, which the logits no longer need: a piece of CW features of
// every token at a time is written there from the accumulator layout and read
// back row by row, so each store instruction writes whole CW * 4-byte runs of
// phi rows (the accumulator layout writes 32-byte pieces of 32 rows per
// instruction; measured at 256 x 32 tokens x 16 heads, FW = 64: 40.7 us).
// Roofline: HBM. Algorithmic bytes per (token, head): the row read (2 d) and
// phi written (4 F); W once per head per launch.
// DEV: the rows are stored non-temporal at device scope (buffer stores; see
// kStorePolicy), which the launcher takes at d = 128, FW = 64 (the one shape
// where the buffer offsets keep the kernel in its occupancy step) for up to
// kFmapDevScopeUnitsPerCu units per CU. Measured at 16 heads, B = 32, same
// bits, three alternated runs: 64 requests 8.62-8.69 -> 7.15-7.42 us, 256:
// 19.17-19.54 -> 18.06-18.72 us, 1,024 (16 units per CU): 67.6-67.7 ->
// 74.8-75.2 us (slower).
constexpr int kFmapDevScopeUnitsPerCu = 4;

template <int D, int FW, bool DEV>
__global__ __launch_bounds__(64 * (D / 32)) void feature_map_mfma_kernel(PhiArgs a, int nunits)
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
    const int NG = gridDim.x;  // a multiple of H: every unit of a work-group has its head
    int unit = blockIdx.x;    // tile unit / H of head unit % H
    if (unit >= nunits) return;
    const int h = unit % a.H;
    const int64_t ntok = static_cast<int64_t>(a.R) * a.B;
    WChunks<D, FW, NT> wc;
    wc.load(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(h) * a.wh, tid);
    // a tile's rows, 16 bytes per thread per step (rows past the batch read
    // its last row and are not stored)
    u32x4 xv[TOK * CH / NT];
    auto load_x = [&](int uu) {
        const int64_t tt0 = static_cast<int64_t>(uu / a.H) * TOK;
#pragma unroll
        for (int i = 0; i < TOK * CH / NT; ++i) {
            const int idx = tid + i * NT, row = idx / CH, ch = idx % CH;
            const int64_t tk = tt0 + row < ntok ? tt0 + row : ntok - 1;
            const int64_t r = tk / a.B, t = tk % a.B;
            const uint16_t* src = static_cast<const uint16_t*>(a.x) + r * a.xs.req + t * a.xs.tok +
                                  static_cast<int64_t>(h) * a.xs.head + 8 * ch;
            xv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        }
    };
    // W_h's loads and the first unit's rows go out together; W_h reaches LDS
    // once all have been issued
    load_x(unit);
    wc.template store_rows<C::RS>(Ws, tid);
    for (; unit < nunits; unit += NG) {
        const int64_t t0 = static_cast<int64_t>(unit / a.H) * TOK;
        __syncthreads();  // the previous unit's staged pieces are read
#pragma unroll
        for (int i = 0; i < TOK * CH / NT; ++i) {
            const int idx = tid + i * NT, row = idx / CH, ch = idx % CH;
            *reinterpret_cast<u32x4*>(Xs + row * C::RS + 8 * ch) = xv[i];
        }
        __syncthreads();
        if (unit + NG < nunits) load_x(unit + NG);  // the next unit's rows stream in during this one
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
        float* const prow0 = a.phi + (tw * a.H + h) * F;  // its row of head h
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
                    if (tk < ntok) {
                        const f32x4 x = *reinterpret_cast<const f32x4*>(stage + row * CS + 4 * c4);
                        if constexpr (DEV)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(u32x4, x), wave_buffer(prow0, 32u * a.H * F * 4u),
                                4 * ((row * a.H) * F + hf * FW + c0 + 4 * c4), 0, kStorePolicy<true>);
                        else
                            *reinterpret_cast<f32x4*>(a.phi + (tk * a.H + h) * F + hf * FW + c0 + 4 * c4) = x;
                    }
                }
            }
    }
}

template <int D>
hipError_t feature_map_by_fw(const PhiArgs& a, hipStream_t s)
{
    constexpr int TOK = 32 * (D / 32);
    const int64_t tiles = (static_cast<int64_t>(a.R) * a.B + TOK - 1) / TOK;
    const int nunits = static_cast<int>(tiles * a.H);
    // two waves per SIMD (two four-wave work-groups per CU at d = 128)
    int64_t NG = static_cast<int64_t>(compute_units()) * 2 * 4 / (D / 32);
    NG = (NG / a.H) * a.H;
    if (NG < a.H) NG = a.H;
    if (NG > nunits) NG = nunits;
    const dim3 grid(static_cast<uint32_t>(NG)), block(64 * (D / 32));
    const int nt = nunits;
    // device-scope stores (a wave's 32 rows span 32 H F floats: byte offsets
    // within 31 bits)
    const bool dev = D == 128 && nunits <= static_cast<int64_t>(kFmapDevScopeUnitsPerCu) * compute_units() &&
                     int64_t(32) * a.H * (2 * a.FW) * 4 <= INT32_MAX;
    switch (a.FW) {
        case 32: return launch_kernel(feature_map_mfma_kernel<D, 32, false>, grid, block, s, a, nt);
        case 64:
            return dev ? launch_kernel(feature_map_mfma_kernel<D, 64, true>, grid, block, s, a, nt)
                       : launch_kernel(feature_map_mfma_kernel<D, 64, false>, grid, block, s, a, nt);
        default: return launch_kernel(feature_map_mfma_kernel<D, 128, false>, grid, block, s, a, nt);
    }
}

}  // namespace

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
