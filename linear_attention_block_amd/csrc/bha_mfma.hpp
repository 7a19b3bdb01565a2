// gfx950 matrix-core and LDS primitives shared by the bf16 kernels: MFMA
// tiles, operand fragments read from LDS, the transposing LDS read and the
// bank-conflict-free layout of tiles read transposed.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace bha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

typedef short i16x4 __attribute__((ext_vector_type(4)));

// gfx950 transposing LDS read (ds_read_b64_tr_b16). Within each group of 16
// lanes, lane k supplies the 8-byte address of row k/4, columns 4(k%4) .. +3 of
// a 4 x 16 block, and receives column k of that block's 4 rows.
__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* p)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// A-operand fragment of V^T for the 32x32x16 product over tokens: lane
// (n, g) = (lane % 32, lane / 32) gets V[j][c0 + n] for
// j = 16 kb + 4 g + {0..3} and 16 kb + 8 + 4 g + {0..3}, from V stored
// row-major (row stride RS elements) in LDS.
template <int RS>
__device__ __forceinline__ bf16x8 vt_frag(const uint16_t* Vs, int c0, int kb, int lane)
{
    const int m = lane & 15, q = lane >> 4, g = lane >> 5;
    const int col = c0 + 16 * (q & 1) + 4 * (m & 3);
    const int row = 16 * kb + 4 * g + (m >> 2);
    const i16x4 lo = lds_read_tr(Vs + row * RS + col);
    const i16x4 hi = lds_read_tr(Vs + (row + 8) * RS + col);
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Tiles read transposed with no padding, stored in 8-byte pieces: piece p of
// row t (RB pieces per row) sits at position p ^ lds_piece_swizzle<RB>(t).
// The swizzle is even, so 16-byte chunks stay whole, and it is chosen for the
// 64 banks of the LDS: the four rows one half-wave's transposed read touches
// fall into four distinct 64-byte bank groups, and the sixteen rows a 16-lane
// group writes at one column land in sixteen distinct pieces.
template <int RB>
__device__ __forceinline__ int lds_piece_swizzle(int t)
{
    return RB >= 32 ? 8 * (t & 3) + 2 * ((t >> 2) & 3) : 8 * ((t >> 1) & 1) + 2 * ((t >> 2) & 3);
}

// vt_frag for a piece-swizzled tile of RB pieces per row.
template <int RB>
__device__ __forceinline__ bf16x8 vt_frag_ps(const uint16_t* Xs, int c0, int kb, int lane)
{
    const int m = lane & 15, q = lane >> 4, g = lane >> 5;
    const int piece = (c0 >> 2) + 4 * (q & 1) + (m & 3);
    const int row = 16 * kb + 4 * g + (m >> 2);
    const i16x4 lo = lds_read_tr(Xs + row * (4 * RB) + ((piece ^ lds_piece_swizzle<RB>(row)) << 2));
    const i16x4 hi = lds_read_tr(Xs + (row + 8) * (4 * RB) + ((piece ^ lds_piece_swizzle<RB>(row + 8)) << 2));
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Row-major tiles of 16-byte chunks read as MFMA fragments (16 rows at one
// chunk index per 16-lane group): chunk ch of row t sits at position
// k_chunk_pos<D>(t, ch), XOR-swizzled so that those 16 rows fall into 16
// distinct 16-byte bank groups (rows of D bf16: 256 bytes at D = 128, 128 at
// D = 64), and the 16 (or 2 x 8) chunks one 16-lane group writes do too.
template <int D>
__device__ __forceinline__ int k_chunk_pos(int t, int ch)
{
    return D == 128 ? (ch ^ (t & 15)) : (ch ^ ((t >> 1) & 7));
}

// v_mfma_f32_16x16x32_bf16: A lane l holds row l % 16, k = 8 (l / 16) .. + 7;
// B lane l holds column l % 16, the same k; C lane l holds column l % 16,
// rows 4 (l / 16) .. + 3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace
}  // namespace bha
