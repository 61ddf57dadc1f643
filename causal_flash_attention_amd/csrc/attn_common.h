// Device-side building blocks shared by the attention kernels (gfx950).
//
// MFMA conventions used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   lane l, half h = l / 32, column/row index l % 32
//   A operand (32 x 16): lane holds row l%32, 8 consecutive k (8h .. 8h+7)
//   B operand (16 x 32): lane holds column l%32, the same 8 k
//   C/D (32 x 32, fp32): lane holds column l%32, register i holds row
//                        8*(i/4) + 4h + (i%4)
// Any relabelling of k applied to both A and B leaves the product unchanged;
// the kernels use that freedom to feed a C result back in as a B operand: the
// 16 k of one MFMA step that lane half h supplies are then rows
// {8*(j/4) + 4h + (j%4) : j = 0..7} of the C tile, and the operand that is
// read from LDS is stored with its 16-element chunks permuted to match
// (see perm16 below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int HEAD_DIM = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Padded LDS row: 64 bf16 of data + 8 bf16 of padding (144 bytes), so that
// 16 lanes reading 16 bytes each from 16 consecutive rows hit 64 distinct
// banks.
constexpr int LDS_ROW = 72;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// 16-byte global load (8 bf16) with zero fill when `ok` is false.
__device__ __forceinline__ u32x4 load16(const bf16* p, bool ok) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4*>(p);
    return v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 lds_read8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ void lds_write16(bf16* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

// Round 8 floats to nearest-even bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
    f32x8 v = {a0, a1, a2, a3, a4, a5, a6, a7};
    return __builtin_convertvector(v, bf16x8);
}

// Elements 8*half .. 8*half+7 of a C tile, rounded to bf16: the B operand for
// the 16-row chunk `2*blk + half` of that tile under the k relabelling above.
__device__ __forceinline__ bf16x8 c_rows_to_operand(const f32x16& c, int half) {
    const int o = 8 * half;
    return to_bf16x8(c[o + 0], c[o + 1], c[o + 2], c[o + 3],
                     c[o + 4], c[o + 5], c[o + 6], c[o + 7]);
}

__device__ __forceinline__ u32x2 to_bf16x4_bits(float a0, float a1, float a2, float a3) {
    f32x4 v = {a0, a1, a2, a3};
    bf16x4 b = __builtin_convertvector(v, bf16x4);
    return __builtin_bit_cast(u32x2, b);
}

// Position of element `k` (0..63) of a transposed LDS row: inside each group
// of 16, the 4-element groups are stored in the order 0, 2, 1, 3, so that lane
// half h reads its 8 operand elements {4h..4h+3, 8+4h..8+4h+3} as one
// contiguous 16-byte chunk at offset 8h.
__device__ __forceinline__ int perm16(int k) {
    const int g = (k >> 2) & 3;
    const int pg = ((g & 1) << 1) | (g >> 1);
    return (k & ~15) | (pg << 2) | (k & 3);
}

// Stage one 64 x 64 bf16 tile of rows [r0, r0+64) of a strided matrix into
// LDS. Thread t (of 256) owns rows 2*(t/8) and 2*(t/8)+1, columns 8*(t%8)..+7.
// Rows at or beyond `nrows` read as zero.
struct TilePair {
    u32x4 a;  // row 2p
    u32x4 b;  // row 2p + 1
};

__device__ __forceinline__ TilePair load_tile_pair(const bf16* base, long long row_stride,
                                                   int r0, int nrows, int tid) {
    const int rp = tid >> 3, cc = tid & 7;
    const int ra = r0 + 2 * rp, rb = ra + 1;
    TilePair t;
    t.a = load16(base + (long long)ra * row_stride + cc * 8, ra < nrows);
    t.b = load16(base + (long long)rb * row_stride + cc * 8, rb < nrows);
    return t;
}

// Row-major copy: lds[row][col], padded rows.
__device__ __forceinline__ void store_tile_rows(bf16* lds, const TilePair& t, int tid) {
    const int rp = tid >> 3, cc = tid & 7;
    lds_write16(lds + (2 * rp) * LDS_ROW + cc * 8, t.a);
    lds_write16(lds + (2 * rp + 1) * LDS_ROW + cc * 8, t.b);
}

// Transposed copy: lds[col][perm16(row)], padded rows. Rows 2p and 2p+1 stay
// adjacent under perm16, so each column pair is one 32-bit LDS write.
__device__ __forceinline__ void store_tile_transposed(bf16* lds, const TilePair& t, int tid) {
    const int rp = tid >> 3, cc = tid & 7;
    const int pos = perm16(2 * rp);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const unsigned int wa = t.a[e >> 1], wb = t.b[e >> 1];
        const unsigned int lo = (e & 1) ? (wa >> 16) : (wa & 0xffffu);
        const unsigned int hi = (e & 1) ? (wb >> 16) : (wb & 0xffffu);
        *reinterpret_cast<unsigned int*>(lds + (cc * 8 + e) * LDS_ROW + pos) = lo | (hi << 16);
    }
}

// Value of the other lane half (lane ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
    return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ float fast_exp2(float x) {
    return __builtin_amdgcn_exp2f(x);
}

}  // namespace cattn
