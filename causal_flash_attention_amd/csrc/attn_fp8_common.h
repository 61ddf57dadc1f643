// FP8 (MXFP8) building blocks shared by the FP8 forward and backward
// kernels (gfx950): E4M3 codes with E8M0 block exponents, the block-scale
// rule, and the operand layout of the scaled 32x32x64 MFMA with 8-bit
// operands (checked on the hardware): lane (r = l%32, half h = l/32) holds 32
// bytes; byte j of half h meets byte j of the other operand's lane of the
// same half, and bytes 0..15 of both halves form one 32-element scale block
// whose E8M0 scale comes from the half-0 lane, bytes 16..31 the other block,
// scaled by the half-1 lane. So lane (r, h) carries elements [16h, 16h + 16)
// and [32 + 16h, +16) of a 64-long contraction, and the scale of block h.
#pragma once

#include "attn_common.h"

namespace cattn {
namespace {

typedef unsigned char u8;
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int F8_EXP_TILE = 384;
constexpr int P_SCALE = 127 - 8;  // E8M0 byte of 2^-8: probabilities enter as 2^8 p
constexpr int ONE_SCALE = 127;    // E8M0 byte of 1
constexpr unsigned int E4M3_ONES = 0x38383838u;  // four E4M3 1.0

struct Fp8Layout {
    long long k, v, e;  // byte offsets of the K codes, V codes and exponents
    int Tp, NT;
};

Fp8Layout fp8_layout(int B, int T, int H) {
    Fp8Layout L;
    L.Tp = (T + 63) / 64 * 64;
    L.NT = L.Tp / 64;
    const long long codes = (long long)B * H * L.Tp * 64;
    L.k = codes;
    L.v = 2 * codes;
    L.e = 3 * codes;
    return L;
}

// ---------------------------------------------------------------------------
// Quantization
// ---------------------------------------------------------------------------

// Exponent of a block whose largest magnitude is `amax`: the smallest e with
// amax <= 448 * 2^e, clamped to [-127, 127]. With amax = f 2^E, f in [1, 2),
// 448 * 2^(E - 8) = 1.75 * 2^E, so e = E - 8, plus one when f > 1.75. A zero
// block, or one below 2^-126, takes -127 (no element then exceeds 448 either).
__device__ __forceinline__ int mx_exponent(float amax) {
    const unsigned int bits = __float_as_uint(amax);
    const int ef = (int)((bits >> 23) & 0xffu);
    if (ef == 0) return -127;
    const int e = ef - 127 - 8 + ((bits & 0x7fffffu) > 0x600000u ? 1 : 0);
    return e < -127 ? -127 : e;
}

// Four E4M3 codes (round to nearest even) of x[0..3] * 2^-e in one dword,
// x[0] in the low byte. Multiplying by a power of two is exact here.
__device__ __forceinline__ unsigned int e4m3x4(const float* x, int e) {
    int d = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[0], -e), ldexpf(x[1], -e), 0, false);
    d = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[2], -e), ldexpf(x[3], -e), d, true);
    return (unsigned int)d;
}

__device__ __forceinline__ void bf16x16_to_f32(const bf16* p, bool ok, float* x) {
    const bf16x8 a = as_bf16x8(load16(p, ok));
    const bf16x8 b = as_bf16x8(load16(p + 8, ok));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[i] = (float)a[i];
        x[8 + i] = (float)b[i];
    }
}

// 16 codes of one thread and the exponent of its 32-element block, whose
// other half sits in the neighbouring lane (lane ^ 1).
__device__ __forceinline__ int quantize16(const float* x, u32x4& codes) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    const int e = mx_exponent(amax);
#pragma unroll
    for (int w = 0; w < 4; ++w) codes[w] = e4m3x4(x + 4 * w, e);
    return e;
}

__device__ __forceinline__ int key_of_row(int r) {
    return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}
// Chunk swizzles: the 16 lanes of a read phase hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz_k(int row) { return ((row >> 2) & 1) | ((row >> 3) & 2); }
__device__ __forceinline__ int swz_v(int ch) { return (ch >> 2) & 3; }

typedef __attribute__((address_space(3))) const u8 lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

__device__ __forceinline__ lds_u8* lds_view(const u8* p) {
    unsigned int a = (unsigned int)(uintptr_t)(lds_u8*)p;
    asm volatile("" : "+v"(a));
    return (lds_u8*)(uintptr_t)a;
}

// The same for a tile given by its LDS byte address.
__device__ __forceinline__ lds_u8* lds_view_at(unsigned int a) {
    asm volatile("" : "+v"(a));
    return (lds_u8*)(uintptr_t)a;
}

__device__ __forceinline__ unsigned int lds_addr_u(const u8* p) {
    return __builtin_amdgcn_readfirstlane((unsigned int)(uintptr_t)(lds_u8*)p);
}

__device__ __forceinline__ i32x8 lds_operand(lds_u8* tile, const int (&off)[2]) {
    const u32x4 a = *reinterpret_cast<lds_u32x4*>(tile + off[0]);
    const u32x4 b = *reinterpret_cast<lds_u32x4*>(tile + off[1]);
    const i32x8 r = {(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                     (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    return r;
}

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c, int scale_a, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

// E4M3 codes of 2^8 p for the 32 keys of a lane: the B operand P^T.
__device__ __forceinline__ i32x8 p_operand(const f32x16 (&x)[2]) {
    i32x8 r;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // Both halves of the word are written, so its old value does not
            // matter: an empty asm output names a register without setting it.
            int old;
            asm volatile("" : "=v"(old));
            int d = __builtin_amdgcn_cvt_pk_fp8_f32(x[kb][4 * w], x[kb][4 * w + 1], old, false);
            d = __builtin_amdgcn_cvt_pk_fp8_f32(x[kb][4 * w + 2], x[kb][4 * w + 3], d, true);
            r[4 * kb + w] = d;
        }
    return r;
}

}  // namespace
}  // namespace cattn
