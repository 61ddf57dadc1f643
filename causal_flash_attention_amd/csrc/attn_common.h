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
// {8*(j/4) + 4h + (j%4) : j = 0..7} of the C tile, and the operand read
// from LDS by transposing reads takes the same rows (atile_tr_offsets).
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

// ---------------------------------------------------------------------------
// Asynchronous tiles: 64 rows x 64 bf16, 128-byte rows with no padding,
// filled by direct global->LDS loads (no VGPRs, no LDS write instructions)
// and read either row-major (ds_read_b128) or transposed (ds_read_b64_tr_b16).
// The 16-byte chunk c of row r sits at chunk c ^ swz(r); swz maps r/2 to a
// permutation of 0..7 whose consecutive pairs differ in bit 2, which keeps
// both read patterns free of bank conflicts.
// ---------------------------------------------------------------------------
constexpr int ATILE_ELEMS = 64 * 64;

__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// One direct global->LDS load: 16 bytes from `g` (per lane) to LDS address
// m0 + 16 * lane. Issued from asm so that the compiler does not track it as
// a pending LDS write: otherwise it waits for every such load before each
// transposing LDS read, which would drain the prefetch pipeline. The
// instruction has no output registers; ordering against the readers comes
// from explicit vmcnt waits (wait_vmem) and the workgroup barrier.
__device__ __forceinline__ void lds_dma16(const void* g, unsigned int lds_byte_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_byte_addr)
                 : "memory", "m0");
}

__device__ __forceinline__ unsigned int lds_addr(const void* p) {
    return (unsigned int)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Raw buffer descriptor (stride 0, 32-bit data format) over `num_bytes`
// bytes at `base`: buffer loads at byte offsets past num_bytes return zeros.
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, unsigned int num_bytes) {
    const unsigned long long p = (unsigned long long)(uintptr_t)base;
    i32x4 r;
    r.x = (int)(unsigned int)p;
    r.y = (int)((unsigned int)(p >> 32) & 0xffffu);
    r.z = (int)num_bytes;
    r.w = 0x00020000;
    return r;
}

// One direct buffer->LDS load: 16 bytes per lane from byte offset
// `voff` + `soff` of the buffer to LDS address m0 + 16 * lane, zeros where
// the access lies past the descriptor's range. Issued from asm for the same
// reason as lds_dma16.
__device__ __forceinline__ void lds_dma16_buf(i32x4 rsrc, unsigned int voff, unsigned int soff,
                                              unsigned int lds_byte_addr) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_byte_addr)
                 : "memory", "m0");
}

// Per-lane constants of the tile loads from one strided bf16 matrix. Wave w
// (of 4) loads tile rows 16w .. 16w + 15 with two instructions, each writing
// 8 whole rows (1 KB) at lane-contiguous LDS addresses: lane l moves chunk
// (l & 7) ^ swz(row) of row 16w + 8i + l/8. The byte offsets need
// 64 * row_stride * 2 < 2^32 (the host checks the channel count).
struct TileLoader {
    unsigned int voff[2];  // byte offset of the lane's chunk from the tile's first row
    unsigned int lds[2];   // byte offset of the instruction's rows within a tile
};

__device__ __forceinline__ TileLoader tile_loader(long long row_stride, int wave, int lane) {
    TileLoader L;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tr = 16 * wave + 8 * i + (lane >> 3);
        const int col = ((lane & 7) ^ swz(tr)) * 8;
        L.voff[i] = (unsigned int)(((long long)tr * row_stride + col) * 2);
        L.lds[i] = __builtin_amdgcn_readfirstlane((unsigned int)(16 * wave + 8 * i) * 128u);
    }
    return L;
}

// Descriptor over rows [r0, nrows) of a strided bf16 matrix (row stride
// `row_stride` elements, nrows > r0): loads of rows past the matrix return
// zeros (callers mask or zero-weight them).
__device__ __forceinline__ i32x4 rows_rsrc(const bf16* base, long long row_stride, int r0,
                                           int nrows) {
    const unsigned long long bytes = (unsigned long long)(nrows - r0) * row_stride * 2;
    return buffer_rsrc(base + (long long)r0 * row_stride,
                       bytes > 0xffffffffull ? 0xffffffffu : (unsigned int)bytes);
}

// Issue the loads of the 64 rows of a descriptor from rows_rsrc into the LDS
// tile at byte address `lds_tile`; `soff` (bytes) selects columns further
// along the same rows (V next to K in the packed qkv rows). A row is in range
// when its offset without `soff` is, and also with it, since soff + 128
// bytes stays within one row.
__device__ __forceinline__ void atile_load(unsigned int lds_tile, i32x4 rsrc, unsigned int soff,
                                           const TileLoader& L) {
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16_buf(rsrc, L.voff[i], soff, lds_tile + L.lds[i]);
}

// Wave-uniform LDS byte address of a tile.
__device__ __forceinline__ unsigned int atile_addr(const bf16* tile) {
    return __builtin_amdgcn_readfirstlane(lds_addr(tile));
}

// LDS address of a tile as seen by its readers. The direct loads above write
// a whole wave's 1 KB per instruction, but the compiler models them as
// writing only the 16 bytes at the base it is given, and would otherwise fold
// reads of the rest of the tile to undefined values. Passing the address
// through an empty asm statement (after the barrier that publishes the tile)
// hides where it points.
typedef __attribute__((address_space(3))) const bf16 lds_bf16;

__device__ __forceinline__ lds_bf16* atile_view(const bf16* tile) {
    unsigned int a = (unsigned int)(uintptr_t)(lds_bf16*)tile;
    asm volatile("" : "+v"(a));
    return (lds_bf16*)(uintptr_t)a;
}

// The same for a tile given by its LDS byte address.
__device__ __forceinline__ lds_bf16* atile_view_at(unsigned int a) {
    asm volatile("" : "+v"(a));
    return (lds_bf16*)(uintptr_t)a;
}

// Row-major operand: 8 bf16 of tile row r, logical 16-byte chunk c.
__device__ __forceinline__ bf16x8 atile_row(lds_bf16* tile, int r, int c) {
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
    return *reinterpret_cast<lds_bf16x8*>(tile + r * 64 + ((c ^ swz(r)) << 3));
}


// Offsets (in bf16 elements) of the two transposed reads that build the
// A operand X^T (rows d = 32*db + l%32, k = tile rows 16*kc + {4h..4h+3,
// 8+4h..8+4h+3}) for kc = 0; add 16*64*kc for other chunks (swz is periodic
// in 16 rows). ds_read_b64_tr_b16 hands lane i of each 16-lane group element
// (i % 4) of the 8-byte pieces addressed by lanes i/4, 4 + i/4, 8 + i/4 and
// 12 + i/4 of that group, so lane i addresses row 4h + i/4 at columns
// 32*db + 16*((l/16)%2) + 4*(i%4).
__device__ __forceinline__ void atile_tr_offsets(int lane, int db, int* off0, int* off1) {
    const int i = lane & 15, grp = lane >> 4, h = grp >> 1;
    const int d = db * 32 + 16 * (grp & 1) + 4 * (i & 3);
    const int r0 = 4 * h + (i >> 2), r1 = r0 + 8;
    *off0 = r0 * 64 + (((d >> 3) ^ swz(r0)) << 3) + (d & 7);
    *off1 = r1 * 64 + (((d >> 3) ^ swz(r1)) << 3) + (d & 7);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// A operand X^T of chunk kc through the transposing-read intrinsic: the
// compiler tracks these reads and waits for each only where it is used.
__device__ __forceinline__ bf16x8 atile_tr(lds_bf16* tile, int off0, int off1, int kc) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + kc * 16 * 64 + off0));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + kc * 16 * 64 + off1));
    const i16x4 v[2] = {a, b};
    return __builtin_bit_cast(bf16x8, v);
}

// Wait until at most n of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Value of the other lane half (lane ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
    return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ float fast_exp2(float x) {
    return __builtin_amdgcn_exp2f(x);
}

}  // namespace cattn
