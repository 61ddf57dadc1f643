// Causal attention forward in FP8: MXFP8 operands (OCP E4M3 elements with one
// power-of-two E8M0 scale per 32 elements), fp32 accumulation, on the scaled
// MFMA of gfx950 (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// The llm.c page ("Réimplémenter à bas coût le modèle GPT-2 avec llm.c",
// FAQ) lists FP8 training as planned without a recipe. The variant here:
//   - each block of 32 elements gets the smallest scale 2^e with
//     max|x| <= 448 * 2^e (so no element saturates), elements round to
//     nearest-even E4M3;
//   - Q and K are blocked along channels (the contraction of Q K^T), V along
//     positions (the contraction of P V), V stored transposed;
//   - per query row, with base-2 logits z and an integer reference m =
//     ceil(max z), the probabilities enter P V as E4M3(2^(z - m + 8)) with
//     the fixed scale 2^-8; their sum (taken on the MFMA from the same codes)
//     normalises O, and LSE = ln 2 (m + log2 sum).
// The kernel keeps a running integer reference that only grows, so every
// rescale is an exact power of two and, E4M3 rounding commuting with powers
// of two in its normal range, the codes match those of the final reference
// apart from probabilities below 2^-13 and float32 rounding ties.
//
// FP8 buffer (one call, BH = batch * heads, Tp = round_up(T, 64), NT = Tp/64):
//   [0, BH Tp 64)            Q codes  [BH][Tp][64 channels]
//   [BH Tp 64, 2 BH Tp 64)   K codes  [BH][Tp][64 channels]
//   [2 BH Tp 64, 3 BH Tp 64) V codes  [BH][64 channels][Tp]   (transposed)
//   [3 BH Tp 64, + BH NT 384) exponent bytes e + 127 per tile of 64 positions:
//        [0, 128)   Q: position p of the tile, channel block b at 2p + b
//        [128, 256) K: likewise
//        [256, 384) V: position block b (of 2) of the tile, channel c at 64b + c
// Positions in [T, Tp) hold zero codes and exponent byte 0.
#include "attn_fp8_common.h"

#ifndef CATTN_FP8_WAVES_PER_SIMD
#define CATTN_FP8_WAVES_PER_SIMD 1
#endif

namespace cattn {
namespace {

// Workgroup bh * NT + t: tile t of 64 positions of batch * head bh. Q and K blocks of
// 32 channels (thread: position tid/4, channels 16 (tid%4) ..), then V blocks
// of 32 positions (thread: channel tid/4, positions 16 (tid%4) ..) through a
// float copy of the tile in LDS.
__global__ __launch_bounds__(256) void attn_quantize_fp8_kernel(const bf16* __restrict__ qkv,
                                                                u8* __restrict__ buf, int T, int H,
                                                                Fp8Layout L) {
    __shared__ float vt[64][65];
    const int bh = blockIdx.x / L.NT, t = blockIdx.x - bh * L.NT, b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x;
    const int C = H * HEAD_DIM;
    const long long rs = 3LL * C;
    const int p = tid >> 2, cq = tid & 3;
    const int pos = t * 64 + p;
    const bool valid = pos < T;
    const bf16* row = qkv + ((long long)b * T + (valid ? pos : 0)) * rs + h * HEAD_DIM + 16 * cq;
    u8* ex = buf + L.e + ((long long)bh * L.NT + t) * F8_EXP_TILE;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        float x[16];
        bf16x16_to_f32(row + m * C, valid, x);
        u32x4 codes;
        const int e = quantize16(x, codes);
        u8* dst = buf + (m == 0 ? 0 : L.k) + ((long long)bh * L.Tp + pos) * 64 + 16 * cq;
        *reinterpret_cast<u32x4*>(dst) = codes;
        if ((cq & 1) == 0) ex[128 * m + 2 * p + (cq >> 1)] = (u8)(e + 127);
    }
    {
        float x[16];
        bf16x16_to_f32(row + 2 * C, valid, x);
#pragma unroll
        for (int i = 0; i < 16; ++i) vt[p][16 * cq + i] = x[i];
    }
    __syncthreads();
    const int c = tid >> 2, pq = tid & 3;
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = vt[16 * pq + i][c];
    u32x4 codes;
    const int e = quantize16(y, codes);
    *reinterpret_cast<u32x4*>(buf + L.v + ((long long)bh * 64 + c) * L.Tp + t * 64 + 16 * pq) =
        codes;
    if ((pq & 1) == 0) ex[256 + 64 * (pq >> 1) + c] = (u8)(e + 127);
}

// ---------------------------------------------------------------------------
// Forward
//
// Operands follow the scaled-MFMA layout described in attn_fp8_common.h.
//
// S^T = K Q^T per 32-key block kb: A = K rows, B = Q^T; A row r is key
// 32 kb + key_of_row(r), which makes register i of a lane half h hold key
// 32 kb + 16h + i, so a lane's 16 + 16 scores are exactly the keys that the
// same lane must supply as the B operand P^T of O^T = V^T P^T.
// ---------------------------------------------------------------------------
constexpr int FWD_BM = 128;  // queries per workgroup (32 per wave)
constexpr int FWD_BN = 64;   // keys per tile
// Tile j + 2 is issued during step j, into the stage that tile j - 1 has left.
constexpr int PREFETCH = 2;
constexpr int NSTAGE = PREFETCH + 1;

struct Fp8Smem {
    u8 k[NSTAGE][64 * 64];  // K codes [key][channel], 16-byte chunks swizzled by swz_k
    u8 v[NSTAGE][64 * 64];  // V codes [channel][key], chunks swizzled by swz_v
    u8 e[NSTAGE][256];      // the tile's K exponents (128 bytes), then its V exponents
};

// Per-lane LDS offsets of one wave's operands.
struct F8Offsets {
    int k[2][2];  // K rows of block kb, chunks h and 2 + h
    int v[2][2];  // V rows (channels) of block db, chunks h and 2 + h
    int ek[2];    // K exponent of the lane's key in block kb, channel block h
    int ev[2];    // V exponent of channel 32 db + r, position block h
};

__device__ __forceinline__ F8Offsets f8_offsets(int l32, int hf) {
    F8Offsets o;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + key_of_row(l32);
        o.k[kb][0] = row * 64 + 16 * (hf ^ swz_k(row));
        o.k[kb][1] = row * 64 + 16 * ((2 + hf) ^ swz_k(row));
        o.ek[kb] = 2 * row + hf;
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        const int ch = 32 * db + l32;
        o.v[db][0] = ch * 64 + 16 * (hf ^ swz_v(ch));
        o.v[db][1] = ch * 64 + 16 * ((2 + hf) ^ swz_v(ch));
        o.ev[db] = 128 + 64 * hf + ch;
    }
    return o;
}

// S^T of one 64-key tile: two scaled MFMAs (one per 32-key block).
__device__ __forceinline__ void scores_f8(lds_u8* kt, lds_u8* et, const F8Offsets& o,
                                          const i32x8& qop, int qs, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_f8(lds_operand(kt, o.k[kb]), qop, zero16(), et[o.ek[kb]], qs);
}

// Register i of block kb holds key k0 + 32 kb + 16 h + i against query
// qw + r; `lim` = qw - k0 + r - 16 h.
__device__ __forceinline__ void mask_f8(f32x16 (&s)[2], int lim) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (32 * kb + i > lim) s[kb][i] = -INFINITY;
}

__device__ __forceinline__ float tile_max_f8(const f32x16 (&s)[2]) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    return fmaxf(mx, swap_halves(mx));
}

// Raise the integer reference to ceil(tile max) where that is larger; the
// accumulators scale by 2^(old - new), exactly (0 on the first tile).
__device__ __forceinline__ void update_ref(float zmax, float& m_run, f32x16 (&acc)[2],
                                           f32x16& lsum) {
    const float mt = ceilf(zmax);
    const bool grow = mt > m_run;
    if (__any(grow)) {
        asm volatile("");
        const float alpha = grow ? fast_exp2(m_run - mt) : 1.0f;
        m_run = grow ? mt : m_run;
        lsum[0] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
}

__global__ __launch_bounds__(256, CATTN_FP8_WAVES_PER_SIMD) void attn_fwd_fp8_kernel(
    const u8* __restrict__ buf, bf16* __restrict__ out, float* __restrict__ lse, int B, int T,
    int H, int n_qt, Fp8Layout L, float c_log2) {
    __shared__ Fp8Smem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;

    // Workgroup -> (query tile, head), heaviest first, heads grouped by XCD.
    const int BH = B * H;
    const int blk = blockIdx.x;
    int qt, bh;
    if ((BH & 7) == 0) {
        const int per = BH >> 3, xcd = blk & 7, s = blk >> 3;
        qt = n_qt - 1 - s / per;
        bh = xcd * per + s % per;
    } else {
        qt = n_qt - 1 - blk / BH;
        bh = blk % BH;
    }
    const int b = bh / H, h = bh - b * H;
    const int C = H * HEAD_DIM;
    const int Tp = L.Tp;

    const u8* qcodes = buf + (long long)bh * Tp * 64;
    const u8* kcodes = buf + L.k + (long long)bh * Tp * 64;
    const u8* vcodes = buf + L.v + (long long)bh * 64 * Tp;
    const u8* exps = buf + L.e + (long long)bh * L.NT * F8_EXP_TILE;
    const i32x4 rs_k = buffer_rsrc(kcodes, (unsigned int)(Tp * 64));
    const i32x4 rs_v = buffer_rsrc(vcodes, (unsigned int)(Tp * 64));
    const i32x4 rs_e = buffer_rsrc(exps, (unsigned int)(L.NT * F8_EXP_TILE));

    const int q0 = qt * FWD_BM;
    const int qw = q0 + wave * 32;
    const int kend = min(q0 + FWD_BM, T);
    const int n_kt = (kend + FWD_BN - 1) / FWD_BN;
    const int j_last = min((qw + 31) / FWD_BN, n_kt - 1);

    // Direct loads: wave w moves K rows 16w .. 16w + 15 and V channels
    // 16w .. 16w + 15 of a tile (lane l: row 16w + l/4, stored chunk l%4);
    // lanes 0..15 of wave 0 move the tile's 256 exponent bytes.
    const int lrow = 16 * wave + (lane >> 2), lpos = lane & 3;
    const unsigned int voff_k = (unsigned int)(lrow * 64 + 16 * (lpos ^ swz_k(lrow)));
    const unsigned int voff_v = (unsigned int)(lrow * Tp + 16 * (lpos ^ swz_v(lrow)));
    const unsigned int voff_e = (unsigned int)(16 * lane);
    const unsigned int wave_lds = __builtin_amdgcn_readfirstlane((unsigned int)(1024 * wave));
    // Wave-uniform LDS byte addresses of stage 0; stage st sits st stages on.
    const unsigned int k_l = lds_addr_u(sm.k[0]), v_l = lds_addr_u(sm.v[0]), e_l = lds_addr_u(sm.e[0]);
    constexpr unsigned int K_ST = sizeof(sm.k[0]), V_ST = sizeof(sm.v[0]), E_ST = sizeof(sm.e[0]);
    auto issue = [&](int j) {
        const unsigned int st = (unsigned int)j % NSTAGE;
        lds_dma16_buf(rs_k, voff_k, (unsigned int)(j * 64 * 64), k_l + st * K_ST + wave_lds);
        lds_dma16_buf(rs_v, voff_v, (unsigned int)(j * 64), v_l + st * V_ST + wave_lds);
        if (wave == 0 && lane < 16)
            lds_dma16_buf(rs_e, voff_e, (unsigned int)(j * F8_EXP_TILE + 128), e_l + st * E_ST);
    };
#pragma unroll
    for (int j = 0; j < PREFETCH; ++j)
        if (j < n_kt) issue(j);

    // Q^T operand (B of S^T): channels [16h, 16h + 16) and [32 + 16h, +16) of
    // this lane's query, with the exponent of channel block h.
    i32x8 qop;
    int qs = 0;
    {
        const int q = qw + l32;
        const bool ok = q < Tp;
        const u8* p = qcodes + (long long)(ok ? q : 0) * 64;
        const u32x4 a = ok ? *reinterpret_cast<const u32x4*>(p + 16 * hf) : u32x4{0u, 0u, 0u, 0u};
        const u32x4 c = ok ? *reinterpret_cast<const u32x4*>(p + 32 + 16 * hf) : u32x4{0u, 0u, 0u, 0u};
        qop = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
        if (ok) qs = exps[(q >> 6) * F8_EXP_TILE + 2 * (q & 63) + hf];
    }
    const unsigned int one_word = l32 == 0 ? E4M3_ONES : 0u;
    const i32x8 ones = {(int)one_word, (int)one_word, (int)one_word, (int)one_word,
                        (int)one_word, (int)one_word, (int)one_word, (int)one_word};
    const F8Offsets o = f8_offsets(l32, hf);
    wait_vmem<0>();
    __syncthreads();

    // One tile per step: scores, reference update, probabilities, then the
    // P V and row-sum products. (Overlapping the scores of tile j + 1 with the
    // exponentials of tile j needs 32 more registers per lane, which drops
    // the kernel to two waves per SIMD and measured slower than three.)
    float m_run = -INFINITY;                 // integer reference of base-2 logits
    f32x16 acc[2] = {zero16(), zero16()};    // O^T per channel block
    f32x16 lsum = zero16();                  // row 0: sum of the probabilities
    for (int j = 0; j < n_kt; ++j) {
        // Tile j must have landed; the loads of tile j + 1 may stay in flight
        // (each wave issues two per tile, wave 0 a third).
        if (j >= 1 && j + 1 < n_kt) {
            if (wave == 0) wait_vmem<3>();
            else wait_vmem<2>();
        } else {
            wait_vmem<0>();
        }
        __syncthreads();
        if (j + PREFETCH < n_kt) issue(j + PREFETCH);
        if (j > j_last) continue;  // tiles above this wave's diagonal
        const unsigned int st = (unsigned int)j % NSTAGE;
        lds_u8* kt = lds_view_at(k_l + st * K_ST);
        lds_u8* vt = lds_view_at(v_l + st * V_ST);
        lds_u8* et = lds_view_at(e_l + st * E_ST);
        f32x16 s[2];
        scores_f8(kt, et, o, qop, qs, s);
        const i32x8 va = lds_operand(vt, o.v[0]);
        const i32x8 vb = lds_operand(vt, o.v[1]);
        const int vsa = et[o.ev[0]], vsb = et[o.ev[1]];
        if (j == j_last) mask_f8(s, qw - j * FWD_BN + l32 - 16 * hf);
        update_ref(tile_max_f8(s) * c_log2, m_run, acc, lsum);
        const float m8 = m_run - 8.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(fmaf(s[kb][i], c_log2, -m8));
        const i32x8 pop = p_operand(s);
        acc[0] = mfma_f8(va, pop, acc[0], vsa, P_SCALE);
        acc[1] = mfma_f8(vb, pop, acc[1], vsb, P_SCALE);
        lsum = mfma_f8(ones, pop, lsum, ONE_SCALE, P_SCALE);
    }

    // O = acc / l (bf16), LSE = ln 2 (m + log2 l); row 0 of lsum lives in half 0.
    const int q = qw + l32;
    const float l_tot = lsum[0] + swap_halves(lsum[0]);
    const float inv = 1.0f / l_tot;
    if (q < T) {
        bf16* op = out + ((long long)b * T + q) * C + h * HEAD_DIM;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * hf;
                *reinterpret_cast<u32x2*>(op + d) =
                    to_bf16x4_bits(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
                                   acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
            }
        if (hf == 0) lse[(long long)bh * T + q] = (m_run + log2f(l_tot)) * LN2;
    }
}

}  // namespace

long long fp8_buffer_bytes(int B, int T, int H) {
    const Fp8Layout L = fp8_layout(B, T, H);
    return L.e + (long long)B * H * L.NT * F8_EXP_TILE;
}

hipError_t launch_attn_quantize_fp8(const void* qkv, void* buf, int B, int T, int H,
                                    hipStream_t stream) {
    const Fp8Layout L = fp8_layout(B, T, H);
    const long long blocks = (long long)B * H * L.NT;
    hipLaunchKernelGGL(attn_quantize_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16*>(qkv), static_cast<u8*>(buf), T, H, L);
    return hipGetLastError();
}

hipError_t launch_attn_fwd_fp8(const void* buf, void* out, float* lse, int B, int T, int H,
                               hipStream_t stream) {
    const Fp8Layout L = fp8_layout(B, T, H);
    const int n_qt = (T + FWD_BM - 1) / FWD_BM;
    const long long blocks = (long long)B * H * n_qt;
    hipLaunchKernelGGL(attn_fwd_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u8*>(buf), static_cast<bf16*>(out), lse, B, T, H, n_qt, L,
                       LOG2E / 8.0f);
    return hipGetLastError();
}

}  // namespace cattn
