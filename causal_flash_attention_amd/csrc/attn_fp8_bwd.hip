// Causal attention backward in FP8 (MXFP8 operands, fp32 accumulation) on the
// scaled MFMA of gfx950, the backward of the FP8 forward variant (the llm.c
// page, "Réimplémenter à bas coût le modèle GPT-2 avec llm.c", FAQ, has FP8
// training planned without a recipe).
//
// Every product takes E4M3 operands blocked along its own contraction:
//   S = Q K^T and dP = dO V^T  over channels (Q, K from the forward's FP8
//                              buffer; V, dO blocked along channels here)
//   dV = P^T dO, dK = dS^T Q   over queries (dO, Q blocked along positions)
//   dQ = dS K                  over keys    (K blocked along positions)
// with P = 2^(z - LSE log2 e) entering dV on the forward's fixed 2^-8 grid,
// D = rowsum(dO * O), dS = P (dP - D), and dS quantized on the fly per block
// of 32 queries (for dK) or 32 keys (for dQ) with the forward's block-scale
// rule (smallest e with max|x| <= 448 * 2^e).
//
// Backward FP8 buffer (BH = batch * heads, Tp = round_up(T, 64), NT = Tp / 64,
// n = BH * Tp * 64 bytes):
//   [0, n)      V codes, channel blocks    [BH][Tp][64]
//   [n, 2n)     dO codes, channel blocks   [BH][Tp][64]
//   [2n, 3n)    Q codes, position blocks   [BH][64][Tp]  (channel-major)
//   [3n, 4n)    K codes, position blocks   [BH][64][Tp]
//   [4n, 5n)    dO codes, position blocks  [BH][64][Tp]
//   [5n, ...)   BH * NT side tiles of 1152 bytes per 64 positions:
//     [0, 128) V exponents, [128, 256) K (position blocks), [256, 384) dO
//     (channel blocks), [384, 512) Q (position blocks), [512, 640) dO
//     (position blocks), [640, 896) LSE * log2 e (float32, +inf past T),
//     [896, 1152) D (float32, 0 past T).
// Exponent bytes are e + 127; channel-blocked arrays keep 2 per position
// (block c of position p at 2p + c), position-blocked arrays 64 per block
// of 32 positions (channel k of block c at 64c + k).
#include "attn_fp8_common.h"

// Waves per SIMD the register allocation aims at: three for dQ (159 VGPRs, no
// spills; measured 4% faster than two); the dK/dV kernel needs about 230
// and runs at two (holding its K and V operands in LDS to fit three measured
// slower).
#ifndef CATTN_FP8_DQ_WAVES_PER_SIMD
#define CATTN_FP8_DQ_WAVES_PER_SIMD 3
#endif
#ifndef CATTN_FP8_DKDV_WAVES_PER_SIMD
#define CATTN_FP8_DKDV_WAVES_PER_SIMD 1
#endif

namespace cattn {
namespace {

constexpr int SIDE_TILE = 1152;
constexpr int SD_V = 0, SD_KP = 128, SD_G = 256, SD_QP = 384, SD_GP = 512, SD_LSE = 640, SD_D = 896;

struct Fp8BwdLayout {
    long long g, qp, kp, gp, side;  // byte offsets
    int Tp, NT;
};

Fp8BwdLayout fp8_bwd_layout(int B, int T, int H) {
    Fp8BwdLayout L;
    L.Tp = (T + 63) / 64 * 64;
    L.NT = L.Tp / 64;
    const long long n = (long long)B * H * L.Tp * 64;
    L.g = n;
    L.qp = 2 * n;
    L.kp = 3 * n;
    L.gp = 4 * n;
    L.side = 5 * n;
    return L;
}

// ---------------------------------------------------------------------------
// Quantization of the backward's operands, one workgroup per (head, tile of
// 64 positions): V and dO rows in channel blocks (thread: position tid / 4,
// 16 channels); D and LSE * log2 e of the tile's rows; then Q, K and dO in
// position blocks through float copies in LDS (thread: channel tid / 4, 16
// positions).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_quantize_bwd_fp8_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ dout, const bf16* __restrict__ out,
    const float* __restrict__ lse, u8* __restrict__ buf, int T, int H, Fp8BwdLayout L) {
    __shared__ float tile[3][64][65];
    const int bh = blockIdx.x / L.NT, t = blockIdx.x - bh * L.NT, b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x;
    const int C = H * HEAD_DIM;
    const int p = tid >> 2, cq = tid & 3;
    const int pos = t * 64 + p;
    const bool valid = pos < T;
    const long long tok = (long long)b * T + (valid ? pos : 0);
    const bf16* qrow = qkv + tok * 3 * C + h * HEAD_DIM + 16 * cq;
    const bf16* grow = dout + tok * C + h * HEAD_DIM + 16 * cq;
    const bf16* orow = out + tok * C + h * HEAD_DIM + 16 * cq;
    u8* side = buf + L.side + ((long long)bh * L.NT + t) * SIDE_TILE;

    float xq[16], xk[16], xv[16], xg[16], xo[16];
    bf16x16_to_f32(qrow, valid, xq);
    bf16x16_to_f32(qrow + C, valid, xk);
    bf16x16_to_f32(qrow + 2 * C, valid, xv);
    bf16x16_to_f32(grow, valid, xg);
    bf16x16_to_f32(orow, valid, xo);

    const long long row_off = ((long long)bh * L.Tp + pos) * 64 + 16 * cq;
    u32x4 codes;
    int e = quantize16(xv, codes);
    *reinterpret_cast<u32x4*>(buf + row_off) = codes;
    if ((cq & 1) == 0) side[SD_V + 2 * p + (cq >> 1)] = (u8)(e + 127);
    e = quantize16(xg, codes);
    *reinterpret_cast<u32x4*>(buf + L.g + row_off) = codes;
    if ((cq & 1) == 0) side[SD_G + 2 * p + (cq >> 1)] = (u8)(e + 127);

    // D: the 16 products of each quarter in channel order, then
    // (q0 + q1) + (q2 + q3).
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) part = fmaf(xg[i], xo[i], part);
    part += __shfl_xor(part, 1, 64);
    part += __shfl_xor(part, 2, 64);
    if (cq == 0) {
        float* sf = reinterpret_cast<float*>(side);
        sf[SD_LSE / 4 + p] = valid ? lse[(long long)bh * T + pos] * LOG2E : INFINITY;
        sf[SD_D / 4 + p] = valid ? part : 0.0f;
    }

#pragma unroll
    for (int i = 0; i < 16; ++i) {
        tile[0][p][16 * cq + i] = xq[i];
        tile[1][p][16 * cq + i] = xk[i];
        tile[2][p][16 * cq + i] = xg[i];
    }
    __syncthreads();
    const int c = tid >> 2, pq = tid & 3;
    const long long col_off = ((long long)bh * 64 + c) * L.Tp + t * 64 + 16 * pq;
    const long long dst[3] = {L.qp, L.kp, L.gp};
    const int sd[3] = {SD_QP, SD_KP, SD_GP};
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        float y[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = tile[m][16 * pq + i][c];
        e = quantize16(y, codes);
        *reinterpret_cast<u32x4*>(buf + dst[m] + col_off) = codes;
        if ((pq & 1) == 0) side[sd[m] + 64 * (pq >> 1) + c] = (u8)(e + 127);
    }
}

// ---------------------------------------------------------------------------
// Shared pieces of the two gradient kernels.
// ---------------------------------------------------------------------------
constexpr int NSTAGE = 3;

// A operand rows of a 64-row code tile (rows swizzled by swz_k): row
// 32 blk + key_of_row(r), chunks h and 2 + h.
__device__ __forceinline__ void row_offsets(int l32, int hf, int (&off)[2][2], int (&row)[2]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int r = 32 * blk + key_of_row(l32);
        row[blk] = r;
        off[blk][0] = r * 64 + 16 * (hf ^ swz_k(r));
        off[blk][1] = r * 64 + 16 * ((2 + hf) ^ swz_k(r));
    }
}

// A operand rows of a channel-major tile (rows = channels, swizzled by
// swz_v): channel 32 db + r, chunks h and 2 + h.
__device__ __forceinline__ void col_offsets(int l32, int hf, int (&off)[2][2]) {
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        const int ch = 32 * db + l32;
        off[db][0] = ch * 64 + 16 * (hf ^ swz_v(ch));
        off[db][1] = ch * 64 + 16 * ((2 + hf) ^ swz_v(ch));
    }
}

// E4M3 codes of x / 2^e for the two 16-value halves of a lane's operand
// (block kb of x with exponent e[kb]), x[kb][0] in the low byte.
__device__ __forceinline__ i32x8 scaled_operand(const f32x16 (&x)[2], const int (&e)[2]) {
    i32x8 r;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            int old;
            asm volatile("" : "=v"(old));
            int d = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[kb][4 * w], -e[kb]),
                                                    ldexpf(x[kb][4 * w + 1], -e[kb]), old, false);
            d = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[kb][4 * w + 2], -e[kb]),
                                                ldexpf(x[kb][4 * w + 3], -e[kb]), d, true);
            r[4 * kb + w] = d;
        }
    return r;
}

// Block exponents of dS for the operand above: block kb holds register block
// kb of both lane halves (32 values), so its maximum spans the lane pair.
__device__ __forceinline__ void block_exponents(const f32x16 (&x)[2], int (&e)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(x[kb][i]));
        e[kb] = mx_exponent(fmaxf(m, swap_halves(m)));
    }
}

__device__ __forceinline__ i32x8 reg_operand(const u8* row, int hf, bool ok) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 a = ok ? *reinterpret_cast<const u32x4*>(row + 16 * hf) : z;
    const u32x4 c = ok ? *reinterpret_cast<const u32x4*>(row + 32 + 16 * hf) : z;
    const i32x8 r = {(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                     (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
    return r;
}

// Store a transposed accumulator (rows = channels 32 db + 8(i/4) + 4h + i%4,
// column = the lane's row of the output) times `mul` as bf16.
__device__ __forceinline__ void store_rows(bf16* dst, const f32x16 (&acc)[2], int hf, float mul) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + 8 * g + 4 * hf;
            *reinterpret_cast<u32x2*>(dst + d) =
                to_bf16x4_bits(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul,
                               acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul);
        }
}

// Workgroup -> (tile, head), heads grouped per XCD when the count allows;
// `first_heavy` walks tiles from the last (dQ: most keys) or the first
// (dK/dV: most queries).
__device__ __forceinline__ void wg_tile(int BH, int n_t, bool last_first, int& tl, int& bh) {
    const int blk = blockIdx.x;
    int s;
    if ((BH & 7) == 0) {
        const int per = BH >> 3, xcd = blk & 7;
        s = blk >> 3;
        bh = xcd * per + s % per;
        s /= per;
    } else {
        s = blk / BH;
        bh = blk % BH;
    }
    tl = last_first ? n_t - 1 - s : s;
}

struct DqSmem {
    u8 k[NSTAGE][64 * 64];   // K codes, channel blocks, rows = keys
    u8 v[NSTAGE][64 * 64];   // V codes, channel blocks, rows = keys
    u8 kt[NSTAGE][64 * 64];  // K codes, position blocks, rows = channels
    u8 e[NSTAGE][384];       // exponents: K rows, V rows, K position blocks
};

// ---------------------------------------------------------------------------
// dQ: one workgroup per (128 queries, head), wave w owns queries q0 + 32w ..
// +31, key tiles of 64 up to the diagonal. Per tile: S^T = K Q^T and dP^T =
// V dO^T (A = K, V rows from LDS, B = Q, dO rows of the lane's query in
// registers), P and dS on the VALU (LSE and D of the lane's query in
// registers), dS^T quantized per 32 keys, dQ^T += K_p^T dS^T.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, CATTN_FP8_DQ_WAVES_PER_SIMD) void attn_bwd_fp8_dq_kernel(
    const u8* __restrict__ f8, const u8* __restrict__ b8, bf16* __restrict__ dqkv, int B, int T,
    int H, Fp8Layout LF, Fp8BwdLayout LB, float c_log2) {
    __shared__ DqSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int BH = B * H;
    const int n_qt = (T + 127) / 128;
    int qt, bh;
    wg_tile(BH, n_qt, true, qt, bh);
    const int b = bh / H, h = bh - b * H;
    const int C = H * HEAD_DIM;
    const int Tp = LF.Tp;

    const u8* qc = f8 + (long long)bh * Tp * 64;
    const u8* kc = f8 + LF.k + (long long)bh * Tp * 64;
    const u8* fexp = f8 + LF.e + (long long)bh * LF.NT * 384;
    const u8* vc = b8 + (long long)bh * Tp * 64;
    const u8* gc = b8 + LB.g + (long long)bh * Tp * 64;
    const u8* kp = b8 + LB.kp + (long long)bh * 64 * Tp;
    const u8* side = b8 + LB.side + (long long)bh * LB.NT * SIDE_TILE;
    const i32x4 rs_k = buffer_rsrc(kc, (unsigned int)(Tp * 64));
    const i32x4 rs_v = buffer_rsrc(vc, (unsigned int)(Tp * 64));
    const i32x4 rs_kt = buffer_rsrc(kp, (unsigned int)(Tp * 64));
    const i32x4 rs_fe = buffer_rsrc(fexp, (unsigned int)(LF.NT * 384));
    const i32x4 rs_sd = buffer_rsrc(side, (unsigned int)(LB.NT * SIDE_TILE));

    const int q0 = qt * 128, qw = q0 + 32 * wave;
    const int n_kt = (min(q0 + 128, T) + 63) / 64;
    const int j_last = min((qw + 31) / 64, n_kt - 1);

    const int lrow = 16 * wave + (lane >> 2), lpos = lane & 3;
    const unsigned int voff_r = (unsigned int)(lrow * 64 + 16 * (lpos ^ swz_k(lrow)));
    const unsigned int voff_c = (unsigned int)(lrow * Tp + 16 * (lpos ^ swz_v(lrow)));
    const unsigned int wave_lds = __builtin_amdgcn_readfirstlane((unsigned int)(1024 * wave));
    // Wave-uniform LDS byte addresses of stage 0; stage st sits st stages on.
    const unsigned int k_l = lds_addr_u(sm.k[0]), v_l = lds_addr_u(sm.v[0]);
    const unsigned int c_l = lds_addr_u(sm.kt[0]), e_l = lds_addr_u(sm.e[0]);
    constexpr unsigned int K_ST = sizeof(sm.k[0]), C_ST = sizeof(sm.kt[0]), E_ST = sizeof(sm.e[0]);
    auto issue = [&](int j) {
        const unsigned int st = (unsigned int)j % NSTAGE;
        lds_dma16_buf(rs_k, voff_r, (unsigned int)(j * 4096), k_l + st * K_ST + wave_lds);
        lds_dma16_buf(rs_v, voff_r, (unsigned int)(j * 4096), v_l + st * K_ST + wave_lds);
        lds_dma16_buf(rs_kt, voff_c, (unsigned int)(j * 64), c_l + st * C_ST + wave_lds);
        if (wave == 0 && lane < 8)   // K exponents of the forward buffer
            lds_dma16_buf(rs_fe, (unsigned int)(128 + 16 * lane), (unsigned int)(j * 384),
                          e_l + st * E_ST);
        if (wave == 1 && lane < 16)  // V and K position-block exponents
            lds_dma16_buf(rs_sd, (unsigned int)(16 * lane), (unsigned int)(j * SIDE_TILE),
                          e_l + st * E_ST + 128);
    };
    issue(0);
    if (n_kt > 1) issue(1);

    // B operands of the lane's query: Q and dO in channel blocks.
    const int q = qw + l32;
    const bool qok = q < Tp;
    const long long qrow = (long long)(qok ? q : 0) * 64;
    const i32x8 qop = reg_operand(qc + qrow, hf, qok);
    const i32x8 gop = reg_operand(gc + qrow, hf, qok);
    int qs = 0, gs = 0;
    float lse2 = INFINITY, dd = 0.0f;
    if (qok) {
        const int tq = q >> 6, pq = q & 63;
        qs = fexp[tq * 384 + 2 * pq + hf];
        gs = side[tq * SIDE_TILE + SD_G + 2 * pq + hf];
        lse2 = reinterpret_cast<const float*>(side + tq * SIDE_TILE + SD_LSE)[pq];
        dd = reinterpret_cast<const float*>(side + tq * SIDE_TILE + SD_D)[pq];
    }
    int aoff[2][2], arow[2], coff[2][2];
    row_offsets(l32, hf, aoff, arow);
    col_offsets(l32, hf, coff);
    wait_vmem<0>();
    __syncthreads();

    f32x16 acc[2] = {zero16(), zero16()};  // dQ^T per channel block
    for (int j = 0; j < n_kt; ++j) {
        if (j >= 1 && j + 1 < n_kt) {
            if (wave < 2) wait_vmem<4>();
            else wait_vmem<3>();
        } else {
            wait_vmem<0>();
        }
        __syncthreads();
        if (j + 2 < n_kt) issue(j + 2);
        if (j > j_last) continue;
        const unsigned int st = (unsigned int)j % NSTAGE;
        lds_u8* kt = lds_view_at(k_l + st * K_ST);
        lds_u8* vt = lds_view_at(v_l + st * K_ST);
        lds_u8* ct = lds_view_at(c_l + st * C_ST);
        lds_u8* et = lds_view_at(e_l + st * E_ST);
        f32x16 s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = mfma_f8(lds_operand(kt, aoff[kb]), qop, zero16(), et[2 * arow[kb] + hf], qs);
            dp[kb] = mfma_f8(lds_operand(vt, aoff[kb]), gop, zero16(), et[128 + 2 * arow[kb] + hf], gs);
        }
        const i32x8 ka = lds_operand(ct, coff[0]);
        const i32x8 kb1 = lds_operand(ct, coff[1]);
        const int ksa = et[256 + 64 * hf + l32], ksb = et[256 + 64 * hf + 32 + l32];
        // register i of block kb holds key 64 j + 32 kb + 16 h + i
        if (j == j_last) {
            const int lim = qw - 64 * j + l32 - 16 * hf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kb + i > lim) s[kb][i] = -INFINITY;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pr = fast_exp2(fmaf(s[kb][i], c_log2, -lse2));
                s[kb][i] = pr * (dp[kb][i] - dd);  // dS
            }
        int e[2];
        block_exponents(s, e);
        const i32x8 dsop = scaled_operand(s, e);
        const int ds_scale = e[hf] + 127;
        acc[0] = mfma_f8(ka, dsop, acc[0], ksa, ds_scale);
        acc[1] = mfma_f8(kb1, dsop, acc[1], ksb, ds_scale);
    }
    if (q < T)
        store_rows(dqkv + ((long long)b * T + q) * 3 * C + h * HEAD_DIM, acc, hf, 0.125f);
}

struct DkdvSmem {
    u8 q[NSTAGE][64 * 64];   // Q codes, channel blocks, rows = queries
    u8 g[NSTAGE][64 * 64];   // dO codes, channel blocks, rows = queries
    u8 qt[NSTAGE][64 * 64];  // Q codes, position blocks, rows = channels
    u8 gt[NSTAGE][64 * 64];  // dO codes, position blocks, rows = channels
    u8 e[NSTAGE][1024];      // Q rows, dO rows, Q and dO position-block exponents; LSE2, D
};

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (128 keys, head), wave w owns keys k0 + 32w ..
// +31, query tiles of 64 from the diagonal on. Per tile: S = Q K^T and dP =
// dO V^T (A = Q, dO rows from LDS, B = K, V rows of the lane's key in
// registers), P and dS on the VALU (LSE and D per query from LDS), dV^T +=
// dO_p^T P^ and dK^T += Q_p^T dS_q (dS quantized per 32 queries).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, CATTN_FP8_DKDV_WAVES_PER_SIMD) void attn_bwd_fp8_dkdv_kernel(
    const u8* __restrict__ f8, const u8* __restrict__ b8, bf16* __restrict__ dqkv, int B, int T,
    int H, Fp8Layout LF, Fp8BwdLayout LB, float c_log2) {
    __shared__ DkdvSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int BH = B * H;
    const int n_kt = (T + 127) / 128;
    int kt, bh;
    wg_tile(BH, n_kt, false, kt, bh);
    const int b = bh / H, h = bh - b * H;
    const int C = H * HEAD_DIM;
    const int Tp = LF.Tp;

    const u8* qc = f8 + (long long)bh * Tp * 64;
    const u8* kc = f8 + LF.k + (long long)bh * Tp * 64;
    const u8* fexp = f8 + LF.e + (long long)bh * LF.NT * 384;
    const u8* vc = b8 + (long long)bh * Tp * 64;
    const u8* gc = b8 + LB.g + (long long)bh * Tp * 64;
    const u8* qp = b8 + LB.qp + (long long)bh * 64 * Tp;
    const u8* gp = b8 + LB.gp + (long long)bh * 64 * Tp;
    const u8* side = b8 + LB.side + (long long)bh * LB.NT * SIDE_TILE;
    const i32x4 rs_q = buffer_rsrc(qc, (unsigned int)(Tp * 64));
    const i32x4 rs_g = buffer_rsrc(gc, (unsigned int)(Tp * 64));
    const i32x4 rs_qt = buffer_rsrc(qp, (unsigned int)(Tp * 64));
    const i32x4 rs_gt = buffer_rsrc(gp, (unsigned int)(Tp * 64));
    const i32x4 rs_fe = buffer_rsrc(fexp, (unsigned int)(LF.NT * 384));
    const i32x4 rs_sd = buffer_rsrc(side, (unsigned int)(LB.NT * SIDE_TILE));

    const int k0 = kt * 128, kw = k0 + 32 * wave;
    const int j0 = k0 / 64;                 // first query tile with a query >= k0
    const int n_qt = LF.NT;                 // query tiles of 64
    const int n_steps = n_qt - j0;

    const int lrow = 16 * wave + (lane >> 2), lpos = lane & 3;
    const unsigned int voff_r = (unsigned int)(lrow * 64 + 16 * (lpos ^ swz_k(lrow)));
    const unsigned int voff_c = (unsigned int)(lrow * Tp + 16 * (lpos ^ swz_v(lrow)));
    const unsigned int wave_lds = __builtin_amdgcn_readfirstlane((unsigned int)(1024 * wave));
    // Wave-uniform LDS byte addresses of stage 0; stage st sits st stages on.
    const unsigned int q_l = lds_addr_u(sm.q[0]), g_l = lds_addr_u(sm.g[0]);
    const unsigned int qc_l = lds_addr_u(sm.qt[0]), gc_l = lds_addr_u(sm.gt[0]);
    const unsigned int e_l = lds_addr_u(sm.e[0]);
    constexpr unsigned int R_ST = sizeof(sm.q[0]), C_ST = sizeof(sm.qt[0]), E_ST = sizeof(sm.e[0]);
    auto issue = [&](int j, int it) {
        const unsigned int st = (unsigned int)it % NSTAGE;
        lds_dma16_buf(rs_q, voff_r, (unsigned int)(j * 4096), q_l + st * R_ST + wave_lds);
        lds_dma16_buf(rs_g, voff_r, (unsigned int)(j * 4096), g_l + st * R_ST + wave_lds);
        lds_dma16_buf(rs_qt, voff_c, (unsigned int)(j * 64), qc_l + st * C_ST + wave_lds);
        lds_dma16_buf(rs_gt, voff_c, (unsigned int)(j * 64), gc_l + st * C_ST + wave_lds);
        if (wave == 0 && lane < 56)  // dO, Q, dO exponents, LSE2, D of the side tile
            lds_dma16_buf(rs_sd, (unsigned int)(SD_G + 16 * lane), (unsigned int)(j * SIDE_TILE),
                          e_l + st * E_ST + 128);
        if (wave == 1 && lane < 8)   // Q exponents of the forward buffer
            lds_dma16_buf(rs_fe, (unsigned int)(16 * lane), (unsigned int)(j * 384),
                          e_l + st * E_ST);
    };
    issue(j0, 0);
    if (n_steps > 1) issue(j0 + 1, 1);

    // B operands of the lane's key: K and V in channel blocks.
    const int key = kw + l32;
    const bool kok = key < Tp;
    const long long krow = (long long)(kok ? key : 0) * 64;
    const i32x8 kop = reg_operand(kc + krow, hf, kok);
    const i32x8 vop = reg_operand(vc + krow, hf, kok);
    int ks = 0, vs = 0;
    if (kok) {
        ks = fexp[(key >> 6) * 384 + 128 + 2 * (key & 63) + hf];
        vs = side[(key >> 6) * SIDE_TILE + SD_V + 2 * (key & 63) + hf];
    }
    int aoff[2][2], arow[2], coff[2][2];
    row_offsets(l32, hf, aoff, arow);
    col_offsets(l32, hf, coff);
    wait_vmem<0>();
    __syncthreads();

    f32x16 dk[2] = {zero16(), zero16()}, dv[2] = {zero16(), zero16()};  // transposed, per channel block
    for (int it = 0; it < n_steps; ++it) {
        const int j = j0 + it;
        if (it >= 1 && it + 1 < n_steps) {
            if (wave < 2) wait_vmem<5>();
            else wait_vmem<4>();
        } else {
            wait_vmem<0>();
        }
        __syncthreads();
        if (it + 2 < n_steps) issue(j + 2, it + 2);
        if (64 * j + 63 < kw) continue;  // every query of the tile is before the wave's keys
        const unsigned int st = (unsigned int)it % NSTAGE;
        lds_u8* qt_ = lds_view_at(q_l + st * R_ST);
        lds_u8* gt_ = lds_view_at(g_l + st * R_ST);
        lds_u8* qpt = lds_view_at(qc_l + st * C_ST);
        lds_u8* gpt = lds_view_at(gc_l + st * C_ST);
        lds_u8* et = lds_view_at(e_l + st * E_ST);
        f32x16 s[2], dp[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            s[qb] = mfma_f8(lds_operand(qt_, aoff[qb]), kop, zero16(), et[2 * arow[qb] + hf], ks);
            dp[qb] = mfma_f8(lds_operand(gt_, aoff[qb]), vop, zero16(), et[128 + 2 * arow[qb] + hf], vs);
        }
        const i32x8 ga = lds_operand(gpt, coff[0]), gb = lds_operand(gpt, coff[1]);
        const i32x8 qa = lds_operand(qpt, coff[0]), qbo = lds_operand(qpt, coff[1]);
        const int gsa = et[384 + 64 * hf + l32], gsb = et[384 + 64 * hf + 32 + l32];
        const int qsa = et[256 + 64 * hf + l32], qsb = et[256 + 64 * hf + 32 + l32];
        // register i of block qb holds query 64 j + 32 qb + 16 h + i
        typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
        lds_f32x4* lse4 = reinterpret_cast<lds_f32x4*>(et + 512);
        lds_f32x4* d4 = reinterpret_cast<lds_f32x4*>(et + 768);
        if (64 * j < kw + 31) {  // the tile holds queries before some of the wave's keys
            const int lim = kw + l32 - 64 * j - 16 * hf;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * qb + i < lim) s[qb][i] = -INFINITY;
        }
        f32x16 pp[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 l = lse4[8 * qb + 4 * hf + g4];
                const f32x4 dd = d4[8 * qb + 4 * hf + g4];
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int i = 4 * g4 + e4;
                    const float pr = fast_exp2(fmaf(s[qb][i], c_log2, -l[e4]));
                    pp[qb][i] = pr * 256.0f;
                    s[qb][i] = pr * (dp[qb][i] - dd[e4]);  // dS
                }
            }
        const i32x8 pop = p_operand(pp);
        dv[0] = mfma_f8(ga, pop, dv[0], gsa, P_SCALE);
        dv[1] = mfma_f8(gb, pop, dv[1], gsb, P_SCALE);
        int e[2];
        block_exponents(s, e);
        const i32x8 dsop = scaled_operand(s, e);
        const int ds_scale = e[hf] + 127;
        dk[0] = mfma_f8(qa, dsop, dk[0], qsa, ds_scale);
        dk[1] = mfma_f8(qbo, dsop, dk[1], qsb, ds_scale);
    }
    if (key < T) {
        bf16* row = dqkv + ((long long)b * T + key) * 3 * C + h * HEAD_DIM;
        store_rows(row + C, dk, hf, 0.125f);
        store_rows(row + 2 * C, dv, hf, 1.0f);
    }
}

}  // namespace

long long fp8_bwd_buffer_bytes(int B, int T, int H) {
    const Fp8BwdLayout L = fp8_bwd_layout(B, T, H);
    return L.side + (long long)B * H * L.NT * SIDE_TILE;
}

hipError_t launch_attn_quantize_bwd_fp8(const void* dout, const void* qkv, const void* out,
                                        const float* lse, void* b8, int B, int T, int H,
                                        hipStream_t stream) {
    const Fp8BwdLayout L = fp8_bwd_layout(B, T, H);
    const long long blocks = (long long)B * H * L.NT;
    hipLaunchKernelGGL(attn_quantize_bwd_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16*>(qkv), static_cast<const bf16*>(dout),
                       static_cast<const bf16*>(out), lse, static_cast<u8*>(b8), T, H, L);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_fp8(const void* f8, const void* b8, void* dqkv, int B, int T, int H,
                               hipStream_t stream) {
    const Fp8Layout LF = fp8_layout(B, T, H);
    const Fp8BwdLayout LB = fp8_bwd_layout(B, T, H);
    const long long blocks = (long long)B * H * ((T + 127) / 128);
    const float c_log2 = LOG2E / 8.0f;
    hipLaunchKernelGGL(attn_bwd_fp8_dq_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u8*>(f8), static_cast<const u8*>(b8),
                       static_cast<bf16*>(dqkv), B, T, H, LF, LB, c_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_bwd_fp8_dkdv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u8*>(f8), static_cast<const u8*>(b8),
                       static_cast<bf16*>(dqkv), B, T, H, LF, LB, c_log2);
    return hipGetLastError();
}

}  // namespace cattn
