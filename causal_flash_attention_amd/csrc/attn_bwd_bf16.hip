// Causal attention backward, bf16 storage, fp32 accumulation, MFMA (gfx950).
//
// Gradients of L = sum(dO * O) for O = softmax(scale * Q K^T + mask) V, with
// the probabilities recomputed from the forward's per-row log-sum-exp instead
// of being stored, which is what lets the method of "Let's reproduce GPT-2
// (124M)" (chapter list, 02:00:18; glossary row "flash attention" of the
// theprofessional.online summary) keep memory traffic linear in T in every
// training step:
//
//   D   = rowsum(dO * O)                       (attn_bwd_pre_bf16_kernel)
//   P   = exp(scale * Q K^T - LSE),  dP = dO V^T,  dS = P * (dP - D)
//   dV  = P^T dO,  dK = scale * dS^T Q         (attn_bwd_dkdv_bf16_kernel)
//   dQ  = scale * dS K                         (attn_bwd_dq_bf16_kernel)
//
// The dK/dV and dQ kernels each own disjoint output rows, so the backward
// uses no atomics and is bitwise reproducible run to run.
//
// Workspace (float32, per (batch, head) row padded to Tp = round_up(T, 64);
// 10 * BH * Tp floats in all):
//   ws[0 .. BH*Tp)        D,            0 for t >= T
//   ws[BH*Tp .. 2*BH*Tp)  LSE * log2 e, +inf for t >= T (so P = 0 there)
//   ws[2*BH*Tp .. )       the dK/dV kernel's extra MFMA k-step operands, 32
//                         bytes per row: for 8 * LSE and for D, three bf16
//                         values whose sum is the float exactly, then five
//                         zeros (mfma_terms). Per group of 32 rows the 32
//                         rows' LSE terms come first, then their D terms
//                         (term_m, term_d); padding rows take terms that make
//                         P = 0 (mfma_terms_pad)
#include <type_traits>

#include "attn_common.h"

namespace cattn {
namespace {

#ifndef CATTN_DKDV_WAVES_PER_SIMD
#define CATTN_DKDV_WAVES_PER_SIMD 2
#endif

constexpr int ROW_PAD = 64;
constexpr int NSTAGE = 3;

// ---------------------------------------------------------------------------
// Preprocess: D[b, h, t] = sum_k dO[b,t,h,k] O[b,t,h,k] and LSE * log2 e, with
// the padding of both. The dQ kernel can do the same work for its own rows
// (the fused form used by attn_bwd); both compute D in one fixed order, so
// the staged and fused workspaces agree bit for bit.
// ---------------------------------------------------------------------------

// Half of D: the 32 products of k = 16kk + 8*half + e, kk and e ascending,
// in one fmaf chain from zero. D = (half 0) + (half 1).
__device__ __forceinline__ float dot_half(const bf16x8 (&g)[4], const bf16x8 (&o)[4]) {
    float acc = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)g[kk][e], (float)o[kk][e], acc);
    return acc;
}

// The MFMA form of a row statistic x: eight bf16 [x1 x2 x3 0 0 0 0 0] with
// x1 = bf16(x), x2 = bf16(x - x1), x3 = bf16(x - x1 - x2), so x1 + x2 + x3
// equals x for every normal float. One extra MFMA k-step with these terms as
// A and -1 as B subtracts x from a whole score row inside the accumulator.
__device__ __forceinline__ u32x4 mfma_terms(float x) {
    const bf16 a = (bf16)x;
    const float r = x - (float)a;
    const bf16 b = (bf16)r;
    const bf16 c = (bf16)(r - (float)b);
    const bf16 z = (bf16)0.0f;
    const bf16x8 v = {a, b, c, z, z, z, z, z};
    return __builtin_bit_cast(u32x4, v);
}

// The m terms of a row past T: the largest finite bf16, so that P = 0 there
// while every product in the MFMA stays finite.
__device__ __forceinline__ u32x4 mfma_terms_pad() {
    const u32x4 v = {0x7F7Fu, 0u, 0u, 0u};
    return v;
}

// The MFMA terms of the workspace rows (m = 8 * LSE, and D), 16 bytes each,
// in groups of 32 rows: the m terms of the group's 32 rows, then their D
// terms, so that 16 lanes reading 16 consecutive rows' terms touch 256
// consecutive bytes (no LDS bank conflict once the group is staged).
__device__ __forceinline__ u32x4* ws_terms(float* ws, long long n_pad_rows) {
    return reinterpret_cast<u32x4*>(ws + 2 * n_pad_rows);
}
__device__ __forceinline__ long long term_m(long long r) { return (r >> 5) * 64 + (r & 31); }
__device__ __forceinline__ long long term_d(long long r) { return term_m(r) + 32; }

// Blocks [0, nb_d): D, two lanes per (b, t, h) row (one per half).
// Blocks [nb_d, ...): one thread per padded (bh, t): LSE * log2 e and the m
// terms, and the padding of all of them.
__global__ __launch_bounds__(256) void attn_bwd_pre_bf16_kernel(
    const bf16* __restrict__ dout, const bf16* __restrict__ out, const float* __restrict__ lse,
    float* __restrict__ ws, int T, int Tp, int H, long long n_rows, long long nb_d,
    long long n_pad_rows) {
    const long long blk = blockIdx.x;
    float* __restrict__ dd = ws;
    float* __restrict__ lse2 = ws + n_pad_rows;
    if (blk < nb_d) {
        const long long row = blk * 128 + (threadIdx.x >> 1);
        const int half = threadIdx.x & 1;
        float acc = 0.0f;
        if (row < n_rows) {
            const long long off = row * HEAD_DIM + half * 8;  // rows are (b, t, h) in memory order
            bf16x8 g[4], o[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                g[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(dout + off + 16 * kk));
                o[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(out + off + 16 * kk));
            }
            acc = dot_half(g, o);
        }
        acc += __shfl_xor(acc, 1, 64);
        if (row < n_rows) {
            const long long bt = row / H;
            const int h = (int)(row - bt * H);
            const long long b = bt / T;
            const int t = (int)(bt - b * T);
            const long long r = (b * H + h) * Tp + t;
            if (half == 0) dd[r] = acc;
            else ws_terms(ws, n_pad_rows)[term_d(r)] = mfma_terms(acc);
        }
    } else {
        const long long i = (blk - nb_d) * 256 + threadIdx.x;  // padded (bh, t)
        if (i < n_pad_rows) {
            const long long bh = i / Tp;
            const int t = (int)(i - bh * Tp);
            u32x4* terms = ws_terms(ws, n_pad_rows);
            if (t < T) {
                const float l = lse[bh * T + t];
                lse2[i] = l * LOG2E;
                terms[term_m(i)] = mfma_terms(8.0f * l);
            } else {
                lse2[i] = INFINITY;
                dd[i] = 0.0f;
                terms[term_m(i)] = mfma_terms_pad();
                terms[term_d(i)] = mfma_terms(0.0f);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dK, dV. One workgroup = 4 waves = 128 keys of one (batch, head); wave w owns
// keys k0 + 32w .. +31, with K and V of those keys held in registers. Query
// tiles of 64 rows (Q, dO, and the MFMA terms of their 8 * LSE and D) stream
// through a three-stage ring of LDS buffers filled by direct loads. Per tile
// and wave: S - 8 LSE and dP - D on MFMA (lane l%32 owns key l%32; the row
// statistics enter as one extra k-step of each product, so no lane reads
// them), P and dS in registers, then dV^T += dO^T P and dK^T += Q^T dS on MFMA with
// P and dS fed straight from registers and Q^T, dO^T read from the row-major
// tiles by transposing LDS reads. Query tiles entirely before a wave's keys
// are skipped.
// ---------------------------------------------------------------------------
constexpr int KV_BN = 128;  // keys per workgroup
constexpr int KV_BM = 64;   // queries per LDS tile

struct alignas(16) DkdvSmem {
    bf16 q[NSTAGE][ATILE_ELEMS];
    bf16 g[NSTAGE][ATILE_ELEMS];
    bf16 terms[NSTAGE][KV_BM * 16];  // two groups of 32 rows: 32 m terms, then 32 D terms
};

// The dK/dV step on a 64-query tile runs as two 32-query halves (QB), each
// in three phases: S and dP on MFMA; P and dS on the VALU; then
// dV^T += dO^T P and dK^T += Q^T dS on MFMA. The phases are ordered so that
// one half's VALU work sits between MFMAs of the other half that do not
// depend on it. MASK applies the causal mask (the tile holding this wave's
// diagonal only).
// S - 8 LSE and dP - D of one half: four k-steps over d, then one over the
// row's terms (A: lane half 0 holds the m terms, half 1 the D terms; B: bs
// is -1 on the m terms and bd is -1 on the D terms, zero elsewhere).
template <int QB>
__device__ __forceinline__ void dkdv_sdp(lds_bf16* qt, lds_bf16* gt, lds_bf16* terms,
                                         const bf16x8 (&kreg)[4], const bf16x8 (&vreg)[4],
                                         const int (&roff)[4], bf16x8 bs, bf16x8 bd, int toff,
                                         f32x16& s, f32x16& dp) {
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
    // All nine operand reads first, then the MFMAs: the scheduling barrier
    // keeps the compiler from pairing each read with the MFMA that uses it,
    // which would expose one LDS latency per MFMA at the start of each half.
    bf16x8 qa[4], ga[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int o = QB * 32 * 64 + roff[kk];
        qa[kk] = *reinterpret_cast<lds_bf16x8*>(qt + o);
        ga[kk] = *reinterpret_cast<lds_bf16x8*>(gt + o);
    }
    const bf16x8 a = *reinterpret_cast<lds_bf16x8*>(terms + QB * 512 + toff);
    __builtin_amdgcn_sched_barrier(0);
    s = zero16();
    dp = zero16();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        s = mfma32(qa[kk], kreg[kk], s);
        dp = mfma32(ga[kk], vreg[kk], dp);
    }
    s = mfma32(a, bs, s);
    dp = mfma32(a, bd, dp);
}

// P = exp2(c (S - 8 LSE)) = exp(scale S - LSE) and dS = P (dP - D).
template <int QB, bool MASK>
__device__ __forceinline__ void dkdv_pds(f32x16& s, f32x16& dp, int lim, float c_log2,
                                         bf16x8 (&pds)[4]) {
    if (MASK) {  // query QB*32 + 8(i/4) + 4hf + (i%4) < my_k - q0  ->  P = 0
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (QB * 32 + 8 * (i >> 2) + (i & 3) < lim) s[i] = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(s[i] * c_log2);
        s[i] = p;
        dp[i] = p * dp[i];
    }
    pds[0] = c_rows_to_operand(s, 0);
    pds[1] = c_rows_to_operand(s, 1);
    pds[2] = c_rows_to_operand(dp, 0);
    pds[3] = c_rows_to_operand(dp, 1);
}

template <int QB>
__device__ __forceinline__ void dkdv_acc(lds_bf16* qt, lds_bf16* gt, const int (&troff)[2][2],
                                         const bf16x8 (&pds)[4], f32x16 (&dvt)[2],
                                         f32x16 (&dkt)[2]) {
    // The eight transposed operands first, then the MFMAs (as for S and dP).
    bf16x8 ga[2][2], qa[2][2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            ga[db][j] = atile_tr(gt, troff[db][0], troff[db][1], 2 * QB + j);
            qa[db][j] = atile_tr(qt, troff[db][0], troff[db][1], 2 * QB + j);
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        dvt[db] = mfma32(ga[db][0], pds[0], dvt[db]);
        dvt[db] = mfma32(ga[db][1], pds[1], dvt[db]);
        dkt[db] = mfma32(qa[db][0], pds[2], dkt[db]);
        dkt[db] = mfma32(qa[db][1], pds[3], dkt[db]);
    }
}

template <bool MASK>
__device__ __forceinline__ void dkdv_tile(lds_bf16* qt, lds_bf16* gt, lds_bf16* terms,
                                          const bf16x8 (&kreg)[4], const bf16x8 (&vreg)[4],
                                          const int (&roff)[4], const int (&troff)[2][2],
                                          bf16x8 bs, bf16x8 bd, int toff, f32x16 (&dvt)[2],
                                          f32x16 (&dkt)[2], int lim, float c_log2) {
    f32x16 s0, dp0, s1, dp1;
    bf16x8 pds0[4], pds1[4];
    dkdv_sdp<0>(qt, gt, terms, kreg, vreg, roff, bs, bd, toff, s0, dp0);
    dkdv_sdp<1>(qt, gt, terms, kreg, vreg, roff, bs, bd, toff, s1, dp1);
    dkdv_pds<0, MASK>(s0, dp0, lim, c_log2, pds0);
    dkdv_acc<0>(qt, gt, troff, pds0, dvt, dkt);
    dkdv_pds<1, MASK>(s1, dp1, lim, c_log2, pds1);
    dkdv_acc<1>(qt, gt, troff, pds1, dvt, dkt);
}

__global__ __launch_bounds__(256, CATTN_DKDV_WAVES_PER_SIMD) void attn_bwd_dkdv_bf16_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ dout, const float* __restrict__ ws,
    bf16* __restrict__ dqkv, int B, int T, int Tp, int H, int n_kt, float c_log2, float scale) {
    __shared__ DkdvSmem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;

    const int BH = B * H;
    const int blk = blockIdx.x;
    int kt, bh;
    if ((BH & 7) == 0) {
        const int per = BH >> 3, xcd = blk & 7, s = blk >> 3;
        kt = s / per;  // first key tiles carry the most query tiles
        bh = xcd * per + s % per;
    } else {
        kt = blk / BH;
        bh = blk % BH;
    }
    const int b = bh / H, h = bh - b * H;
    const int C = H * HEAD_DIM;
    const long long rs = 3LL * C;
    const TileLoader ld_rs = tile_loader(rs, wave, lane);
    const TileLoader ld_C = tile_loader(C, wave, lane);
    const bf16* qbase = qkv + (long long)b * T * rs + h * HEAD_DIM;
    const bf16* kbase = qbase + C;
    const bf16* vbase = qbase + 2 * C;
    const bf16* gbase = dout + (long long)b * T * C + h * HEAD_DIM;
    // This head's rows of MFMA terms (32 bytes each) in the workspace.
    const char* terms_rows = reinterpret_cast<const char*>(ws + 2LL * BH * Tp) + (long long)bh * Tp * 32;

    const int k0 = kt * KV_BN;
    const int kw = k0 + wave * 32;
    const int my_k = kw + l32;

    // Per-lane LDS offsets: row-major reads of rows qb*32 + l32, chunks 2kk + hf;
    // transposed reads for d blocks 0 and 1.
    int roff[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) roff[kk] = l32 * 64 + (((2 * kk + hf) ^ swz(l32)) << 3);
    int troff[2][2];
#pragma unroll
    for (int db = 0; db < 2; ++db) atile_tr_offsets(lane, db, &troff[db][0], &troff[db][1]);

    f32x16 dvt[2] = {zero16(), zero16()};  // dV^T, d blocks
    f32x16 dkt[2] = {zero16(), zero16()};  // dK^T / scale, d blocks

    const int qt_begin = k0 / KV_BM;
    const int n_it = (T + KV_BM - 1) / KV_BM - qt_begin;

    // Extra k-step operands: A = the row's terms (lane half 0: m, half 1: D),
    // read at toff; B = -1 on the first three k of the matching half.
    const int toff = hf * 256 + l32 * 8;  // row l32's m (hf 0) or D (hf 1) terms
    const bf16 m1 = (bf16)-1.0f, z0 = (bf16)0.0f;
    const bf16x8 neg3 = {m1, m1, m1, z0, z0, z0, z0, z0}, zero8 = {z0, z0, z0, z0, z0, z0, z0, z0};
    const bf16x8 bs = hf == 0 ? neg3 : zero8;
    const bf16x8 bd = hf == 0 ? zero8 : neg3;
    // Issue the loads of query tile `it` (relative) into stage `st`: Q and dO
    // by every wave, the tile's 2 KB of terms by waves 0 and 1 (1 KB each).
    // Wave-uniform LDS byte addresses of stage 0 (stage st sits st stages on).
    const unsigned int q_lds = atile_addr(sm.q[0]), g_lds = atile_addr(sm.g[0]);
    const unsigned int t_lds = atile_addr(sm.terms[0]);
    constexpr unsigned int STAGE_BYTES = ATILE_ELEMS * 2, TSTAGE_BYTES = KV_BM * 16 * 2;
    auto issue = [&](int it) {
        const unsigned int st = (unsigned int)it % NSTAGE;
        const int q0 = (qt_begin + it) * KV_BM;
        atile_load(q_lds + st * STAGE_BYTES, rows_rsrc(qbase, rs, q0, T), 0, ld_rs);
        atile_load(g_lds + st * STAGE_BYTES, rows_rsrc(gbase, C, q0, T), 0, ld_C);
        if (wave < 2)
            lds_dma16(terms_rows + (long long)(q0 + 32 * wave) * 32 + lane * 16,
                      __builtin_amdgcn_readfirstlane(t_lds + st * TSTAGE_BYTES + wave * 1024));
    };
#pragma unroll
    for (int j = 0; j < NSTAGE - 1; ++j)
        if (j < n_it) issue(j);

    // K and V of this lane's key as B operands (of S = Q K^T and dP = dO V^T).
    bf16x8 kreg[4], vreg[4];
    {
        const bool ok = my_k < T;
        const bf16* kp = kbase + (long long)my_k * rs + hf * 8;
        const bf16* vp = vbase + (long long)my_k * rs + hf * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            kreg[kk] = as_bf16x8(load16(kp + kk * 16, ok));
            vreg[kk] = as_bf16x8(load16(vp + kk * 16, ok));
        }
    }
    // The first tiles and K, V land before the loop (no waits on K, V inside it).
    wait_vmem<0>();

    // One query tile: wait for its loads, refill the ring, then the tile's
    // work. Only the first two tiles of a workgroup can precede a wave's keys
    // or hold its diagonal (keys are 128-aligned, query tiles 64 rows), so the
    // later tiles run in a loop of their own with no masking branch, which
    // keeps the accumulators in the same registers from tile to tile.
    static_assert(KV_BN == 2 * KV_BM, "diagonal within the first two tiles");
    auto step = [&](int it, auto maybe_diag) {
        if (it + 1 < n_it) {
            if (wave < 2) wait_vmem<5>();
            else wait_vmem<4>();
        } else {
            wait_vmem<0>();
        }
        __syncthreads();
        if (it + NSTAGE - 1 < n_it) issue(it + NSTAGE - 1);
        const int q0 = (qt_begin + it) * KV_BM;
        const unsigned int st = (unsigned int)it % NSTAGE;
        lds_bf16* qt = atile_view_at(q_lds + st * STAGE_BYTES);
        lds_bf16* gt = atile_view_at(g_lds + st * STAGE_BYTES);
        lds_bf16* terms = atile_view_at(t_lds + st * TSTAGE_BYTES);
        const int lim = my_k - q0 - 4 * hf;
        if (decltype(maybe_diag)::value) {
            if (q0 + KV_BM - 1 < kw) return;  // every query of the tile precedes this wave's keys
            if (q0 == (kw & ~(KV_BM - 1))) {  // the tile holding this wave's diagonal
                dkdv_tile<true>(qt, gt, terms, kreg, vreg, roff, troff, bs, bd, toff, dvt, dkt,
                                lim, c_log2);
                return;
            }
        }
        dkdv_tile<false>(qt, gt, terms, kreg, vreg, roff, troff, bs, bd, toff, dvt, dkt, lim,
                         c_log2);
    };
    const int n_head_it = n_it < 2 ? n_it : 2;
    for (int it = 0; it < n_head_it; ++it) step(it, std::true_type());
    for (int it = n_head_it; it < n_it; ++it) step(it, std::false_type());

    if (my_k < T) {
        bf16* dkp = dqkv + ((long long)b * T + my_k) * rs + C + h * HEAD_DIM;
        bf16* dvp = dkp + C;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = db * 32 + 8 * g4 + 4 * hf;
                const int i = 4 * g4;
                *reinterpret_cast<u32x2*>(dkp + d) =
                    to_bf16x4_bits(dkt[db][i] * scale, dkt[db][i + 1] * scale,
                                   dkt[db][i + 2] * scale, dkt[db][i + 3] * scale);
                *reinterpret_cast<u32x2*>(dvp + d) =
                    to_bf16x4_bits(dvt[db][i], dvt[db][i + 1], dvt[db][i + 2], dvt[db][i + 3]);
            }
    }
}

// The kernel the library launches for dK/dV: the same work as above with the
// wave's whole program scheduled by hand (attn_dkdv_asm.inc, written by
// gen_attn_dkdv_asm.py). The program pipelines 32-query halves: while the
// VALU forms P and dS of one half, the matrix cores take dV/dK of the half
// before it and S/dP of the half after it, each LDS operand read a few MFMAs
// ahead. C++ maps the workgroup to (key tile, head) as above and hands the
// program wave-uniform scalars.
#include "attn_dkdv_asm.inc"

__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_bf16_asm_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ dout, const float* __restrict__ ws,
    bf16* __restrict__ dqkv, int B, int T, int Tp, int H, int n_kt, float c_log2, float scale) {
    __shared__ DkdvSmem sm;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int BH = B * H;
    const int blk = blockIdx.x;
    int kt, bh;
    if ((BH & 7) == 0) {
        const int per = BH >> 3, xcd = blk & 7, s = blk >> 3;
        kt = s / per;
        bh = xcd * per + s % per;
    } else {
        kt = blk / BH;
        bh = blk % BH;
    }
    const int b = bh / H, h = bh - b * H;
    const int C = H * HEAD_DIM;
    const long long rs = 3LL * C;
    const int k0 = kt * KV_BN;
    const int kw = k0 + wave * 32;
    const int qt_begin = k0 / KV_BM;
    const int n_it = (T + KV_BM - 1) / KV_BM - qt_begin;
    const int q0 = qt_begin * KV_BM;
    typedef unsigned long long u64;
    const u64 q_at = (u64)(uintptr_t)(qkv + ((long long)b * T + q0) * rs + h * HEAD_DIM);
    const u64 q_left = (u64)(T - q0) * (u64)rs * 2;
    const u64 g_at = (u64)(uintptr_t)(dout + ((long long)b * T + q0) * C + h * HEAD_DIM);
    const u64 g_left = (u64)(T - q0) * (u64)C * 2;
    const u64 t_at = (u64)(uintptr_t)(reinterpret_cast<const char*>(ws + 2LL * BH * Tp) +
                                      ((long long)bh * Tp + q0) * 32 + wave * 1024);
    const u64 k_row = (u64)(uintptr_t)(qkv + ((long long)b * T + kw) * rs + C + h * HEAD_DIM);
    const u64 dk_row = (u64)(uintptr_t)(dqkv + ((long long)b * T + kw) * rs + C + h * HEAD_DIM);
    const unsigned int q_lds = atile_addr(sm.q[0]);
    asm volatile(CATTN_DKDV_ASM_BODY
                 :
                 : [qlds] "s"(q_lds), [qldw] "s"(q_lds + 2048u * wave),
                   [tldw] "s"(q_lds + 1024u * wave), [wave] "s"(wave), [wave16] "s"(16 * wave),
                   [rs2] "s"((unsigned int)(rs * 2)), [c2] "s"((unsigned int)(C * 2)),
                   [qtb] "s"((unsigned int)(KV_BM * rs * 2)), [gtb] "s"((unsigned int)(KV_BM * C * 2)),
                   [qat_lo] "s"((unsigned int)q_at), [qat_hi] "s"((unsigned int)(q_at >> 32)),
                   [qleft_lo] "s"((unsigned int)q_left), [qleft_hi] "s"((unsigned int)(q_left >> 32)),
                   [gat_lo] "s"((unsigned int)g_at), [gat_hi] "s"((unsigned int)(g_at >> 32)),
                   [gleft_lo] "s"((unsigned int)g_left), [gleft_hi] "s"((unsigned int)(g_left >> 32)),
                   [tat_lo] "s"((unsigned int)t_at), [tat_hi] "s"((unsigned int)(t_at >> 32)),
                   [nit] "s"(n_it), [nk] "s"(T - kw), [lim0] "s"(32 * (wave & 1)),
                   [cbits] "s"(__builtin_bit_cast(unsigned int, c_log2)),
                   [sbits] "s"(__builtin_bit_cast(unsigned int, scale)),
                   [kbase] "s"(k_row), [vbase] "s"(k_row + 2ull * C),
                   [dkbase] "s"(dk_row), [dvbase] "s"(dk_row + 2ull * C)
                 : CATTN_DKDV_ASM_CLOBBERS, "vcc", "m0", "scc", "exec", "memory");
}

// ---------------------------------------------------------------------------
// dQ. One workgroup = 4 waves = 128 queries of one (batch, head); wave w owns
// queries q0 + 32w .. +31 with Q, dO, LSE*log2 e and D of its query in
// registers. Key tiles of 64 rows (K and V) stream through a three-stage ring
// of LDS buffers filled by direct global->LDS loads. Per tile and wave:
// S^T = K Q^T and dP^T = V dO^T on MFMA (lane l%32 owns query l%32), P^T and
// dS^T in registers, dQ^T += K^T dS^T on MFMA with K^T read from the
// row-major K tile by transposing LDS reads.
// ---------------------------------------------------------------------------
constexpr int DQ_BM = 128;  // queries per workgroup
constexpr int DQ_BN = 64;   // keys per LDS tile

struct DqSmem {
    bf16 k[NSTAGE][ATILE_ELEMS];
    bf16 v[NSTAGE][ATILE_ELEMS];
};

// One 32-key half (KB) of a key tile for the dQ kernel: S^T and dP^T on
// MFMA, P^T and dS^T on the VALU, then dQ^T += K^T dS^T. MASK applies the
// causal mask (the tile holding this wave's diagonal only).
template <int KB, bool MASK>
__device__ __forceinline__ void dq_half(lds_bf16* kt, lds_bf16* vt, const bf16x8 (&qreg)[4],
                                        const bf16x8 (&greg)[4], const int (&roff)[4],
                                        const int (&troff)[2][2], f32x16 (&dqt)[2], int lim,
                                        float lse2, float dd, float c_log2) {
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int o = KB * 32 * 64 + roff[kk];
        s = mfma32(*reinterpret_cast<lds_bf16x8*>(kt + o), qreg[kk], s);
        dp = mfma32(*reinterpret_cast<lds_bf16x8*>(vt + o), greg[kk], dp);
    }
    if (MASK) {  // key KB*32 + 8(i/4) + 4hf + (i%4) > my_q - k0  ->  P = 0
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (KB * 32 + 8 * (i >> 2) + (i & 3) > lim) s[i] = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[i], c_log2, -lse2));
        dp[i] = p * (dp[i] - dd);
    }
    const bf16x8 ds0 = c_rows_to_operand(dp, 0), ds1 = c_rows_to_operand(dp, 1);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        dqt[db] = mfma32(atile_tr(kt, troff[db][0], troff[db][1], 2 * KB), ds0, dqt[db]);
        dqt[db] = mfma32(atile_tr(kt, troff[db][0], troff[db][1], 2 * KB + 1), ds1, dqt[db]);
    }
}

template <bool MASK>
__device__ __forceinline__ void dq_tile(lds_bf16* kt, lds_bf16* vt, const bf16x8 (&qreg)[4],
                                        const bf16x8 (&greg)[4], const int (&roff)[4],
                                        const int (&troff)[2][2], f32x16 (&dqt)[2], int lim,
                                        float lse2, float dd, float c_log2) {
    dq_half<0, MASK>(kt, vt, qreg, greg, roff, troff, dqt, lim, lse2, dd, c_log2);
    dq_half<1, MASK>(kt, vt, qreg, greg, roff, troff, dqt, lim, lse2, dd, c_log2);
}

// FUSED_PRE: also compute D and LSE * log2 e of this workgroup's rows from
// dout, out and lse (instead of reading them from the workspace) and write
// them, with the padding, to the workspace for the dK/dV kernel.
template <bool FUSED_PRE>
__global__ __launch_bounds__(256) void attn_bwd_dq_bf16_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ dout, const bf16* __restrict__ out,
    const float* __restrict__ lse, float* __restrict__ ws, bf16* __restrict__ dqkv, int B, int T,
    int Tp, int H, int n_qt, float c_log2, float scale) {
    __shared__ DqSmem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;

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
    const long long rs = 3LL * C;
    const TileLoader ld_rs = tile_loader(rs, wave, lane);
    const bf16* qbase = qkv + (long long)b * T * rs + h * HEAD_DIM;
    const bf16* kbase = qbase + C;
    const bf16* gbase = dout + (long long)b * T * C + h * HEAD_DIM;

    const int q0 = qt * DQ_BM;
    const int qw = q0 + wave * 32;
    const int my_q = qw + l32;
    const bool q_ok = my_q < T;

    int roff[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) roff[kk] = l32 * 64 + (((2 * kk + hf) ^ swz(l32)) << 3);
    int troff[2][2];
#pragma unroll
    for (int db = 0; db < 2; ++db) atile_tr_offsets(lane, db, &troff[db][0], &troff[db][1]);

    f32x16 dqt[2] = {zero16(), zero16()};  // dQ^T / scale, d blocks

    const int kend = min(q0 + DQ_BM, T);
    const int n_kt = (kend + DQ_BN - 1) / DQ_BN;

    // K and V rows [k0, k0 + 64) into stage st: one descriptor, since V sits
    // C elements after K in every packed row.
    const unsigned int k_lds = atile_addr(sm.k[0]), v_lds = atile_addr(sm.v[0]);
    constexpr unsigned int STAGE_BYTES = ATILE_ELEMS * 2;
    auto issue = [&](int t) {
        const unsigned int st = (unsigned int)t % NSTAGE;
        const i32x4 kv = rows_rsrc(kbase, rs, t * DQ_BN, T);
        atile_load(k_lds + st * STAGE_BYTES, kv, 0, ld_rs);
        atile_load(v_lds + st * STAGE_BYTES, kv, 2u * C, ld_rs);
    };
#pragma unroll
    for (int j = 0; j < NSTAGE - 1; ++j)
        if (j < n_kt) issue(j);

    bf16x8 qreg[4], greg[4];
    {
        const bf16* qp = qbase + (long long)my_q * rs + hf * 8;
        const bf16* gp = gbase + (long long)my_q * C + hf * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            qreg[kk] = as_bf16x8(load16(qp + kk * 16, q_ok));
            greg[kk] = as_bf16x8(load16(gp + kk * 16, q_ok));
        }
    }
    float dd, lse2;
    if (FUSED_PRE) {
        bf16x8 oreg[4];
        const bf16* op = out + ((long long)b * T + my_q) * C + h * HEAD_DIM + hf * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) oreg[kk] = as_bf16x8(load16(op + kk * 16, q_ok));
        const float part = dot_half(greg, oreg);  // zero past T
        dd = part + swap_halves(part);
        lse2 = q_ok ? lse[(long long)bh * T + my_q] * LOG2E : INFINITY;
    } else {
        const long long ws_i = (long long)bh * Tp + min(my_q, Tp - 1);
        dd = q_ok ? ws[ws_i] : 0.0f;
        lse2 = q_ok ? ws[(long long)BH * Tp + ws_i] : INFINITY;
    }
    // The first tiles and this lane's Q, dO, LSE, D land before the loop.
    wait_vmem<0>();

    for (int j = 0; j < n_kt; ++j) {
        if (j + 1 < n_kt) wait_vmem<4>();
        else wait_vmem<0>();
        __syncthreads();
        if (j + NSTAGE - 1 < n_kt) issue(j + NSTAGE - 1);
        const int k0 = j * DQ_BN;
        if (k0 > qw + 31) continue;  // whole tile after this wave's queries
        const unsigned int st = (unsigned int)j % NSTAGE;
        lds_bf16* kt = atile_view_at(k_lds + st * STAGE_BYTES);
        lds_bf16* vt = atile_view_at(v_lds + st * STAGE_BYTES);
        const int lim = my_q - k0 - 4 * hf;
        if (k0 == (qw & ~(DQ_BN - 1)))  // the tile holding this wave's diagonal
            dq_tile<true>(kt, vt, qreg, greg, roff, troff, dqt, lim, lse2, dd, c_log2);
        else
            dq_tile<false>(kt, vt, qreg, greg, roff, troff, dqt, lim, lse2, dd, c_log2);
    }

    // The workspace rows of this workgroup, written last (the dK/dV kernel
    // reads them after this kernel has finished): D, LSE * log2 e and their
    // MFMA terms, with the padding past T.
    if (FUSED_PRE && hf == 0 && my_q < Tp) {
        const long long r = (long long)bh * Tp + my_q;
        ws[r] = dd;
        ws[(long long)BH * Tp + r] = lse2;
        u32x4* terms = ws_terms(ws, (long long)BH * Tp);
        terms[term_m(r)] = q_ok ? mfma_terms(8.0f * lse[(long long)bh * T + my_q]) : mfma_terms_pad();
        terms[term_d(r)] = mfma_terms(dd);
    }

    if (q_ok) {
        bf16* dqp = dqkv + ((long long)b * T + my_q) * rs + h * HEAD_DIM;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = db * 32 + 8 * g4 + 4 * hf;
                const int i = 4 * g4;
                *reinterpret_cast<u32x2*>(dqp + d) =
                    to_bf16x4_bits(dqt[db][i] * scale, dqt[db][i + 1] * scale,
                                   dqt[db][i + 2] * scale, dqt[db][i + 3] * scale);
            }
    }
}

// The kernel the library launches for dQ with the preprocess: the wave's
// whole program scheduled by hand (attn_dq_asm.inc, written by
// gen_attn_dq_asm.py). It forms D and LSE * log2 e of its queries (the same
// fmaf chain as the preprocess kernel, so the workspace matches it bit for
// bit), stores the workspace rows while the tile loop runs, and pipelines
// 32-key halves as the dK/dV program does: the scores and dP of one half and
// dQ of another on MFMA while P and dS of the half between run on the VALU.
#include "attn_dq_asm.inc"

__global__ __launch_bounds__(256, 3) void attn_bwd_dq_pre_bf16_asm_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ dout, const bf16* __restrict__ out,
    const float* __restrict__ lse, float* __restrict__ ws, bf16* __restrict__ dqkv, int B, int T,
    int Tp, int H, int n_qt, float c_log2, float scale) {
    __shared__ DqSmem sm;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int l32 = lane & 31, hf = lane >> 5;
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
    const long long rs = 3LL * C;
    const int q0 = qt * DQ_BM;
    const int qw = q0 + wave * 32;
    const int my_q = qw + l32;
    const bool q_ok = my_q < T;

    const int kend = min(q0 + DQ_BM, T);
    const int n_kt = (kend + DQ_BN - 1) / DQ_BN;
    const int k1 = min(qw / 32, 2 * n_kt - 1);  // this wave's last (diagonal) half
    typedef unsigned long long u64;
    const u64 k_at = (u64)(uintptr_t)(qkv + (long long)b * T * rs + C + h * HEAD_DIM);
    const u64 k_left = (u64)T * (u64)rs * 2;
    const u64 q_row = (u64)(uintptr_t)(qkv + ((long long)b * T + qw) * rs + h * HEAD_DIM);
    const u64 g_row = (u64)(uintptr_t)(dout + ((long long)b * T + qw) * C + h * HEAD_DIM);
    const u64 dq_row = (u64)(uintptr_t)(dqkv + ((long long)b * T + qw) * rs + h * HEAD_DIM);
    const u64 o_row = (u64)(uintptr_t)(out + ((long long)b * T + qw) * C + h * HEAD_DIM);
    const u64 l_row = (u64)(uintptr_t)(lse + (long long)bh * T + qw);
    // this wave's workspace rows: D, LSE log2 e, and the 32-byte term rows
    const long long r0 = (long long)bh * Tp + qw;
    const u64 wsd = (u64)(uintptr_t)(ws + r0);
    const u64 wsl = (u64)(uintptr_t)(ws + (long long)BH * Tp + r0);
    const u64 wst = (u64)(uintptr_t)(reinterpret_cast<const char*>(ws + 2LL * BH * Tp) + r0 * 32);
    const unsigned int k_lds = atile_addr(sm.k[0]);
    asm volatile(CATTN_DQ_ASM_BODY
                 :
                 : [klds] "s"(k_lds), [kldw] "s"(k_lds + 2048u * wave), [wave16] "s"(16 * wave),
                   [rs2] "s"((unsigned int)(rs * 2)), [c2] "s"((unsigned int)(C * 2)),
                   [voffs] "s"((unsigned int)(C * 2)),
                   [tbytes] "s"((unsigned int)(DQ_BN * rs * 2)),
                   [kat_lo] "s"((unsigned int)k_at), [kat_hi] "s"((unsigned int)(k_at >> 32)),
                   [kleft_lo] "s"((unsigned int)k_left), [kleft_hi] "s"((unsigned int)(k_left >> 32)),
                   [nkt] "s"(n_kt), [k1] "s"(k1), [limb] "s"(qw - 32 * k1), [nq] "s"(T - qw),
                   [cbits] "s"(__builtin_bit_cast(unsigned int, c_log2)),
                   [sbits] "s"(__builtin_bit_cast(unsigned int, scale)),
                   [qbase] "s"(q_row), [gbase] "s"(g_row), [dqbase] "s"(dq_row),
                   [obase] "s"(o_row),
                   [lbase_lo] "s"(__builtin_amdgcn_readfirstlane((unsigned int)l_row)),
                   [lbase_hi] "s"(__builtin_amdgcn_readfirstlane((unsigned int)(l_row >> 32))),
                   [wsd_lo] "s"(__builtin_amdgcn_readfirstlane((unsigned int)wsd)),
                   [wsd_hi] "s"(__builtin_amdgcn_readfirstlane((unsigned int)(wsd >> 32))),
                   [wsl_lo] "s"(__builtin_amdgcn_readfirstlane((unsigned int)wsl)),
                   [wsl_hi] "s"(__builtin_amdgcn_readfirstlane((unsigned int)(wsl >> 32))),
                   [wst_lo] "s"(__builtin_amdgcn_readfirstlane((unsigned int)wst)),
                   [wst_hi] "s"(__builtin_amdgcn_readfirstlane((unsigned int)(wst >> 32))),
                   [nw] "s"(min(32, Tp - qw))
                 : CATTN_DQ_ASM_CLOBBERS, "vcc", "m0", "scc", "exec", "memory");
}

}  // namespace

int bwd_padded_rows(int T) { return (T + ROW_PAD - 1) / ROW_PAD * ROW_PAD; }

hipError_t launch_attn_bwd_pre_bf16(const void* dout, const void* out, const float* lse, float* ws,
                                    int B, int T, int H, hipStream_t stream) {
    const int Tp = bwd_padded_rows(T);
    const long long n_rows = (long long)B * T * H;
    const long long nb_d = (n_rows + 127) / 128;
    const long long n_pad_rows = (long long)B * H * Tp;
    const long long nb_l = (n_pad_rows + 255) / 256;
    hipLaunchKernelGGL(attn_bwd_pre_bf16_kernel, dim3((unsigned)(nb_d + nb_l)), dim3(256), 0,
                       stream, static_cast<const bf16*>(dout), static_cast<const bf16*>(out), lse,
                       ws, T, Tp, H, n_rows, nb_d, n_pad_rows);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv_bf16(const void* qkv, const void* dout, const float* ws, void* dqkv,
                                     int B, int T, int H, hipStream_t stream) {
    const int n_kt = (T + KV_BN - 1) / KV_BN;
    const long long blocks = (long long)B * H * n_kt;
#ifdef CATTN_DKDV_COMPILED
    hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
#else
    hipLaunchKernelGGL(attn_bwd_dkdv_bf16_asm_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
#endif
                       static_cast<const bf16*>(qkv), static_cast<const bf16*>(dout), ws,
                       static_cast<bf16*>(dqkv), B, T, bwd_padded_rows(T), H, n_kt,
                       LOG2E / 8.0f, 0.125f);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dq_bf16(const void* qkv, const void* dout, const float* ws, void* dqkv,
                                   int B, int T, int H, hipStream_t stream) {
    const int n_qt = (T + DQ_BM - 1) / DQ_BM;
    const long long blocks = (long long)B * H * n_qt;
    hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16*>(qkv), static_cast<const bf16*>(dout), nullptr,
                       nullptr, const_cast<float*>(ws), static_cast<bf16*>(dqkv), B, T,
                       bwd_padded_rows(T), H, n_qt, LOG2E / 8.0f, 0.125f);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dq_pre_bf16(const void* qkv, const void* dout, const void* out,
                                       const float* lse, float* ws, void* dqkv, int B, int T,
                                       int H, hipStream_t stream) {
    const int n_qt = (T + DQ_BM - 1) / DQ_BM;
    const long long blocks = (long long)B * H * n_qt;
#ifdef CATTN_DQ_COMPILED
    hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
#else
    hipLaunchKernelGGL(attn_bwd_dq_pre_bf16_asm_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       stream,
#endif
                       static_cast<const bf16*>(qkv), static_cast<const bf16*>(dout),
                       static_cast<const bf16*>(out), lse, ws, static_cast<bf16*>(dqkv), B, T,
                       bwd_padded_rows(T), H, n_qt, LOG2E / 8.0f, 0.125f);
    return hipGetLastError();
}

}  // namespace cattn
