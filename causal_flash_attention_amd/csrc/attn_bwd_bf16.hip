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
#include "attn_common.h"

namespace cattn {
namespace {

// ---------------------------------------------------------------------------
// D[b, h, t] = sum_k dO[b, t, h, k] * O[b, t, h, k]; 8 lanes per (b, t, h).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_bwd_pre_bf16_kernel(
    const bf16* __restrict__ dout, const bf16* __restrict__ out, float* __restrict__ delta,
    int T, int H, long long n_rows) {
    const long long row = (long long)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int part = threadIdx.x & 7;
    float acc = 0.0f;
    if (row < n_rows) {
        const long long off = row * HEAD_DIM + part * 8;  // rows are (b, t, h) in memory order
        const bf16x8 g = as_bf16x8(*reinterpret_cast<const u32x4*>(dout + off));
        const bf16x8 o = as_bf16x8(*reinterpret_cast<const u32x4*>(out + off));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)g[e], (float)o[e], acc);
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 4, 64);
    if (row < n_rows && part == 0) {
        const long long bt = row / H;
        const int h = (int)(row - bt * H);
        const long long b = bt / T;
        const int t = (int)(bt - b * T);
        delta[(b * H + h) * T + t] = acc;
    }
}

// ---------------------------------------------------------------------------
// dK, dV. One workgroup = 4 waves = 128 keys of one (batch, head); wave w owns
// keys k0 + 32w .. +31, with K and V of those keys held in registers. Query
// tiles of 64 rows stream through double-buffered LDS as Q, Q^T, dO, dO^T,
// LSE*log2(e) and D. Per tile and wave: S = Q K^T and dP = dO V^T on MFMA
// (lane l%32 owns key l%32), P and dS in registers, then
// dV^T += dO^T P and dK^T += Q^T dS on MFMA with P and dS fed straight from
// registers. Query tiles entirely before a wave's keys are skipped.
// ---------------------------------------------------------------------------
constexpr int KV_BN = 128;  // keys per workgroup
constexpr int KV_BM = 64;   // queries per LDS tile

struct DkdvSmem {
    bf16 q[2][KV_BM * LDS_ROW];
    bf16 qt[2][HEAD_DIM * LDS_ROW];
    bf16 g[2][KV_BM * LDS_ROW];
    bf16 gt[2][HEAD_DIM * LDS_ROW];
    float lse2[2][KV_BM];
    float dd[2][KV_BM];
};

__device__ __forceinline__ void stage_rowstats(float* lse2_s, float* dd_s, const float* lse_row,
                                               const float* d_row, int q0, int T, int tid) {
    if (tid < KV_BM) {
        const int q = q0 + tid;
        lse2_s[tid] = q < T ? lse_row[q] * LOG2E : INFINITY;  // P = 0 past the end
        dd_s[tid] = q < T ? d_row[q] : 0.0f;
    }
}

__global__ __launch_bounds__(256) void attn_bwd_dkdv_bf16_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, bf16* __restrict__ dqkv, int B, int T, int H, int n_kt,
    float c_log2, float scale) {
    __shared__ DkdvSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    const bf16* qbase = qkv + (long long)b * T * rs + h * HEAD_DIM;
    const bf16* kbase = qbase + C;
    const bf16* vbase = qbase + 2 * C;
    const bf16* gbase = dout + (long long)b * T * C + h * HEAD_DIM;
    const float* lse_row = lse + (long long)bh * T;
    const float* d_row = delta + (long long)bh * T;

    const int k0 = kt * KV_BN;
    const int kw = k0 + wave * 32;
    const int my_k = kw + l32;

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

    f32x16 dvt[2] = {zero16(), zero16()};  // dV^T, d blocks
    f32x16 dkt[2] = {zero16(), zero16()};  // dK^T / scale, d blocks

    const int qt_begin = k0 / KV_BM;
    const int qt_end = (T + KV_BM - 1) / KV_BM;

    {
        const int q0 = qt_begin * KV_BM;
        TilePair tq = load_tile_pair(qbase, rs, q0, T, tid);
        TilePair tg = load_tile_pair(gbase, C, q0, T, tid);
        store_tile_rows(sm.q[0], tq, tid);
        store_tile_transposed(sm.qt[0], tq, tid);
        store_tile_rows(sm.g[0], tg, tid);
        store_tile_transposed(sm.gt[0], tg, tid);
        stage_rowstats(sm.lse2[0], sm.dd[0], lse_row, d_row, q0, T, tid);
    }
    __syncthreads();

    for (int it = qt_begin; it < qt_end; ++it) {
        const int buf = (it - qt_begin) & 1;
        const int q0 = it * KV_BM;
        const bool has_next = it + 1 < qt_end;
        TilePair nq, ng;
        if (has_next) {
            nq = load_tile_pair(qbase, rs, q0 + KV_BM, T, tid);
            ng = load_tile_pair(gbase, C, q0 + KV_BM, T, tid);
        }
        if (q0 + KV_BM - 1 >= kw) {
            // S = Q K^T and dP = dO V^T : two 32-query blocks each.
            f32x16 s[2], dp[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                s[qb] = zero16();
                dp[qb] = zero16();
                const bf16* qp = sm.q[buf] + (qb * 32 + l32) * LDS_ROW + hf * 8;
                const bf16* gp = sm.g[buf] + (qb * 32 + l32) * LDS_ROW + hf * 8;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    s[qb] = mfma32(lds_read8(qp + kk * 16), kreg[kk], s[qb]);
                    dp[qb] = mfma32(lds_read8(gp + kk * 16), vreg[kk], dp[qb]);
                }
            }
            // P = exp2(c*s - LSE*log2 e), masked where key > query; dS = P (dP - D).
            const bool need_mask = q0 < kw + 31;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int qi = qb * 32 + 8 * g4 + 4 * hf;
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][qi]);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dd[buf][qi]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 4 * g4 + r;
                        float p = fast_exp2(fmaf(s[qb][i], c_log2, -l4[r]));
                        if (need_mask && my_k > q0 + qi + r) p = 0.0f;
                        s[qb][i] = p;
                        dp[qb][i] = p * (dp[qb][i] - d4[r]);
                    }
                }
            bf16x8 pb[4], dsb[4];
#pragma unroll
            for (int qc = 0; qc < 4; ++qc) {
                pb[qc] = c_rows_to_operand(s[qc >> 1], qc & 1);
                dsb[qc] = c_rows_to_operand(dp[qc >> 1], qc & 1);
            }
            // dV^T += dO^T P, dK^T += Q^T dS : K = 64 queries in four chunks.
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const bf16* gtp = sm.gt[buf] + (db * 32 + l32) * LDS_ROW + hf * 8;
                const bf16* qtp = sm.qt[buf] + (db * 32 + l32) * LDS_ROW + hf * 8;
#pragma unroll
                for (int qc = 0; qc < 4; ++qc) {
                    dvt[db] = mfma32(lds_read8(gtp + qc * 16), pb[qc], dvt[db]);
                    dkt[db] = mfma32(lds_read8(qtp + qc * 16), dsb[qc], dkt[db]);
                }
            }
        }
        if (has_next) {
            const int nb = buf ^ 1;
            store_tile_rows(sm.q[nb], nq, tid);
            store_tile_transposed(sm.qt[nb], nq, tid);
            store_tile_rows(sm.g[nb], ng, tid);
            store_tile_transposed(sm.gt[nb], ng, tid);
            stage_rowstats(sm.lse2[nb], sm.dd[nb], lse_row, d_row, q0 + KV_BM, T, tid);
        }
        __syncthreads();
    }

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

// ---------------------------------------------------------------------------
// dQ. One workgroup = 4 waves = 128 queries of one (batch, head); wave w owns
// queries q0 + 32w .. +31 with Q, dO, LSE and D of its query in registers.
// Key tiles of 64 rows stream through double-buffered LDS as K, K^T and V.
// Per tile and wave: S^T = K Q^T and dP^T = V dO^T on MFMA (lane l%32 owns
// query l%32), P^T and dS^T in registers, dQ^T += K^T dS^T on MFMA.
// ---------------------------------------------------------------------------
constexpr int DQ_BM = 128;  // queries per workgroup
constexpr int DQ_BN = 64;   // keys per LDS tile

struct DqSmem {
    bf16 k[2][DQ_BN * LDS_ROW];
    bf16 kt[2][HEAD_DIM * LDS_ROW];
    bf16 v[2][DQ_BN * LDS_ROW];
};

__global__ __launch_bounds__(256) void attn_bwd_dq_bf16_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, bf16* __restrict__ dqkv, int B, int T, int H, int n_qt,
    float c_log2, float scale) {
    __shared__ DqSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    const bf16* qbase = qkv + (long long)b * T * rs + h * HEAD_DIM;
    const bf16* kbase = qbase + C;
    const bf16* vbase = qbase + 2 * C;
    const bf16* gbase = dout + (long long)b * T * C + h * HEAD_DIM;

    const int q0 = qt * DQ_BM;
    const int qw = q0 + wave * 32;
    const int my_q = qw + l32;
    const bool q_ok = my_q < T;

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
    const float lse2 = q_ok ? lse[(long long)bh * T + my_q] * LOG2E : INFINITY;
    const float dd = q_ok ? delta[(long long)bh * T + my_q] : 0.0f;

    f32x16 dqt[2] = {zero16(), zero16()};  // dQ^T / scale, d blocks

    const int kend = min(q0 + DQ_BM, T);
    const int n_kt = (kend + DQ_BN - 1) / DQ_BN;

    {
        TilePair tk = load_tile_pair(kbase, rs, 0, T, tid);
        TilePair tv = load_tile_pair(vbase, rs, 0, T, tid);
        store_tile_rows(sm.k[0], tk, tid);
        store_tile_transposed(sm.kt[0], tk, tid);
        store_tile_rows(sm.v[0], tv, tid);
    }
    __syncthreads();

    for (int j = 0; j < n_kt; ++j) {
        const int buf = j & 1;
        const int k0 = j * DQ_BN;
        const bool has_next = j + 1 < n_kt;
        TilePair nk, nv;
        if (has_next) {
            nk = load_tile_pair(kbase, rs, k0 + DQ_BN, T, tid);
            nv = load_tile_pair(vbase, rs, k0 + DQ_BN, T, tid);
        }
        if (k0 <= qw + 31) {
            f32x16 s[2], dp[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = zero16();
                dp[kb] = zero16();
                const bf16* kp = sm.k[buf] + (kb * 32 + l32) * LDS_ROW + hf * 8;
                const bf16* vp = sm.v[buf] + (kb * 32 + l32) * LDS_ROW + hf * 8;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    s[kb] = mfma32(lds_read8(kp + kk * 16), qreg[kk], s[kb]);
                    dp[kb] = mfma32(lds_read8(vp + kk * 16), greg[kk], dp[kb]);
                }
            }
            const bool need_mask = k0 + DQ_BN - 1 > qw;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float p = fast_exp2(fmaf(s[kb][i], c_log2, -lse2));
                    if (need_mask) {
                        const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                        if (key > my_q) p = 0.0f;
                    }
                    dp[kb][i] = p * (dp[kb][i] - dd);
                }
            bf16x8 dsb[4];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) dsb[kc] = c_rows_to_operand(dp[kc >> 1], kc & 1);
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const bf16* ktp = sm.kt[buf] + (db * 32 + l32) * LDS_ROW + hf * 8;
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) dqt[db] = mfma32(lds_read8(ktp + kc * 16), dsb[kc], dqt[db]);
            }
        }
        if (has_next) {
            const int nb = buf ^ 1;
            store_tile_rows(sm.k[nb], nk, tid);
            store_tile_transposed(sm.kt[nb], nk, tid);
            store_tile_rows(sm.v[nb], nv, tid);
        }
        __syncthreads();
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

}  // namespace

hipError_t launch_attn_bwd_pre_bf16(const void* dout, const void* out, float* delta, int B, int T,
                                    int H, hipStream_t stream) {
    const long long n_rows = (long long)B * T * H;
    const long long blocks = (n_rows + 31) / 32;
    hipLaunchKernelGGL(attn_bwd_pre_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16*>(dout), static_cast<const bf16*>(out), delta, T, H,
                       n_rows);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv_bf16(const void* qkv, const void* dout, const float* lse,
                                     const float* delta, void* dqkv, int B, int T, int H,
                                     hipStream_t stream) {
    const int n_kt = (T + KV_BN - 1) / KV_BN;
    const long long blocks = (long long)B * H * n_kt;
    hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16*>(qkv), static_cast<const bf16*>(dout), lse, delta,
                       static_cast<bf16*>(dqkv), B, T, H, n_kt, LOG2E / 8.0f, 0.125f);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dq_bf16(const void* qkv, const void* dout, const float* lse,
                                   const float* delta, void* dqkv, int B, int T, int H,
                                   hipStream_t stream) {
    const int n_qt = (T + DQ_BM - 1) / DQ_BM;
    const long long blocks = (long long)B * H * n_qt;
    hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16*>(qkv), static_cast<const bf16*>(dout), lse, delta,
                       static_cast<bf16*>(dqkv), B, T, H, n_qt, LOG2E / 8.0f, 0.125f);
    return hipGetLastError();
}

}  // namespace cattn
