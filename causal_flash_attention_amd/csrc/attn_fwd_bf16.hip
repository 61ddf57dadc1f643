// Causal attention forward, bf16 storage, fp32 accumulation, MFMA (gfx950).
//
// Computes O = softmax(scale * Q K^T + causal mask) V and LSE per row without
// ever holding the T x T score matrix in memory: the FlashAttention method of
// "Let's reproduce GPT-2 (124M)" (chapter list, 02:00:18; glossary table of
// the theprofessional.online summary, row "flash attention"), written for
// CDNA4 from the definition rather than from any published kernel.
//
// One workgroup = 4 waves = 128 queries of one (batch, head); wave w owns
// queries q0 + 32w .. q0 + 32w + 31. Key/value tiles of 64 rows stream
// through double-buffered LDS (K row-major, V transposed). Per tile, each
// wave computes S^T = K Q^T on MFMA (so that lane l%32 owns query l%32 and
// the row statistics are per lane), applies the causal mask only on tiles
// that straddle its diagonal, updates the running max / sum in base 2, and
// accumulates O^T += V^T P^T on MFMA with P^T fed straight from registers.
// Tiles entirely above a wave's diagonal are skipped.
#include "attn_common.h"

namespace cattn {
namespace {

constexpr int FWD_BM = 128;  // queries per workgroup
constexpr int FWD_BN = 64;   // keys per LDS tile

struct FwdSmem {
    bf16 k[2][FWD_BN * LDS_ROW];     // K tile, row-major [key][d]
    bf16 vt[2][HEAD_DIM * LDS_ROW];  // V tile, transposed [d][perm16(key)]
};

__global__ __launch_bounds__(256) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ qkv, bf16* __restrict__ out, float* __restrict__ lse,
    int B, int T, int H, int n_qt, float c_log2) {
    __shared__ FwdSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;

    // Workgroup -> (query tile, head): heaviest (last) query tiles first;
    // when the head count allows, the heads are split into 8 contiguous
    // groups, one per XCD, so that K/V of a head stay in one L2.
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
    const long long rs = 3LL * C;  // qkv token stride, elements
    const bf16* qbase = qkv + (long long)b * T * rs + h * HEAD_DIM;
    const bf16* kbase = qbase + C;
    const bf16* vbase = qbase + 2 * C;

    const int q0 = qt * FWD_BM;
    const int qw = q0 + wave * 32;
    const int my_q = qw + l32;

    // Q^T operand (B of S^T = K Q^T): d = 16kk + 8hf .. +7 of query my_q.
    bf16x8 qreg[4];
    {
        const bool ok = my_q < T;
        const bf16* p = qbase + (long long)my_q * rs + hf * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qreg[kk] = as_bf16x8(load16(p + kk * 16, ok));
    }

    const int kend = min(q0 + FWD_BM, T);
    const int n_kt = (kend + FWD_BN - 1) / FWD_BN;

    float m_run = -INFINITY;  // running max of scale*log2(e)*s
    float l_run = 0.0f;       // this lane half's share of the running sum
    f32x16 acc[2] = {zero16(), zero16()};  // O^T, d blocks 0..31 and 32..63

    {
        TilePair kt = load_tile_pair(kbase, rs, 0, T, tid);
        TilePair vt = load_tile_pair(vbase, rs, 0, T, tid);
        store_tile_rows(sm.k[0], kt, tid);
        store_tile_transposed(sm.vt[0], vt, tid);
    }
    __syncthreads();

    for (int j = 0; j < n_kt; ++j) {
        const int buf = j & 1;
        const int k0 = j * FWD_BN;
        const bool has_next = j + 1 < n_kt;
        TilePair nk, nv;
        if (has_next) {
            nk = load_tile_pair(kbase, rs, k0 + FWD_BN, T, tid);
            nv = load_tile_pair(vbase, rs, k0 + FWD_BN, T, tid);
        }
        if (k0 <= qw + 31) {
            // S^T = K Q^T : two 32-key blocks.
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = zero16();
                const bf16* kp = sm.k[buf] + (kb * 32 + l32) * LDS_ROW + hf * 8;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) s[kb] = mfma32(lds_read8(kp + kk * 16), qreg[kk], s[kb]);
            }
            if (k0 + FWD_BN - 1 > qw) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                        if (key > my_q) s[kb][i] = -INFINITY;
                    }
            }
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
            mx = fmaxf(mx, swap_halves(mx));
            const float m_new = fmaxf(m_run, mx * c_log2);
            const float alpha = fast_exp2(m_run - m_new);
            float rsum = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(fmaf(s[kb][i], c_log2, -m_new));
                    s[kb][i] = p;
                    rsum += p;
                }
            l_run = fmaf(l_run, alpha, rsum);
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;

            // O^T += V^T P^T over four 16-key chunks.
            bf16x8 pb[4];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) pb[kc] = c_rows_to_operand(s[kc >> 1], kc & 1);
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const bf16* vp = sm.vt[buf] + (db * 32 + l32) * LDS_ROW + hf * 8;
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) acc[db] = mfma32(lds_read8(vp + kc * 16), pb[kc], acc[db]);
            }
        }
        if (has_next) {
            store_tile_rows(sm.k[buf ^ 1], nk, tid);
            store_tile_transposed(sm.vt[buf ^ 1], nv, tid);
        }
        __syncthreads();
    }

    // Epilogue: O = acc / l (rounded to bf16), LSE = ln(sum) + max in natural units.
    const float l_tot = l_run + swap_halves(l_run);
    const float inv = 1.0f / l_tot;
    if (my_q < T) {
        bf16* op = out + ((long long)b * T + my_q) * C + h * HEAD_DIM;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * hf;
                *reinterpret_cast<u32x2*>(op + d) =
                    to_bf16x4_bits(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
                                   acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
            }
        if (hf == 0) lse[(long long)bh * T + my_q] = (m_run + log2f(l_tot)) * LN2;
    }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* qkv, void* out, float* lse, int B, int T, int H,
                                hipStream_t stream) {
    const int n_qt = (T + FWD_BM - 1) / FWD_BM;
    const long long blocks = (long long)B * H * n_qt;
    const float c_log2 = LOG2E / 8.0f;  // scale = 1/sqrt(64)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16*>(qkv), static_cast<bf16*>(out), lse, B, T, H,
                       n_qt, c_log2);
    return hipGetLastError();
}

}  // namespace cattn
