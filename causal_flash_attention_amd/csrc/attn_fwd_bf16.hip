// Causal attention forward, bf16 storage, fp32 accumulation, MFMA (gfx950).
//
// Computes O = softmax(scale * Q K^T + causal mask) V and LSE per row without
// ever holding the T x T score matrix in memory: the FlashAttention method of
// "Let's reproduce GPT-2 (124M)" (chapter list, 02:00:18; glossary table of
// the theprofessional.online summary, row "flash attention"), written for
// CDNA4 from the definition rather than from any published kernel.
//
// One workgroup = 4 waves = 4 * 32 * QB queries of one (batch, head); wave w
// owns QB blocks of 32 queries. Key/value tiles of 64 rows stream through a
// three-stage ring of LDS buffers filled by direct global->LDS loads, so two
// tiles are in flight while a third is consumed. Per tile, a wave computes
// S^T = K Q^T on MFMA (lane l%32 owns query l%32, so row statistics live in
// one lane pair), masks only the tile on its diagonal, and accumulates
// O^T += V^T P^T on MFMA with P^T fed straight from registers and V^T read
// from the row-major V tile by transposing LDS reads. Each LDS operand read
// feeds all QB query blocks. Tiles above a wave's diagonal are skipped.
//
// Softmax in base 2 with a lazily updated running max: the accumulator is
// rescaled only when some row's tile max exceeds its running max by more
// than 2^8; otherwise the stale max is kept and P may reach 2^8, which fp32
// and bf16 hold exactly as well as values below 1. The result is the same
// function: O = acc / l and LSE = ln 2 * (m + log2 l) for whichever m was used.
#include "attn_common.h"

#ifndef CATTN_FWD_QB
#define CATTN_FWD_QB 1
#endif

namespace cattn {
namespace {

constexpr int FWD_QB = CATTN_FWD_QB;  // 32-query blocks per wave
constexpr int FWD_BM = 128 * FWD_QB;  // queries per workgroup
constexpr int FWD_BN = 64;            // keys per tile
constexpr int NSTAGE = 3;
constexpr int LOADS_PER_TILE = 4;     // per wave: 2 for K, 2 for V
constexpr float RESCALE_LOG2 = 8.0f;

struct FwdSmem {
    bf16 k[NSTAGE][ATILE_ELEMS];  // K tiles, row-major [key][d] (swizzled)
    bf16 v[NSTAGE][ATILE_ELEMS];  // V tiles, row-major [key][d] (swizzled)
};

__global__ __launch_bounds__(256) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ qkv, bf16* __restrict__ out, float* __restrict__ lse,
    int B, int T, int H, int n_qt, float c_log2) {
    __shared__ FwdSmem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
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
    const TileLoader ld_rs = tile_loader(rs, wave, lane);
    const bf16* qbase = qkv + (long long)b * T * rs + h * HEAD_DIM;
    const bf16* kbase = qbase + C;

    const int q0 = qt * FWD_BM;
    const int qw = q0 + wave * 32 * FWD_QB;  // first query of this wave

    const int kend = min(q0 + FWD_BM, T);
    const int n_kt = (kend + FWD_BN - 1) / FWD_BN;

    // Per-lane LDS offsets: K rows kb*32 + l32 at chunks 2kk + hf; V^T reads.
    int koff[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) koff[kk] = l32 * 64 + (((2 * kk + hf) ^ swz(l32)) << 3);
    int voff[2][2];
#pragma unroll
    for (int db = 0; db < 2; ++db) atile_tr_offsets(lane, db, &voff[db][0], &voff[db][1]);

    float m_run[FWD_QB], l_run[FWD_QB];
    f32x16 acc[FWD_QB][2];  // O^T per (query block, d block)
#pragma unroll
    for (int qb = 0; qb < FWD_QB; ++qb) {
        m_run[qb] = -INFINITY;  // running max of c*s
        l_run[qb] = 0.0f;       // this lane half's share of the row sum
        acc[qb][0] = acc[qb][1] = zero16();
    }

    // K and V rows [k0, k0 + 64) into stage st: one descriptor, since V sits
    // C elements after K in every packed row.
    auto issue = [&](int k0, int st) {
        const i32x4 kv = rows_rsrc(kbase, rs, k0, T);
        atile_load(atile_addr(sm.k[st]), kv, 0, ld_rs);
        atile_load(atile_addr(sm.v[st]), kv, 2u * C, ld_rs);
    };
#pragma unroll
    for (int j = 0; j < NSTAGE - 1; ++j)
        if (j < n_kt) issue(j * FWD_BN, j);

    // Q^T operands (B of S^T = K Q^T): d = 16kk + 8hf .. +7 of each block's query.
    bf16x8 qreg[FWD_QB][4];
#pragma unroll
    for (int qb = 0; qb < FWD_QB; ++qb) {
        const int q = qw + 32 * qb + l32;
        const bf16* p = qbase + (long long)q * rs + hf * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qreg[qb][kk] = as_bf16x8(load16(p + kk * 16, q < T));
    }
    // Everything issued so far (the first tiles and Q) lands before the loop,
    // so the compiler needs no waits on Q inside it.
    wait_vmem<0>();

    for (int j = 0; j < n_kt; ++j) {
        // Tile j has landed once at most the next tile's loads are pending.
        if (j + 1 < n_kt) wait_vmem<LOADS_PER_TILE>();
        else wait_vmem<0>();
        __syncthreads();
        if (j + NSTAGE - 1 < n_kt) issue((j + NSTAGE - 1) * FWD_BN, (j + NSTAGE - 1) % NSTAGE);
        const int k0 = j * FWD_BN;
        if (k0 > qw + 32 * FWD_QB - 1) continue;  // whole tile above this wave's diagonal
        const int st = j % NSTAGE;
        lds_bf16* kt = atile_view(sm.k[st]);
        lds_bf16* vt = atile_view(sm.v[st]);

        // S^T = K Q^T for every query block; each K operand read feeds QB MFMAs.
        f32x16 s[FWD_QB][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int qb = 0; qb < FWD_QB; ++qb) s[qb][kb] = zero16();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
                const bf16x8 a = *reinterpret_cast<lds_bf16x8*>(kt + kb * 32 * 64 + koff[kk]);
#pragma unroll
                for (int qb = 0; qb < FWD_QB; ++qb) s[qb][kb] = mfma32(a, qreg[qb][kk], s[qb][kb]);
            }
        }
        // Causal mask on the tile that holds a block's diagonal: key > query -> -inf.
#pragma unroll
        for (int qb = 0; qb < FWD_QB; ++qb) {
            const int qblk = qw + 32 * qb;
            if (k0 + FWD_BN - 1 > qblk) {
                const int lim = qblk - k0 + l32 - 4 * hf;  // key - k0 must be <= this
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) s[qb][kb][i] = -INFINITY;
            }
        }
        float mt[FWD_QB];
        bool grow[FWD_QB], any_grow = false;
#pragma unroll
        for (int qb = 0; qb < FWD_QB; ++qb) {
            float mx = s[qb][0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb][kb][i]);
            mx = fmaxf(mx, swap_halves(mx));
            mt[qb] = mx * c_log2;
            grow[qb] = mt[qb] > m_run[qb] + RESCALE_LOG2;
            any_grow |= grow[qb];
        }
        // Each row decides for itself (rows that do not grow keep their max
        // and scale by exactly 1), so a row's arithmetic never depends on the
        // other rows of the wave: later tokens cannot change earlier rows.
        if (__any(any_grow)) {
#pragma unroll
            for (int qb = 0; qb < FWD_QB; ++qb) {
                const float m_new = grow[qb] ? mt[qb] : m_run[qb];
                const float alpha = grow[qb] ? fast_exp2(m_run[qb] - m_new) : 1.0f;
                l_run[qb] *= alpha;
                m_run[qb] = m_new;
#pragma unroll
                for (int db = 0; db < 2; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[qb][db][i] *= alpha;
            }
        }
        bf16x8 pb[FWD_QB][4];
#pragma unroll
        for (int qb = 0; qb < FWD_QB; ++qb) {
            float rsum = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(fmaf(s[qb][kb][i], c_log2, -m_run[qb]));
                    s[qb][kb][i] = p;
                    rsum += p;
                }
            l_run[qb] += rsum;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) pb[qb][kc] = c_rows_to_operand(s[qb][kc >> 1], kc & 1);
        }
        // O^T += V^T P^T over four 16-key chunks; each V^T operand feeds QB MFMAs.
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const bf16x8 a = atile_tr(vt, voff[db][0], voff[db][1], kc);
#pragma unroll
                for (int qb = 0; qb < FWD_QB; ++qb) acc[qb][db] = mfma32(a, pb[qb][kc], acc[qb][db]);
            }
    }

    // Epilogue: O = acc / l (rounded to bf16), LSE = ln 2 * (m + log2 l).
#pragma unroll
    for (int qb = 0; qb < FWD_QB; ++qb) {
        const int q = qw + 32 * qb + l32;
        const float l_tot = l_run[qb] + swap_halves(l_run[qb]);
        const float inv = 1.0f / l_tot;
        if (q < T) {
            bf16* op = out + ((long long)b * T + q) * C + h * HEAD_DIM;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = db * 32 + 8 * g + 4 * hf;
                    const f32x16& a = acc[qb][db];
                    *reinterpret_cast<u32x2*>(op + d) =
                        to_bf16x4_bits(a[4 * g] * inv, a[4 * g + 1] * inv, a[4 * g + 2] * inv,
                                       a[4 * g + 3] * inv);
                }
            if (hf == 0) lse[(long long)bh * T + q] = (m_run[qb] + log2f(l_tot)) * LN2;
        }
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
