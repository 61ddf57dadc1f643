// Causal attention forward, bf16 storage, fp32 accumulation, MFMA (gfx950).
//
// Computes O = softmax(scale * Q K^T + causal mask) V and LSE per row without
// ever holding the T x T score matrix in memory: the FlashAttention method of
// "Let's reproduce GPT-2 (124M)" (chapter list, 02:00:18; glossary table of
// the theprofessional.online summary, row "flash attention"), written for
// CDNA4 from the definition rather than from any published kernel.
//
// One workgroup = 4 waves = 128 queries of one (batch, head); wave w owns
// queries q0 + 32w .. +31. Key/value tiles of 64 rows stream through a
// three-stage ring of LDS buffers filled by direct buffer->LDS loads. Per
// tile, a wave computes S^T = K Q^T on MFMA (lane l%32 owns query l%32, so
// row statistics live in one lane pair), masks only its last tile (the one
// holding its diagonal), and accumulates O^T += V^T P^T on MFMA with P^T fed
// straight from registers and V^T read from the row-major V tile by
// transposing LDS reads. Tiles above a wave's diagonal are skipped.
//
// The tile loop is software-pipelined across tiles: while the exponentials
// of tile j run on the VALU, the MFMAs of S for tile j+1 are in flight, and
// while P V of tile j runs on MFMA, the VALU sums tile j's row and takes the
// row max of tile j+1. So each wave keeps the matrix cores and the vector
// ALU busy at once, instead of alternating between them.
//
// Softmax in base 2 with a lazily updated running max: the accumulator is
// rescaled only when some row's tile max exceeds its running max by more
// than 2^8; otherwise the stale max is kept and P may reach 2^8, which fp32
// and bf16 hold exactly as well as values below 1. The result is the same
// function: O = acc / l and LSE = ln 2 * (m + log2 l) for whichever m was used.
#include "attn_common.h"

#ifndef CATTN_FWD_WAVES_PER_SIMD
#define CATTN_FWD_WAVES_PER_SIMD 1
#endif

namespace cattn {
namespace {

constexpr int FWD_BM = 128;  // queries per workgroup (32 per wave)
constexpr int FWD_BN = 64;   // keys per tile
constexpr int NSTAGE = 3;    // tile j (V), tile j+1 (K) in use, tile j+2 in flight
constexpr float RESCALE_LOG2 = 8.0f;

struct FwdSmem {
    bf16 k[NSTAGE][ATILE_ELEMS];  // K tiles, row-major [key][d] (swizzled)
    bf16 v[NSTAGE][ATILE_ELEMS];  // V tiles, row-major [key][d] (swizzled)
};

typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

// S^T = K Q^T for one 64-key tile: two 32-key blocks of 4 MFMAs each.
__device__ __forceinline__ void scores(lds_bf16* kt, const int (&koff)[4],
                                       const bf16x8 (&qreg)[4], f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        s[kb] = zero16();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            s[kb] = mfma32(*reinterpret_cast<lds_bf16x8*>(kt + kb * 32 * 64 + koff[kk]), qreg[kk],
                           s[kb]);
    }
}

// Causal mask of a wave's last tile: key k0 + kb*32 + 8(i/4) + 4hf + (i%4)
// against query qw + l32; `lim` = qw - k0 + l32 - 4hf.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int lim) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
}

// Row max of a tile (both lane halves), times c = scale * log2 e.
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2], float c_log2) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    return fmaxf(mx, swap_halves(mx)) * c_log2;
}

// Take the new tile max into the running max: a row rescales (acc, l) only
// when its tile max exceeds the running max by more than 2^8. Each row
// decides for itself (rows that keep their max scale by exactly 1), so a
// row's arithmetic never depends on the other rows of the wave and later
// tokens cannot change earlier rows.
__device__ __forceinline__ void update_max(float mt, float& m_run, float& l_run,
                                           f32x16 (&acc)[2]) {
    const bool grow = mt > m_run + RESCALE_LOG2;
    if (__any(grow)) {
        asm volatile("");  // keeps the branch: rescales are rare after the first tiles
        const float m_new = grow ? mt : m_run;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
}

enum NextTile { NEXT_NONE, NEXT_PLAIN, NEXT_MASKED };

// One pipelined tile step: P = exp2(c s - m) of tile j (in place in `s`)
// with the scores of tile j+1 (into `s_next`) on MFMA, then O^T += V^T P^T
// of tile j with the row sum of tile j and the mask and row max of tile j+1
// on the VALU. The caller swaps the roles of the two score buffers.
template <int NEXT>
__device__ __forceinline__ void tile_step(f32x16 (&s)[2], f32x16 (&s_next)[2], lds_bf16* kt_next,
                                          lds_bf16* vt, const int (&koff)[4],
                                          const int (&voff)[2][2], const bf16x8 (&qreg)[4],
                                          f32x16 (&acc)[2], float& m_run, float& l_run,
                                          float c_log2, int lim_next) {
    if (NEXT != NEXT_NONE) scores(kt_next, koff, qreg, s_next);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(fmaf(s[kb][i], c_log2, -m_run));
    bf16x8 pb[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) pb[kc] = c_rows_to_operand(s[kc >> 1], kc & 1);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
            acc[db] = mfma32(atile_tr(vt, voff[db][0], voff[db][1], kc), pb[kc], acc[db]);
    float rsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) rsum += s[kb][i];
    l_run += rsum;
    if (NEXT != NEXT_NONE) {
        if (NEXT == NEXT_MASKED) mask_tile(s_next, lim_next);
        update_max(tile_max(s_next, c_log2), m_run, l_run, acc);
    }
}

__global__ __launch_bounds__(256, CATTN_FWD_WAVES_PER_SIMD) void attn_fwd_bf16_kernel(
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
    const int qw = q0 + wave * 32;  // first query of this wave

    const int kend = min(q0 + FWD_BM, T);
    const int n_kt = (kend + FWD_BN - 1) / FWD_BN;
    // This wave's last tile: the one holding key qw + 31 (its diagonal), or
    // the workgroup's last tile when the sequence ends first. Only this tile
    // can hold keys above one of the wave's queries.
    const int j_last = min((qw + 31) / FWD_BN, n_kt - 1);

    // Per-lane LDS offsets: K rows kb*32 + l32 at chunks 2kk + hf; V^T reads.
    int koff[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) koff[kk] = l32 * 64 + (((2 * kk + hf) ^ swz(l32)) << 3);
    int voff[2][2];
#pragma unroll
    for (int db = 0; db < 2; ++db) atile_tr_offsets(lane, db, &voff[db][0], &voff[db][1]);

    // Wave-uniform LDS byte addresses of stage 0 (stage st sits st * 8 KB on).
    const unsigned int k_lds = atile_addr(sm.k[0]), v_lds = atile_addr(sm.v[0]);
    constexpr unsigned int STAGE_BYTES = ATILE_ELEMS * 2;
    // K and V rows of tile t into stage t % 3: one descriptor, since V sits C
    // elements after K in every packed row. 32-bit LDS addresses and a
    // descriptor derived from t keep the per-tile scalar work small.
    const long long tile_bytes = (long long)FWD_BN * rs * 2;
    const unsigned long long k_at = (unsigned long long)(uintptr_t)kbase;
    const long long k_total = (long long)T * rs * 2;
    auto issue = [&](int t) {
        const unsigned int st = (unsigned int)t % NSTAGE;
        const unsigned long long at = k_at + (unsigned long long)t * tile_bytes;
        const long long left = k_total - (long long)t * tile_bytes;
        i32x4 kv;
        kv.x = (int)(unsigned int)at;
        kv.y = (int)((unsigned int)(at >> 32) & 0xffffu);
        kv.z = (int)(left > 0xffffffffLL ? 0xffffffffu : (unsigned int)left);
        kv.w = 0x00020000;
        atile_load(k_lds + st * STAGE_BYTES, kv, 0, ld_rs);
        atile_load(v_lds + st * STAGE_BYTES, kv, 2u * C, ld_rs);
    };
    issue(0);
    if (n_kt > 1) issue(1);

    // Q^T operands (B of S^T = K Q^T): d = 16kk + 8hf .. +7 of this lane's query.
    bf16x8 qreg[4];
    {
        const int q = qw + l32;
        const bf16* p = qbase + (long long)q * rs + hf * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qreg[kk] = as_bf16x8(load16(p + kk * 16, q < T));
    }
    // Tiles 0 and 1 and Q land before the loop (no waits on Q inside it).
    wait_vmem<0>();
    __syncthreads();

    float m_run = -INFINITY;  // running max of c*s
    float l_run = 0.0f;       // this lane half's share of the row sum
    f32x16 acc[2] = {zero16(), zero16()};  // O^T per d block
    f32x16 s[2], s_next[2];
    {
        scores(atile_view_at(k_lds), koff, qreg, s);
        if (j_last == 0) mask_tile(s, qw + l32 - 4 * hf);
        update_max(tile_max(s, c_log2), m_run, l_run, acc);
    }

    auto step = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        const unsigned int sj = (unsigned int)j % NSTAGE, sn = (unsigned int)(j + 1) % NSTAGE;
        // Tile j+1 (issued one step ago) has landed everywhere, and every wave
        // has left step j-1, so its stage can take tile j+2.
        wait_vmem<0>();
        __syncthreads();
        if (j + 2 < n_kt) issue(j + 2);
        if (j > j_last) return;  // tiles above this wave's diagonal
        lds_bf16* vt = atile_view_at(v_lds + sj * STAGE_BYTES);
        lds_bf16* kt_next = atile_view_at(k_lds + sn * STAGE_BYTES);
        const int lim_next = qw - (j + 1) * FWD_BN + l32 - 4 * hf;
        if (j + 1 < j_last)
            tile_step<NEXT_PLAIN>(cur, nxt, kt_next, vt, koff, voff, qreg, acc, m_run, l_run,
                                  c_log2, lim_next);
        else if (j + 1 == j_last)
            tile_step<NEXT_MASKED>(cur, nxt, kt_next, vt, koff, voff, qreg, acc, m_run, l_run,
                                   c_log2, lim_next);
        else
            tile_step<NEXT_NONE>(cur, nxt, kt_next, vt, koff, voff, qreg, acc, m_run, l_run,
                                 c_log2, lim_next);
    };
    // Two steps per trip, so the two score buffers trade roles without copies.
    for (int j = 0; j < n_kt; j += 2) {
        step(j, s, s_next);
        if (j + 1 < n_kt) step(j + 1, s_next, s);
    }

    // Epilogue: O = acc / l (rounded to bf16), LSE = ln 2 * (m + log2 l).
    const int q = qw + l32;
    const float l_tot = l_run + swap_halves(l_run);
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

// The kernel the library launches: the same computation with the wave's
// whole program scheduled by hand (attn_fwd_asm.inc, written by
// gen_attn_fwd_asm.py): one inline-asm block per wave, from the Q load to
// the O and LSE stores. C++ only maps the workgroup to (query tile, head),
// exactly as above, and hands the program wave-uniform scalars. The program
// issues one MFMA between every few VALU instructions: the scores of tile
// j+1 between the exponentials of tile j, P V of tile j beside the row sums
// of j. It tests the lazy rescale differently from the C++ above: not the
// next tile's row max against m, but each lane's sum of P over its 32 keys of
// the tile against 2^8, after the exponentials. A row whose half-row sum
// passed it (rare after the first tiles) takes an out-of-line block that
// recomputes the tile's scores, moves m to the running max, rescales and
// redoes the exponentials; the other rows recompute the same P and scale by
// exactly 1. Every P used is again at most 2^8, and the common path needs no
// per-tile row max. Compiled from the C++ above (build with
// -DCATTN_FWD_COMPILED), the schedule waits on each operand read just before
// its MFMA and runs about 10% slower.
#include "attn_fwd_asm.inc"

// One (query tile, head) item: the wave's program from the Q load to the O
// and LSE stores.
__device__ __forceinline__ void fwd_asm_item(const bf16* __restrict__ qkv, bf16* __restrict__ out,
                                             float* __restrict__ lse, int T, int H, int b, int h,
                                             int qt, int wave, float c_log2, unsigned int k_lds,
                                             unsigned int v_lds) {
    const int C = H * HEAD_DIM;
    const long long rs = 3LL * C;
    const int q0 = qt * FWD_BM;
    const int qw = q0 + wave * 32;
    const int kend = min(q0 + FWD_BM, T);
    const int n_kt = (kend + FWD_BN - 1) / FWD_BN;
    const int j_last = min((qw + 31) / FWD_BN, n_kt - 1);
    const int nq = T - qw;  // queries of this wave inside the sequence (may be <= 0)
    const int bh = b * H + h;

    const unsigned long long k_at =
        (unsigned long long)(uintptr_t)(qkv + (long long)b * T * rs + C + h * HEAD_DIM);
    const unsigned long long k_left = (unsigned long long)T * rs * 2;
    const unsigned long long q_row =
        (unsigned long long)(uintptr_t)(qkv + ((long long)b * T + qw) * rs + h * HEAD_DIM);
    const unsigned long long o_row =
        (unsigned long long)(uintptr_t)(out + ((long long)b * T + qw) * C + h * HEAD_DIM);
    const unsigned long long l_row = (unsigned long long)(uintptr_t)(lse + (long long)bh * T + qw);

    asm volatile(CATTN_FWD_ASM_BODY
                 :
                 : [klds] "s"(k_lds), [vlds] "s"(v_lds),
                   [kldw] "s"(k_lds + 2048u * wave), [vldw] "s"(v_lds + 2048u * wave),
                   [wave16] "s"(16 * wave), [rs2] "s"((unsigned int)(rs * 2)),
                   [c2] "s"((unsigned int)(C * 2)), [voffs] "s"((unsigned int)(C * 2)),
                   [tbytes] "s"((unsigned int)(FWD_BN * rs * 2)),
                   [kat_lo] "s"((unsigned int)k_at), [kat_hi] "s"((unsigned int)(k_at >> 32)),
                   [kleft_lo] "s"((unsigned int)k_left),
                   [kleft_hi] "s"((unsigned int)(k_left >> 32)),
                   [nkt] "s"(n_kt), [jlast] "s"(j_last), [nq] "s"(nq), [nlse] "s"(min(nq, 32)),
                   [limb] "s"(qw - j_last * FWD_BN),
                   [cbits] "s"(__builtin_bit_cast(unsigned int, c_log2)),
                   [qbase] "s"(q_row), [obase] "s"(o_row), [lbase] "s"(l_row)
                 : CATTN_FWD_ASM_CLOBBERS, "vcc", "m0", "scc", "exec", "memory");
}

// Workgroup -> (query tile, head), heaviest (last) query tiles first; when
// the head count allows, the heads are split into 8 contiguous groups, one
// per XCD, so that K/V of a head stay in one L2.
__global__ __launch_bounds__(256, 1) void attn_fwd_bf16_asm_kernel(
    const bf16* __restrict__ qkv, bf16* __restrict__ out, float* __restrict__ lse,
    int B, int T, int H, int n_qt, float c_log2) {
    __shared__ FwdSmem sm;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
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
    fwd_asm_item(qkv, out, lse, T, H, b, h, qt, wave, c_log2, atile_addr(sm.k[0]),
                 atile_addr(sm.v[0]));
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* qkv, void* out, float* lse, int B, int T, int H,
                                hipStream_t stream) {
    const int n_qt = (T + FWD_BM - 1) / FWD_BM;
    const long long blocks = (long long)B * H * n_qt;
    const float c_log2 = LOG2E / 8.0f;  // scale = 1/sqrt(64)
#ifdef CATTN_FWD_COMPILED
    hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
#else
    hipLaunchKernelGGL(attn_fwd_bf16_asm_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
#endif
                       static_cast<const bf16*>(qkv), static_cast<bf16*>(out), lse, B, T, H,
                       n_qt, c_log2);
    return hipGetLastError();
}

}  // namespace cattn
