// Materialising ("unfused") causal attention, bf16, on MFMA (gfx950).
//
// The work flash attention avoids, done explicitly so that the two can be
// compared kernel against kernel on the same machine: the pages credit flash
// attention with taking a GPT-2 124M training step from 130 ms to 96 ms
// ("Let's reproduce GPT-2 (124M)", chapter list, 01:48:15 to 02:00:18; the
// theprofessional.online summary, glossary row "flash attention"), a whole-
// step figure for the same attention computed with and without the T x T
// matrix in memory.
//
// Per head, like a framework's plain attention with autograd:
//   forward:  S = scale Q K^T (fp32, T x T, to HBM);  P = softmax_rows(mask(S))
//             (bf16, T x T, kept for the backward) and LSE;  O = P V
//   backward: dP = dO V^T (fp32, T x T);  dS = P (dP - rowsum(P dP)) (bf16);
//             dQ = scale dS K;  dK = scale dS^T Q;  dV = P^T dO
// The products run over the whole T x T square, masked entries included, as
// a batched matrix product does; only the softmax applies the mask.
//
// The T x T matrices (S, P, dP, dS) have rows of Tp8 = round_up(T, 8)
// elements, so that no 16-byte chunk of a row reaches into the next one; the
// padding columns of P and dS hold zeros.
//
// One batched GEMM kernel serves all six products. Operands are staged in
// LDS as 64 x 64 bf16 tiles (the layout of the fused kernels) in their
// storage orientation: a "row" operand is stored with k contiguous (its LDS
// tile rows are m or n), a "tr" operand with m or n contiguous (its LDS tile
// rows are k) and is read with transposing LDS reads. Both kinds present the
// MFMA with the same k order within each 16-wide chunk, so any pairing works.
#include "attn_common.h"

namespace cattn {
namespace {

constexpr int G_BM = 128;  // output rows per workgroup
constexpr int G_BK = 64;   // k per LDS stage

enum { OP_ROW = 0, OP_TR = 1 };

// One batched bf16 operand. Element (outer, k) of a row operand, or (k,
// outer) of a tr operand, of head (b, h) sits at
// base + b * stride_b + h * stride_h + first * ld + second.
struct Operand {
    const bf16* base;
    long long stride_b, stride_h, ld;
};

struct Output {
    void* base;  // float or bf16 elements
    long long stride_b, stride_h, ld;
    const bf16* bias;  // added to every row (bias[n] for column n) when not null
};

struct GemmShape {
    int M, N, K, H;
    float alpha;
    int K_tail;  // K of the batches with h = H - 1 (a shorter last K split); K elsewhere
};

// Descriptor over a 64 x 64 tile whose first element is at `p`, with `rows`
// rows of `ld` elements and `cols` valid columns left: loads of rows past
// `rows` return zeros. The range ends with the 16-byte chunk that holds the
// last valid column of the last row (the buffer range check works on whole
// dwords), so the row stride must keep that chunk inside the row: ld and
// the tile's first column are multiples of 8 and the columns past `cols`
// up to the next multiple of 8 belong to the same row (padding or the next
// operand columns), which the other operand multiplies by zero rows or
// which only feed outputs that are not stored.
__device__ __forceinline__ i32x4 tile_rsrc(const bf16* p, long long ld, int rows, int cols) {
    long long n = 0;
    if (rows > 0 && cols > 0)
        n = ((long long)(min(rows, 64) - 1) * ld + ((min(cols, 64) + 7) & ~7)) * 2;
    return buffer_rsrc(p, (unsigned int)n);
}

// The products here relabel k inside each 16-chunk so that lane half h
// holds k = 16kc + 8h .. 8h + 7 of both operands (any labelling works when
// both operands use it): a row-oriented operand is then one 16-byte LDS read
// per lane, and the transposing reads take tile rows 8h + i/4 and 8h + 4 +
// i/4 (lane i of each 16-lane group) instead of the attention kernels' 4h and
// 8 + 4h. Both read patterns stay free of bank conflicts under swz.
__device__ __forceinline__ bf16x8 row_operand(lds_bf16* tile, int r, int kc, int hf) {
    return atile_row(tile, r, 2 * kc + hf);
}

__device__ __forceinline__ void gemm_tr_offsets(int lane, int db, int* off0, int* off1) {
    const int i = lane & 15, grp = lane >> 4, h = grp >> 1;
    const int d = db * 32 + 16 * (grp & 1) + 4 * (i & 3);
    const int r0 = 8 * h + (i >> 2), r1 = r0 + 4;
    *off0 = r0 * 64 + (((d >> 3) ^ swz(r0)) << 3) + (d & 7);
    *off1 = r1 * 64 + (((d >> 3) ^ swz(r1)) << 3) + (d & 7);
}

// C[M x N] = alpha * A[M x K] B[K x N] per head; BN = 192 (waves 2 x 2, each
// 64 x 96), 128 (waves 2 x 2, each 64 x 64) or 64 (waves 4 x 1, each
// 32 x 64). Blocks: x = output tile, y = (b, h). Two LDS stages (80 KB at
// BN = 192, so that two workgroups fill a CU's LDS).
template <int OPA, int OPB, int BN, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(Operand A, Operand B, Output Cout,
                                                        GemmShape g) {
    constexpr int NB_A = 2, NB_B = BN / 64;  // 64 x 64 tiles per stage
    constexpr int WM = BN >= 128 ? 2 : 1;    // 32-row MFMA blocks per wave
    constexpr int WN = BN == 192 ? 3 : 2;    // 32-column MFMA blocks per wave
    __shared__ bf16 sA[2][NB_A][ATILE_ELEMS];
    __shared__ bf16 sB[2][NB_B][ATILE_ELEMS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;

    const int bh = blockIdx.y, b = bh / g.H, h = bh - b * g.H;
    const int K = h == g.H - 1 ? g.K_tail : g.K;
    const int tiles_n = (g.N + BN - 1) / BN;
    const int m0 = (blockIdx.x / tiles_n) * G_BM, n0 = (blockIdx.x % tiles_n) * BN;
    const bf16* Ab = A.base + b * A.stride_b + h * A.stride_h;
    const bf16* Bb = B.base + b * B.stride_b + h * B.stride_h;
    const TileLoader la = tile_loader(A.ld, wave, lane);
    const TileLoader lb = tile_loader(B.ld, wave, lane);

    // Wave's output block: rows wm0 .. wm0 + 32 WM - 1, columns wn0 .. wn0 + 32 WN - 1.
    const int wm0 = BN >= 128 ? (wave & 1) * 64 : wave * 32;
    const int wn0 = BN >= 128 ? (wave >> 1) * 32 * WN : 0;
    int troff[2][2];
#pragma unroll
    for (int db = 0; db < 2; ++db) gemm_tr_offsets(lane, db, &troff[db][0], &troff[db][1]);

    // Tile t (0 .. NB-1) of an operand for k step k0: a row operand's tile t
    // holds rows outer0 + 64t .. +63 and k0 .. k0 + 63; a tr operand's tile t
    // holds k rows k0 .. k0 + 63 and columns outer0 + 64t .. +63.
    auto load = [&](int op, const bf16* base, long long ld, const TileLoader& L, int outer0,
                    int n_outer, int t, int k0, bf16* dst) {
        const int o = outer0 + 64 * t;
        i32x4 r;
        if (op == OP_ROW) r = tile_rsrc(base + (long long)o * ld + k0, ld, n_outer - o, K - k0);
        else r = tile_rsrc(base + (long long)k0 * ld + o, ld, K - k0, n_outer - o);
        atile_load(atile_addr(dst), r, 0, L);
    };
    auto issue = [&](int ks, int st) {
        const int k0 = ks * G_BK;
#pragma unroll
        for (int t = 0; t < NB_A; ++t) load(OPA, Ab, A.ld, la, m0, g.M, t, k0, sA[st][t]);
#pragma unroll
        for (int t = 0; t < NB_B; ++t) load(OPB, Bb, B.ld, lb, n0, g.N, t, k0, sB[st][t]);
    };
    // MFMA operand of the 32-row (outer) block `blk` of a stage, k chunk kc.
    auto operand = [&](int op, bf16* stage_tiles, int blk, int kc) -> bf16x8 {
        const int t = blk >> 1, part = blk & 1;  // 64-wide tile and its 32-half
        lds_bf16* tile = atile_view(stage_tiles + t * ATILE_ELEMS);
        if (op == OP_ROW) return row_operand(tile, part * 32 + l32, kc, hf);
        return atile_tr(tile, troff[part][0], troff[part][1], kc);
    };

    f32x16 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = zero16();

    const int n_k = (K + G_BK - 1) / G_BK;
    issue(0, 0);
    for (int ks = 0; ks < n_k; ++ks) {
        wait_vmem<0>();
        __syncthreads();  // stage ks % 2 is complete; stage (ks + 1) % 2 is free
        if (ks + 1 < n_k) issue(ks + 1, (ks + 1) & 1);
        const int st = ks & 1;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            bf16x8 bop[WN];
#pragma unroll
            for (int nb = 0; nb < WN; ++nb) bop[nb] = operand(OPB, sB[st][0], (wn0 >> 5) + nb, kc);
#pragma unroll
            for (int mb = 0; mb < WM; ++mb) {
                const bf16x8 aop = operand(OPA, sA[st][0], (wm0 >> 5) + mb, kc);
#pragma unroll
                for (int nb = 0; nb < WN; ++nb) acc[mb][nb] = mfma32(aop, bop[nb], acc[mb][nb]);
            }
        }
    }

    // C tile layout: lane holds rows 8(i/4) + 4hf + (i%4) of column l32.
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
#pragma unroll
        for (int nb = 0; nb < WN; ++nb) {
            const int n = n0 + wn0 + nb * 32 + l32;
            if (n >= g.N) continue;
            const float bias = Cout.bias ? (float)Cout.bias[n] : 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + wm0 + mb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                if (m >= g.M) continue;
                const long long off = b * Cout.stride_b + h * Cout.stride_h + (long long)m * Cout.ld + n;
                const float v = g.alpha * acc[mb][nb][i] + bias;
                if (OUT_F32) static_cast<float*>(Cout.base)[off] = v;
                else static_cast<bf16*>(Cout.base)[off] = (bf16)v;
            }
        }
}

// Row kernels: one wave per row of one head, four rows per workgroup. Lane l
// holds the columns 4l + 256c .. +3 (c = 0 .. VPT/4 - 1) in registers, read
// and written as 16-byte (fp32) or 8-byte (bf16) pieces, and the row's max
// and sums are wave reductions. VPT = 16, 32 or 64 values per lane (rows of
// up to 1024, 2048 or 4096 columns), chosen from Tp8.
constexpr int ROWS_PER_WG = 4;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// P = softmax over keys j <= i of the scaled scores of row i (exp, log: the
// accurate device functions), P = 0 for j > i and in the padding, and
// LSE = max + ln(sum).
template <int VPT>
__global__ __launch_bounds__(64 * ROWS_PER_WG) void softmax_rows_kernel(
    const float* __restrict__ S, bf16* __restrict__ P, float* __restrict__ lse, int T, int Tp8,
    long long n_rows) {
    const long long row = (long long)blockIdx.x * ROWS_PER_WG + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int lane = threadIdx.x & 63;
    const int i = (int)(row % T);
    const float* s = S + row * Tp8;
    bf16* p = P + row * Tp8;
    float x[VPT];
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < VPT / 4; ++c) {
        const int j0 = 4 * lane + 256 * c;
        f32x4 v = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (j0 < Tp8) v = *reinterpret_cast<const f32x4*>(s + j0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[4 * c + e] = j0 + e <= i ? v[e] : -INFINITY;
            m = fmaxf(m, x[4 * c + e]);
        }
    }
    m = wave_max(m);
    float sum = 0.0f;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        x[v] = x[v] == -INFINITY ? 0.0f : expf(x[v] - m);
        sum += x[v];
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int c = 0; c < VPT / 4; ++c) {
        const int j0 = 4 * lane + 256 * c;
        if (j0 < Tp8)
            *reinterpret_cast<u32x2*>(p + j0) = to_bf16x4_bits(x[4 * c] * inv, x[4 * c + 1] * inv,
                                                               x[4 * c + 2] * inv, x[4 * c + 3] * inv);
    }
    if (lane == 0) lse[row] = m + logf(sum);
}

// D = sum_j P dP and dS = P (dP - D), bf16, over the visible keys j <= i of
// row i; dS is 0 above the diagonal and in the padding. dP holds only the T
// columns its product wrote: the padding columns are never read, since 0 times
// whatever they hold (possibly not a number) must not reach D.
template <int VPT>
__global__ __launch_bounds__(64 * ROWS_PER_WG) void softmax_bwd_rows_kernel(
    const bf16* __restrict__ P, const float* __restrict__ dP, bf16* __restrict__ dS, int T,
    int Tp8, long long n_rows) {
    const long long row = (long long)blockIdx.x * ROWS_PER_WG + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int lane = threadIdx.x & 63;
    const int i = (int)(row % T);
    const bf16* p = P + row * Tp8;
    const float* g = dP + row * Tp8;
    float pv[VPT], gv[VPT];
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < VPT / 4; ++c) {
        const int j0 = 4 * lane + 256 * c;
        f32x4 gg = {0.0f, 0.0f, 0.0f, 0.0f};
        bf16x4 pp = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
        if (j0 < Tp8) {
            gg = *reinterpret_cast<const f32x4*>(g + j0);
            pp = *reinterpret_cast<const bf16x4*>(p + j0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool vis = j0 + e <= i;
            pv[4 * c + e] = vis ? (float)pp[e] : 0.0f;
            gv[4 * c + e] = vis ? gg[e] : 0.0f;
            acc = fmaf(pv[4 * c + e], gv[4 * c + e], acc);
        }
    }
    const float D = wave_sum(acc);
#pragma unroll
    for (int c = 0; c < VPT / 4; ++c) {
        const int j0 = 4 * lane + 256 * c;
        float d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            d[e] = j0 + e <= i ? pv[4 * c + e] * (gv[4 * c + e] - D) : 0.0f;
        if (j0 < Tp8)
            *reinterpret_cast<u32x2*>(dS + row * Tp8 + j0) = to_bf16x4_bits(d[0], d[1], d[2], d[3]);
    }
}

// Launch a row kernel with the smallest VPT that holds Tp8 columns.
hipError_t launch_softmax(const float* S, bf16* P, float* lse, int T, int Tp8, long long n_rows,
                          hipStream_t stream) {
    const dim3 grid((unsigned)((n_rows + ROWS_PER_WG - 1) / ROWS_PER_WG)), block(64 * ROWS_PER_WG);
    if (Tp8 <= 1024) hipLaunchKernelGGL(softmax_rows_kernel<16>, grid, block, 0, stream, S, P, lse, T, Tp8, n_rows);
    else if (Tp8 <= 2048) hipLaunchKernelGGL(softmax_rows_kernel<32>, grid, block, 0, stream, S, P, lse, T, Tp8, n_rows);
    else hipLaunchKernelGGL(softmax_rows_kernel<64>, grid, block, 0, stream, S, P, lse, T, Tp8, n_rows);
    return hipGetLastError();
}

hipError_t launch_softmax_bwd(const bf16* P, const float* dP, bf16* dS, int T, int Tp8,
                              long long n_rows, hipStream_t stream) {
    const dim3 grid((unsigned)((n_rows + ROWS_PER_WG - 1) / ROWS_PER_WG)), block(64 * ROWS_PER_WG);
    if (Tp8 <= 1024) hipLaunchKernelGGL(softmax_bwd_rows_kernel<16>, grid, block, 0, stream, P, dP, dS, T, Tp8, n_rows);
    else if (Tp8 <= 2048) hipLaunchKernelGGL(softmax_bwd_rows_kernel<32>, grid, block, 0, stream, P, dP, dS, T, Tp8, n_rows);
    else hipLaunchKernelGGL(softmax_bwd_rows_kernel<64>, grid, block, 0, stream, P, dP, dS, T, Tp8, n_rows);
    return hipGetLastError();
}

template <int OPA, int OPB, int BN, bool OUT_F32>
hipError_t gemm(Operand A, Operand B, Output C, int M, int N, int K, int BH, int H, float alpha,
                hipStream_t stream, int K_tail = -1) {
    const long long tiles = (long long)((M + G_BM - 1) / G_BM) * ((N + BN - 1) / BN);
    const GemmShape g{M, N, K, H, alpha, K_tail < 0 ? K : K_tail};
    hipLaunchKernelGGL((gemm_bf16_kernel<OPA, OPB, BN, OUT_F32>), dim3((unsigned)tiles, (unsigned)BH),
                       dim3(256), 0, stream, A, B, C, g);
    return hipGetLastError();
}

}  // namespace

// Column tile of the layer products: 192 where N allows, else 128. At
// N = 768 the 128 x 192 tiles make 512 tiles per 16384 rows, one full round
// of two workgroups per CU, where 128 x 128 tiles leave the second round half
// empty.
int gemm_tile_n(int N) { return N % 192 == 0 ? 192 : 128; }

// K splits of a split product: chunks of round_up(ceil(K / splits), 64)
// elements, the last one shorter; returns how many chunks that makes (at most
// `splits`) and their length.
int gemm_split_count(int K, int splits, int* chunk) {
    if (splits <= 1 || K <= 64) {
        *chunk = K;
        return 1;
    }
    const int c = ((K + splits - 1) / splits + 63) / 64 * 64;
    *chunk = c;
    return (K + c - 1) / c;
}

// One plain (un-batched) product C = A B (+ bias per column) for the linear
// maps around the attention, or a split product: the K range cut as
// gemm_split_count says, chunk s into the s-th consecutive M x N fp32 slab.
// A is M x K, stored k-contiguous (a_tr false, row stride lda) or
// M-contiguous (a_tr true: element (m, k) at k * lda + m); B is K x N, stored
// N-contiguous (b_tr true: element (k, n) at k * ldb + n) or k-contiguous
// (b_tr false: element (k, n) at n * ldb + k). C is M x N row-major (ldc).
// Strides and column offsets are multiples of 8 elements (16 bytes). The
// orientations the layer uses: (A row, B tr) for x W and att W_proj, (A row,
// B row) for dy W_proj^T and dqkv W_attn^T, and (A tr, B tr) with fp32
// output for the weight gradients.
hipError_t launch_gemm_bf16(bool a_tr, bool b_tr, bool out_f32, const void* A_v, long long lda,
                            const void* B_v, long long ldb, void* C_v, long long ldc,
                            const void* bias, int M, int N, int K, int splits,
                            hipStream_t stream) {
    const bf16* A_p = static_cast<const bf16*>(A_v);
    const bf16* B_p = static_cast<const bf16*>(B_v);
    int chunk = K;
    const int n_split = gemm_split_count(K, splits, &chunk);
    const int K_tail = K - (n_split - 1) * chunk;
    // chunk k of the split starts chunk * k elements along k
    const long long a_step = a_tr ? (long long)chunk * lda : chunk;
    const long long b_step = b_tr ? (long long)chunk * ldb : chunk;
    const Operand A{A_p, 0, a_step, lda}, B{B_p, 0, b_step, ldb};
    const Output C{C_v, 0, (long long)M * ldc, ldc, static_cast<const bf16*>(bias)};
    const bool wide = gemm_tile_n(N) == 192;
#define CATTN_GEMM(OA, OB, BN_, F32)                                                              \
    gemm<OA, OB, BN_, F32>(A, B, C, M, N, chunk, n_split, n_split, 1.0f, stream, K_tail)
    if (!a_tr && b_tr && !out_f32)
        return wide ? CATTN_GEMM(OP_ROW, OP_TR, 192, false) : CATTN_GEMM(OP_ROW, OP_TR, 128, false);
    if (!a_tr && !b_tr && !out_f32)
        return wide ? CATTN_GEMM(OP_ROW, OP_ROW, 192, false) : CATTN_GEMM(OP_ROW, OP_ROW, 128, false);
    if (a_tr && b_tr && out_f32)
        return wide ? CATTN_GEMM(OP_TR, OP_TR, 192, true) : CATTN_GEMM(OP_TR, OP_TR, 128, true);
#undef CATTN_GEMM
    return hipErrorInvalidValue;  // orientation not used by the library
}

int unfused_max_T() { return 4096; }  // Tp8 <= 4096 columns fit one wave's registers

long long unfused_row_stride(int T) { return ((long long)T + 7) / 8 * 8; }

// Forward. ws: S as fp32 (B*H*T*Tp8 floats).
hipError_t launch_attn_fwd_unfused_bf16(const void* qkv_v, void* out_v, float* lse, void* probs_v,
                                        void* ws, int B, int T, int H, hipStream_t stream) {
    const bf16* qkv = static_cast<const bf16*>(qkv_v);
    const long long C = (long long)H * HEAD_DIM, rs = 3 * C;
    const int Tp8 = (int)unfused_row_stride(T);
    const long long TT = (long long)T * Tp8;  // one head's T x T matrix
    const int BH = B * H;
    const float scale = 0.125f;  // 1/sqrt(64)
    float* S = static_cast<float*>(ws);
    bf16* P = static_cast<bf16*>(probs_v);
    // S = scale Q K^T: A = Q (rows q, k = d), B = K (rows key, k = d).
    const Operand q{qkv, T * rs, HEAD_DIM, rs}, k{qkv + C, T * rs, HEAD_DIM, rs};
    hipError_t e = gemm<OP_ROW, OP_ROW, 128, true>(q, k, Output{S, H * TT, TT, Tp8}, T, T,
                                                   HEAD_DIM, BH, H, scale, stream);
    if (e != hipSuccess) return e;
    if ((e = launch_softmax(S, P, lse, T, Tp8, (long long)BH * T, stream)) != hipSuccess) return e;
    // O = P V: A = P (rows q, k = key), B = V stored (key, d): tr.
    const Operand p{P, H * TT, TT, Tp8}, v{qkv + 2 * C, T * rs, HEAD_DIM, rs};
    return gemm<OP_ROW, OP_TR, 64, false>(p, v, Output{out_v, T * C, HEAD_DIM, C}, T, HEAD_DIM, T,
                                          BH, H, 1.0f, stream);
}

// Backward. ws: dP as fp32 (B*H*T*Tp8 floats), then dS as bf16.
hipError_t launch_attn_bwd_unfused_bf16(const void* dout_v, const void* qkv_v, const void* probs_v,
                                        void* dqkv_v, void* ws, int B, int T, int H,
                                        hipStream_t stream) {
    const bf16* qkv = static_cast<const bf16*>(qkv_v);
    const bf16* dout = static_cast<const bf16*>(dout_v);
    bf16* dqkv = static_cast<bf16*>(dqkv_v);
    const long long C = (long long)H * HEAD_DIM, rs = 3 * C;
    const int Tp8 = (int)unfused_row_stride(T);
    const long long TT = (long long)T * Tp8;
    const int BH = B * H;
    const float scale = 0.125f;
    float* dP = static_cast<float*>(ws);
    bf16* dS = reinterpret_cast<bf16*>(dP + (long long)BH * TT);
    const bf16* P = static_cast<const bf16*>(probs_v);
    const Operand q{qkv, T * rs, HEAD_DIM, rs}, k{qkv + C, T * rs, HEAD_DIM, rs};
    const Operand v{qkv + 2 * C, T * rs, HEAD_DIM, rs}, g{dout, T * C, HEAD_DIM, C};
    const Operand p{P, H * TT, TT, Tp8}, ds{dS, H * TT, TT, Tp8};
    // dP = dO V^T: A = dO (rows q, k = d), B = V (rows key, k = d).
    hipError_t e = gemm<OP_ROW, OP_ROW, 128, true>(g, v, Output{dP, H * TT, TT, Tp8}, T, T,
                                                   HEAD_DIM, BH, H, 1.0f, stream);
    if (e != hipSuccess) return e;
    if ((e = launch_softmax_bwd(P, dP, dS, T, Tp8, (long long)BH * T, stream)) != hipSuccess)
        return e;
    // dQ = scale dS K: A = dS (rows q, k = key), B = K stored (key, d): tr.
    if ((e = gemm<OP_ROW, OP_TR, 64, false>(ds, k, Output{dqkv, T * rs, HEAD_DIM, rs}, T, HEAD_DIM,
                                            T, BH, H, scale, stream)) != hipSuccess)
        return e;
    // dK = scale dS^T Q: A = dS^T (dS stored (q, key): tr), B = Q stored (q, d): tr.
    if ((e = gemm<OP_TR, OP_TR, 64, false>(ds, q, Output{dqkv + C, T * rs, HEAD_DIM, rs}, T,
                                           HEAD_DIM, T, BH, H, scale, stream)) != hipSuccess)
        return e;
    // dV = P^T dO: A = P^T (tr), B = dO stored (q, d): tr.
    return gemm<OP_TR, OP_TR, 64, false>(p, g, Output{dqkv + 2 * C, T * rs, HEAD_DIM, rs}, T,
                                         HEAD_DIM, T, BH, H, 1.0f, stream);
}

}  // namespace cattn
