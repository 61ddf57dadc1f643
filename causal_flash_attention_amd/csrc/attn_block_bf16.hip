// The attention layer around the fused attention, bf16 storage, fp32
// accumulation (gfx950): c_attn, causal attention, c_proj, forward and
// backward ("Let's reproduce GPT-2 (124M)", chapter list, 00:13:47 for the
// layer; 01:48:15 kernel fusion and 02:00:18 flash attention for making it
// fast).
//
//   forward:  qkv = x W_attn + b_attn;  att, lse = attention(qkv);
//             y = att W_proj + b_proj
//   backward: datt = dy W_proj^T;  dW_proj = att^T dy;  db_proj = colsum(dy);
//             dqkv = attention backward(datt);  dx = dqkv W_attn^T;
//             dW_attn = x^T dqkv;  db_attn = colsum(dqkv)
//
// The neighbours meet the attention in its own layouts, so nothing is
// reshaped, transposed or copied between them: the c_attn product's epilogue
// adds the bias and writes the packed [Q | K | V] rows the attention kernels
// read, and the c_proj product reads the attention's (B, T, C) output as its
// A operand in place (and datt, its gradient, in the layout the backward
// reads as dO). Weights are stored (in, out).
//
// The weight gradients are long contractions (K = B * T) with small outputs,
// so they run split over K (as many splits as fill one round of workgroups)
// into fp32 slabs that a second kernel adds in a fixed order; the bias
// gradients are column sums done the same way. No atomics: the backward is
// deterministic. The slab sum of each weight gradient shares a launch with
// the column-sum partials of its bias, and the two bias sums end in one
// launch.
#include "attn_common.h"

namespace cattn {

hipError_t launch_gemm_bf16(bool a_tr, bool b_tr, bool out_f32, const void* A, long long lda,
                            const void* B, long long ldb, void* C, long long ldc, const void* bias,
                            int M, int N, int K, int splits, hipStream_t stream);
int gemm_tile_n(int N);
int gemm_split_count(int K, int splits, int* chunk);
hipError_t launch_attn_fwd_bf16(const void*, void*, float*, int, int, int, hipStream_t);
hipError_t launch_attn_bwd_dq_pre_bf16(const void*, const void*, const void*, const float*, float*,
                                       void*, int, int, int, hipStream_t);
hipError_t launch_attn_bwd_dkdv_bf16(const void*, const void*, const float*, void*, int, int, int,
                                     hipStream_t);

namespace {

constexpr int COLSUM_ROWS = 256;  // rows per partial column sum
constexpr int COLSUM_COLS = 512;  // columns per workgroup (64 threads x 8)

// parts[s * N + n] = sum of X[r, n] over the COLSUM_ROWS rows r of chunk s,
// for the column block `cb` and chunk `s` of one workgroup: thread t owns
// columns 8 (t % 64) .. +7 of the block (16-byte loads) and rows
// 64 (t / 64) .. +63 of the chunk, summed in row order; the four row groups
// are then added in group order through LDS. N must be a multiple of 8 and
// X's rows 16-byte aligned.
__device__ __forceinline__ void colsum_partial(const bf16* __restrict__ X, long long ld, int R,
                                               int N, float* __restrict__ parts, int cb, int s) {
    __shared__ float red[4][64][9];
    const int t = threadIdx.x, col8 = t & 63, grp = t >> 6;
    const int n0 = cb * COLSUM_COLS + 8 * col8;
    const int r0 = s * COLSUM_ROWS + 64 * grp;
    const int r1 = min(R, r0 + 64);
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (n0 < N) {
        const bf16* p = X + (long long)r0 * ld + n0;
#pragma unroll 8
        for (int r = r0; r < r1; ++r, p += ld) {
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[grp][col8][e] = acc[e];
    __syncthreads();
    if (grp == 0 && n0 < N) {
        float* out = parts + (long long)s * N + n0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            out[e] = ((red[0][col8][e] + red[1][col8][e]) + red[2][col8][e]) + red[3][col8][e];
    }
}

// out[n] = sum over chunks of parts[s * N + n] for the 64 columns of block
// `cb`: thread (column, group) sums the chunks s = group, group + 4, ... in
// order, then the four groups are added in group order.
__device__ __forceinline__ void colsum_final(const float* __restrict__ parts, int S, int N,
                                             float* __restrict__ out, int cb) {
    __shared__ float red[4][64];
    const int t = threadIdx.x, c = t & 63, grp = t >> 6;
    const int n = cb * 64 + c;
    float acc = 0.0f;
    if (n < N)
        for (int s = grp; s < S; s += 4) acc += parts[(long long)s * N + n];
    red[grp][c] = acc;
    __syncthreads();
    if (grp == 0 && n < N) out[n] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// One launch for two independent reductions that follow a weight-gradient
// product: workgroups [0, nb_sum) add its K-split slabs (out[i] = sum over
// s of slabs[s * n + i], in order, 256 elements per workgroup), the others
// compute the column-sum partials of X (column block, then chunk).
__global__ __launch_bounds__(256) void slabs_colsum_kernel(const float* __restrict__ slabs, int S,
                                                           long long n, float* __restrict__ sum,
                                                           int nb_sum, const bf16* __restrict__ X,
                                                           long long ld, int R, int N,
                                                           float* __restrict__ cparts, int n_cb) {
    const int blk = blockIdx.x;
    if (blk < nb_sum) {
        const long long i = (long long)blk * 256 + threadIdx.x;
        if (i >= n) return;
        float acc = 0.0f;
        for (int s = 0; s < S; ++s) acc += slabs[(long long)s * n + i];
        sum[i] = acc;
        return;
    }
    const int c = blk - nb_sum;
    colsum_partial(X, ld, R, N, cparts, c % n_cb, c / n_cb);
}

// Both bias gradients from their column-sum partials: workgroups [0, nb1)
// the first, the rest the second.
__global__ __launch_bounds__(256) void colsum_final2_kernel(const float* __restrict__ p1, int N1,
                                                            float* __restrict__ o1, int nb1,
                                                            const float* __restrict__ p2, int N2,
                                                            float* __restrict__ o2, int S) {
    if ((int)blockIdx.x < nb1) colsum_final(p1, S, N1, o1, blockIdx.x);
    else colsum_final(p2, S, N2, o2, blockIdx.x - nb1);
}

int colsum_chunks(int R) { return (R + COLSUM_ROWS - 1) / COLSUM_ROWS; }

// The slab sum of a split product (when it has more than one slab) and the
// column-sum partials of X, in one launch.
hipError_t slabs_and_colsum(const float* slabs, int S, long long n, float* sum, const bf16* X,
                            long long ld, int R, int N, float* cparts, hipStream_t stream) {
    const int nb_sum = S > 1 ? (int)((n + 255) / 256) : 0;
    const int n_cb = (N + COLSUM_COLS - 1) / COLSUM_COLS;
    const long long blocks = nb_sum + (long long)n_cb * colsum_chunks(R);
    hipLaunchKernelGGL(slabs_colsum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, slabs, S,
                       n, sum, nb_sum, X, ld, R, N, cparts, n_cb);
    return hipGetLastError();
}

}  // namespace

// K splits asked of a weight-gradient product over R = B * T rows: as many
// as make one full round of workgroups (two per CU on 256 CUs) for the
// product's tiles, at most 64 and no more than one per four 64-row steps.
// The fp32 slabs then number slabs_of(R, splits).
constexpr int ROUND_WGS = 512;

int block_splits(long long R, int M, int N) {
    const long long tiles = (long long)((M + 127) / 128) * ((N + gemm_tile_n(N) - 1) / gemm_tile_n(N));
    long long s = ROUND_WGS / tiles;
    if (s > 64) s = 64;
    if (s > R / 256) s = R / 256;
    return s < 1 ? 1 : (int)s;
}

int slabs_of(long long R, int splits) {
    int chunk = 0;
    return gemm_split_count((int)R, splits, &chunk);
}

// Workspace (floats): the attention backward's delta, the K-split slabs of
// the larger weight gradient, then the column-sum partials of dy (chunks x C)
// and of dqkv (chunks x 3C).
struct BlockWs {
    long long delta, slabs, cp_proj, cp_attn, total;
};

BlockWs block_ws(int B, int T, int H) {
    const long long C = (long long)H * HEAD_DIM, R = (long long)B * T;
    const long long tp = ((long long)T + 63) / 64 * 64;
    const long long s_attn = slabs_of(R, block_splits(R, (int)C, (int)(3 * C)));
    const long long s_proj = slabs_of(R, block_splits(R, (int)C, (int)C));
    long long slabs = s_attn * C * 3 * C;
    if (s_proj * C * C > slabs) slabs = s_proj * C * C;
    const long long chunks = colsum_chunks((int)R);
    BlockWs w;
    w.delta = 0;
    w.slabs = 10LL * B * H * tp;
    w.cp_proj = w.slabs + slabs;
    w.cp_attn = w.cp_proj + chunks * C;
    w.total = w.cp_attn + chunks * 3 * C;
    return w;
}

long long block_workspace_floats(int B, int T, int H) { return block_ws(B, T, H).total; }

hipError_t launch_attn_block_fwd_bf16(const void* x, const void* w_attn, const void* b_attn,
                                      const void* w_proj, const void* b_proj, void* qkv, void* att,
                                      float* lse, void* y, int B, int T, int H,
                                      hipStream_t stream) {
    const long long C = (long long)H * HEAD_DIM;
    const int R = B * T;
    hipError_t e = launch_gemm_bf16(false, true, false, x, C, w_attn, 3 * C, qkv, 3 * C, b_attn, R,
                                    (int)(3 * C), (int)C, 1, stream);
    if (e != hipSuccess) return e;
    if ((e = launch_attn_fwd_bf16(qkv, att, lse, B, T, H, stream)) != hipSuccess) return e;
    return launch_gemm_bf16(false, true, false, att, C, w_proj, C, y, C, b_proj, R, (int)C,
                            (int)C, 1, stream);
}

hipError_t launch_attn_block_bwd_bf16(const void* dy, const void* x, const void* w_attn,
                                      const void* w_proj, const void* qkv, const void* att,
                                      const float* lse, void* datt, void* dqkv, void* dx,
                                      float* dw_attn, float* db_attn, float* dw_proj,
                                      float* db_proj, float* ws, int B, int T, int H,
                                      hipStream_t stream) {
    const long long C = (long long)H * HEAD_DIM;
    const int R = B * T;
    const BlockWs w = block_ws(B, T, H);
    float* delta = ws + w.delta;
    float* parts = ws + w.slabs;
    float* cp_proj = ws + w.cp_proj;
    float* cp_attn = ws + w.cp_attn;
    // c_proj backward
    hipError_t e = launch_gemm_bf16(false, false, false, dy, C, w_proj, C, datt, C, nullptr, R,
                                    (int)C, (int)C, 1, stream);
    if (e != hipSuccess) return e;
    const int sp_ask = block_splits(R, (int)C, (int)C), sp = slabs_of(R, sp_ask);
    if ((e = launch_gemm_bf16(true, true, true, att, C, dy, C, sp > 1 ? parts : dw_proj, C,
                              nullptr, (int)C, (int)C, R, sp_ask, stream)) != hipSuccess)
        return e;
    // dW_proj's slab sum and db_proj's column-sum partials
    if ((e = slabs_and_colsum(parts, sp, C * C, dw_proj, static_cast<const bf16*>(dy), C, R,
                              (int)C, cp_proj, stream)) != hipSuccess)
        return e;
    // attention backward: dqkv from datt (the dO of the attention)
    if ((e = launch_attn_bwd_dq_pre_bf16(qkv, datt, att, lse, delta, dqkv, B, T, H, stream)) !=
        hipSuccess)
        return e;
    if ((e = launch_attn_bwd_dkdv_bf16(qkv, datt, delta, dqkv, B, T, H, stream)) != hipSuccess)
        return e;
    // c_attn backward
    if ((e = launch_gemm_bf16(false, false, false, dqkv, 3 * C, w_attn, 3 * C, dx, C, nullptr, R,
                              (int)C, (int)(3 * C), 1, stream)) != hipSuccess)
        return e;
    const int sa_ask = block_splits(R, (int)C, (int)(3 * C)), sa = slabs_of(R, sa_ask);
    if ((e = launch_gemm_bf16(true, true, true, x, C, dqkv, 3 * C, sa > 1 ? parts : dw_attn,
                              3 * C, nullptr, (int)C, (int)(3 * C), R, sa_ask, stream)) !=
        hipSuccess)
        return e;
    // dW_attn's slab sum and db_attn's column-sum partials, then both bias sums
    if ((e = slabs_and_colsum(parts, sa, C * 3 * C, dw_attn, static_cast<const bf16*>(dqkv),
                              3 * C, R, (int)(3 * C), cp_attn, stream)) != hipSuccess)
        return e;
    const int nb1 = (int)((C + 63) / 64), nb2 = (int)((3 * C + 63) / 64);
    hipLaunchKernelGGL(colsum_final2_kernel, dim3((unsigned)(nb1 + nb2)), dim3(256), 0, stream,
                       cp_proj, (int)C, db_proj, nb1, cp_attn, (int)(3 * C), db_attn,
                       colsum_chunks(R));
    return hipGetLastError();
}

}  // namespace cattn
