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
// into fp32 slabs that a second kernel adds in a fixed order; the bias gradients are column sums done the same way. No
// atomics: the backward is deterministic.
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

// parts[s * N + n] = sum of X[r, n] over the COLSUM_ROWS rows r of chunk s.
// Workgroup (column block, chunk s): thread t owns columns 8 (t % 64) .. +7
// of the block (16-byte loads) and rows 64 (t / 64) .. +63 of the chunk,
// summed in row order; the four row groups are then added in group order
// through LDS. N must be a multiple of 8 and X's rows 16-byte aligned.
__global__ __launch_bounds__(256) void colsum_partial_kernel(const bf16* __restrict__ X,
                                                             long long ld, int R, int N,
                                                             float* __restrict__ parts) {
    __shared__ float red[4][64][9];
    const int t = threadIdx.x, col8 = t & 63, grp = t >> 6;
    const int n0 = blockIdx.x * COLSUM_COLS + 8 * col8;
    const int r0 = blockIdx.y * COLSUM_ROWS + 64 * grp;
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
        float* out = parts + (long long)blockIdx.y * N + n0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            out[e] = ((red[0][col8][e] + red[1][col8][e]) + red[2][col8][e]) + red[3][col8][e];
    }
}

// out[n] = sum over chunks of parts[s * N + n]: thread (column, group) sums
// the chunks s = group, group + 4, ... in order, then the four groups are
// added in group order.
__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ parts,
                                                           int S, int N, float* __restrict__ out) {
    __shared__ float red[4][64];
    const int t = threadIdx.x, c = t & 63, grp = t >> 6;
    const int n = blockIdx.x * 64 + c;
    float acc = 0.0f;
    if (n < N)
        for (int s = grp; s < S; s += 4) acc += parts[(long long)s * N + n];
    red[grp][c] = acc;
    __syncthreads();
    if (grp == 0 && n < N) out[n] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// out[i] = sum over s = 0 .. S-1 of parts[s * n + i], in that order.
__global__ __launch_bounds__(256) void sum_slabs_kernel(const float* __restrict__ parts, int S,
                                                        long long n, float* __restrict__ out) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float acc = 0.0f;
    for (int s = 0; s < S; ++s) acc += parts[(long long)s * n + i];
    out[i] = acc;
}

hipError_t colsum(const bf16* X, long long ld, int R, int N, float* parts, float* out,
                  hipStream_t stream) {
    const int chunks = (R + COLSUM_ROWS - 1) / COLSUM_ROWS;
    hipLaunchKernelGGL(colsum_partial_kernel,
                       dim3((unsigned)((N + COLSUM_COLS - 1) / COLSUM_COLS), (unsigned)chunks),
                       dim3(256), 0, stream, X, ld, R, N, parts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(colsum_final_kernel, dim3((unsigned)((N + 63) / 64)), dim3(256), 0, stream,
                       parts, chunks, N, out);
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

long long block_workspace_floats(int B, int T, int H) {
    const long long C = (long long)H * HEAD_DIM, R = (long long)B * T;
    const long long tp = ((long long)T + 63) / 64 * 64;
    const long long delta = 10LL * B * H * tp;
    const long long s_attn = slabs_of(R, block_splits(R, (int)C, (int)(3 * C)));
    const long long s_proj = slabs_of(R, block_splits(R, (int)C, (int)C));
    long long parts = s_attn * C * 3 * C;
    if (s_proj * C * C > parts) parts = s_proj * C * C;
    const long long cs = (R + COLSUM_ROWS - 1) / COLSUM_ROWS * 3 * C;
    if (cs > parts) parts = cs;
    return delta + parts;
}

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
    const long long tp = ((long long)T + 63) / 64 * 64;
    float* delta = ws;
    float* parts = ws + 10LL * B * H * tp;
    // c_proj backward
    hipError_t e = launch_gemm_bf16(false, false, false, dy, C, w_proj, C, datt, C, nullptr, R,
                                    (int)C, (int)C, 1, stream);
    if (e != hipSuccess) return e;
    const int sp_ask = block_splits(R, (int)C, (int)C), sp = slabs_of(R, sp_ask);
    if ((e = launch_gemm_bf16(true, true, true, att, C, dy, C, sp > 1 ? parts : dw_proj, C,
                              nullptr, (int)C, (int)C, R, sp_ask, stream)) != hipSuccess)
        return e;
    if (sp > 1) {
        hipLaunchKernelGGL(sum_slabs_kernel, dim3((unsigned)((C * C + 255) / 256)), dim3(256), 0,
                           stream, parts, sp, C * C, dw_proj);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = colsum(static_cast<const bf16*>(dy), C, R, (int)C, parts, db_proj, stream)) !=
        hipSuccess)
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
    if (sa > 1) {
        hipLaunchKernelGGL(sum_slabs_kernel, dim3((unsigned)((C * 3 * C + 255) / 256)), dim3(256),
                           0, stream, parts, sa, C * 3 * C, dw_attn);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return colsum(static_cast<const bf16*>(dqkv), 3 * C, R, (int)(3 * C), parts, db_attn, stream);
}

}  // namespace cattn
