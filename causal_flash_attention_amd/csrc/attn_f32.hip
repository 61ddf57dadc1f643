// Causal attention forward and backward in float32 storage and arithmetic.
//
// Same operation as the bf16 path (scaled dot-product attention with a causal
// mask and its analytic gradients, computed without a T x T buffer, as
// flash attention does in "Let's reproduce GPT-2 (124M)", chapter list,
// 02:00:18), but on the vector ALUs in float32 with the accurate expf/logf,
// for workloads that need float32 results. Tiles of 64 rows are staged in
// LDS; each row of the owned side is handled by two threads, one per half of
// the head dimension (both compute the full-length dot products).
#include "attn_common.h"

namespace cattn {
namespace {

constexpr int F_ROWS = 64;  // owned rows per workgroup (128 threads)
constexpr int F_TILE = 64;  // streamed rows per LDS tile

struct F32Tiles {
    float a[F_TILE][HEAD_DIM];
    float b[F_TILE][HEAD_DIM];
    float ra[F_TILE];
    float rb[F_TILE];
};

// Copy rows [r0, r0 + 64) of a strided float32 matrix into LDS (zero past n).
__device__ __forceinline__ void stage_f32(float (*dst)[HEAD_DIM], const float* base,
                                          long long row_stride, int r0, int n, int tid) {
    for (int e = tid; e < F_TILE * (HEAD_DIM / 4); e += 128) {
        const int r = e / (HEAD_DIM / 4), c4 = e % (HEAD_DIM / 4);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (r0 + r < n) v = *reinterpret_cast<const f32x4*>(base + (long long)(r0 + r) * row_stride + 4 * c4);
        *reinterpret_cast<f32x4*>(&dst[r][4 * c4]) = v;
    }
}

__device__ __forceinline__ float dot64(const float* x, const float (&y)[HEAD_DIM]) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < HEAD_DIM; ++c) s = fmaf(x[c], y[c], s);
    return s;
}

__global__ __launch_bounds__(128) void attn_fwd_f32_kernel(const float* __restrict__ qkv,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse, int B, int T,
                                                           int H, int n_rt, float scale) {
    __shared__ F32Tiles sm;
    const int tid = threadIdx.x, row = tid & 63, half = tid >> 6;
    const int rt = blockIdx.x % n_rt, bh = blockIdx.x / n_rt;
    const int b = bh / H, h = bh - b * H;
    const int C = H * HEAD_DIM;
    const long long rs = 3LL * C;
    const float* qbase = qkv + (long long)b * T * rs + h * HEAD_DIM;
    const int q = rt * F_ROWS + row;
    const bool ok = q < T;

    float qv[HEAD_DIM];
#pragma unroll
    for (int c = 0; c < HEAD_DIM; ++c) qv[c] = ok ? qbase[(long long)q * rs + c] : 0.f;
    float acc[HEAD_DIM / 2];
#pragma unroll
    for (int c = 0; c < HEAD_DIM / 2; ++c) acc[c] = 0.f;
    float m = -INFINITY, l = 0.f;

    const int kend = min(rt * F_ROWS + F_ROWS, T);
    for (int k0 = 0; k0 < kend; k0 += F_TILE) {
        __syncthreads();
        stage_f32(sm.a, qbase + C, rs, k0, T, tid);
        stage_f32(sm.b, qbase + 2 * C, rs, k0, T, tid);
        __syncthreads();
        const int jn = min(F_TILE, q - k0 + 1);  // keys k0 .. q are visible
        for (int j = 0; j < jn; ++j) {
            const float s = dot64(qv, sm.a[j]) * scale;
            const float m_new = fmaxf(m, s);
            const float alpha = expf(m - m_new);
            const float p = expf(s - m_new);
            l = l * alpha + p;
#pragma unroll
            for (int c = 0; c < HEAD_DIM / 2; ++c)
                acc[c] = fmaf(p, sm.b[j][half * 32 + c], acc[c] * alpha);
            m = m_new;
        }
    }
    if (ok) {
        float* op = out + ((long long)b * T + q) * C + h * HEAD_DIM + half * 32;
        const float inv = 1.0f / l;
#pragma unroll
        for (int c = 0; c < HEAD_DIM / 2; ++c) op[c] = acc[c] * inv;
        if (half == 0) lse[(long long)bh * T + q] = m + logf(l);
    }
}

// Workspace layout shared with the bf16 path: per (batch, head) row padded to
// Tp = round_up(T, 64), D in ws[0 .. BH*Tp) and LSE * log2 e in the second
// half (0 and +inf past T). Blocks [0, nb_d) compute D, 16 lanes per row;
// the rest fill the second half and the padding, one thread per entry.
__global__ __launch_bounds__(256) void attn_bwd_pre_f32_kernel(const float* __restrict__ dout,
                                                               const float* __restrict__ out,
                                                               const float* __restrict__ lse,
                                                               float* __restrict__ ws, int T,
                                                               int Tp, int H, long long n_rows,
                                                               long long nb_d,
                                                               long long n_pad_rows) {
    const long long blk = blockIdx.x;
    if (blk < nb_d) {
        const long long row = blk * 16 + (threadIdx.x >> 4);
        const int part = threadIdx.x & 15;
        float acc = 0.f;
        if (row < n_rows) {
            const f32x4 g = *reinterpret_cast<const f32x4*>(dout + row * HEAD_DIM + 4 * part);
            const f32x4 o = *reinterpret_cast<const f32x4*>(out + row * HEAD_DIM + 4 * part);
            acc = g[0] * o[0];
            acc = fmaf(g[1], o[1], acc);
            acc = fmaf(g[2], o[2], acc);
            acc = fmaf(g[3], o[3], acc);
        }
        acc += __shfl_xor(acc, 1, 64);
        acc += __shfl_xor(acc, 2, 64);
        acc += __shfl_xor(acc, 4, 64);
        acc += __shfl_xor(acc, 8, 64);
        if (row < n_rows && part == 0) {
            const long long bt = row / H;
            const int h = (int)(row - bt * H);
            const long long b = bt / T;
            const int t = (int)(bt - b * T);
            ws[(b * H + h) * Tp + t] = acc;
        }
    } else {
        const long long i = (blk - nb_d) * 256 + threadIdx.x;
        if (i < n_pad_rows) {
            const long long bh = i / Tp;
            const int t = (int)(i - bh * Tp);
            if (t < T) {
                ws[n_pad_rows + i] = lse[bh * T + t] * LOG2E;
            } else {
                ws[n_pad_rows + i] = INFINITY;
                ws[i] = 0.f;
            }
        }
    }
}

// dK and dV for 64 keys; streams query tiles from the first one that can see
// these keys to the end of the sequence.
__global__ __launch_bounds__(128) void attn_bwd_dkdv_f32_kernel(
    const float* __restrict__ qkv, const float* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ ws, float* __restrict__ dqkv, int B, int T, int Tp, int H, int n_rt,
    float scale) {
    __shared__ F32Tiles sm;
    const int tid = threadIdx.x, row = tid & 63, half = tid >> 6;
    const int rt = blockIdx.x % n_rt, bh = blockIdx.x / n_rt;
    const int b = bh / H, h = bh - b * H;
    const int C = H * HEAD_DIM;
    const long long rs = 3LL * C;
    const float* qbase = qkv + (long long)b * T * rs + h * HEAD_DIM;
    const float* gbase = dout + (long long)b * T * C + h * HEAD_DIM;
    const float* lse_row = lse + (long long)bh * T;
    const float* d_row = ws + (long long)bh * Tp;
    const int k = rt * F_ROWS + row;
    const bool ok = k < T;

    float kv[HEAD_DIM], vv[HEAD_DIM];
#pragma unroll
    for (int c = 0; c < HEAD_DIM; ++c) {
        kv[c] = ok ? qbase[(long long)k * rs + C + c] : 0.f;
        vv[c] = ok ? qbase[(long long)k * rs + 2 * C + c] : 0.f;
    }
    float dk[HEAD_DIM / 2], dv[HEAD_DIM / 2];
#pragma unroll
    for (int c = 0; c < HEAD_DIM / 2; ++c) dk[c] = dv[c] = 0.f;

    for (int q0 = rt * F_ROWS; q0 < T; q0 += F_TILE) {
        __syncthreads();
        stage_f32(sm.a, qbase, rs, q0, T, tid);
        stage_f32(sm.b, gbase, C, q0, T, tid);
        if (tid < F_TILE) {
            sm.ra[tid] = q0 + tid < T ? lse_row[q0 + tid] : 0.f;
            sm.rb[tid] = q0 + tid < T ? d_row[q0 + tid] : 0.f;
        }
        __syncthreads();
        if (!ok) continue;
        const int i_first = max(0, k - q0);            // queries >= k see this key
        const int i_last = min(F_TILE, T - q0);
        for (int i = i_first; i < i_last; ++i) {
            const float s = dot64(kv, sm.a[i]) * scale;
            const float p = expf(s - sm.ra[i]);
            const float dp = dot64(vv, sm.b[i]);
            const float ds = p * (dp - sm.rb[i]);
#pragma unroll
            for (int c = 0; c < HEAD_DIM / 2; ++c) {
                dv[c] = fmaf(p, sm.b[i][half * 32 + c], dv[c]);
                dk[c] = fmaf(ds, sm.a[i][half * 32 + c], dk[c]);
            }
        }
    }
    if (ok) {
        float* dkp = dqkv + ((long long)b * T + k) * rs + C + h * HEAD_DIM + half * 32;
        float* dvp = dkp + C;
#pragma unroll
        for (int c = 0; c < HEAD_DIM / 2; ++c) {
            dkp[c] = dk[c] * scale;
            dvp[c] = dv[c];
        }
    }
}

// dQ for 64 queries; streams key tiles up to the diagonal.
__global__ __launch_bounds__(128) void attn_bwd_dq_f32_kernel(
    const float* __restrict__ qkv, const float* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ ws, float* __restrict__ dqkv, int B, int T, int Tp, int H, int n_rt,
    float scale) {
    __shared__ F32Tiles sm;
    const int tid = threadIdx.x, row = tid & 63, half = tid >> 6;
    const int rt = blockIdx.x % n_rt, bh = blockIdx.x / n_rt;
    const int b = bh / H, h = bh - b * H;
    const int C = H * HEAD_DIM;
    const long long rs = 3LL * C;
    const float* qbase = qkv + (long long)b * T * rs + h * HEAD_DIM;
    const float* gbase = dout + (long long)b * T * C + h * HEAD_DIM;
    const int q = rt * F_ROWS + row;
    const bool ok = q < T;

    float qv[HEAD_DIM], gv[HEAD_DIM];
#pragma unroll
    for (int c = 0; c < HEAD_DIM; ++c) {
        qv[c] = ok ? qbase[(long long)q * rs + c] : 0.f;
        gv[c] = ok ? gbase[(long long)q * C + c] : 0.f;
    }
    const float lq = ok ? lse[(long long)bh * T + q] : 0.f;
    const float dq_d = ok ? ws[(long long)bh * Tp + q] : 0.f;
    float dq[HEAD_DIM / 2];
#pragma unroll
    for (int c = 0; c < HEAD_DIM / 2; ++c) dq[c] = 0.f;

    const int kend = min(rt * F_ROWS + F_ROWS, T);
    for (int k0 = 0; k0 < kend; k0 += F_TILE) {
        __syncthreads();
        stage_f32(sm.a, qbase + C, rs, k0, T, tid);
        stage_f32(sm.b, qbase + 2 * C, rs, k0, T, tid);
        __syncthreads();
        if (!ok) continue;
        const int jn = min(F_TILE, q - k0 + 1);
        for (int j = 0; j < jn; ++j) {
            const float s = dot64(qv, sm.a[j]) * scale;
            const float p = expf(s - lq);
            const float dp = dot64(gv, sm.b[j]);
            const float ds = p * (dp - dq_d);
#pragma unroll
            for (int c = 0; c < HEAD_DIM / 2; ++c) dq[c] = fmaf(ds, sm.a[j][half * 32 + c], dq[c]);
        }
    }
    if (ok) {
        float* dqp = dqkv + ((long long)b * T + q) * rs + h * HEAD_DIM + half * 32;
#pragma unroll
        for (int c = 0; c < HEAD_DIM / 2; ++c) dqp[c] = dq[c] * scale;
    }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* qkv, float* out, float* lse, int B, int T, int H,
                               hipStream_t stream) {
    const int n_rt = (T + F_ROWS - 1) / F_ROWS;
    const long long blocks = (long long)B * H * n_rt;
    hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)blocks), dim3(128), 0, stream, qkv, out,
                       lse, B, T, H, n_rt, 0.125f);
    return hipGetLastError();
}

int bwd_padded_rows(int T);

hipError_t launch_attn_bwd_pre_f32(const float* dout, const float* out, const float* lse,
                                   float* ws, int B, int T, int H, hipStream_t stream) {
    const int Tp = bwd_padded_rows(T);
    const long long n_rows = (long long)B * T * H;
    const long long nb_d = (n_rows + 15) / 16;
    const long long n_pad_rows = (long long)B * H * Tp;
    const long long nb_l = (n_pad_rows + 255) / 256;
    hipLaunchKernelGGL(attn_bwd_pre_f32_kernel, dim3((unsigned)(nb_d + nb_l)), dim3(256), 0,
                       stream, dout, out, lse, ws, T, Tp, H, n_rows, nb_d, n_pad_rows);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv_f32(const float* qkv, const float* dout, const float* lse,
                                    const float* ws, float* dqkv, int B, int T, int H,
                                    hipStream_t stream) {
    const int n_rt = (T + F_ROWS - 1) / F_ROWS;
    const long long blocks = (long long)B * H * n_rt;
    hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel, dim3((unsigned)blocks), dim3(128), 0, stream, qkv,
                       dout, lse, ws, dqkv, B, T, bwd_padded_rows(T), H, n_rt, 0.125f);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dq_f32(const float* qkv, const float* dout, const float* lse,
                                  const float* ws, float* dqkv, int B, int T, int H,
                                  hipStream_t stream) {
    const int n_rt = (T + F_ROWS - 1) / F_ROWS;
    const long long blocks = (long long)B * H * n_rt;
    hipLaunchKernelGGL(attn_bwd_dq_f32_kernel, dim3((unsigned)blocks), dim3(128), 0, stream, qkv,
                       dout, lse, ws, dqkv, B, T, bwd_padded_rows(T), H, n_rt, 0.125f);
    return hipGetLastError();
}

}  // namespace cattn
