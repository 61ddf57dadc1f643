// Measurement probes: the sustained rates of the two resources the attention
// kernels are priced against, measured on the GPU the library runs on, so
// that a kernel's rate can be read against what the chip delivers under load
// as well as against its specification (gfx950: 256 CUs, bf16 MFMA
// 32x32x16, HBM3E).
//
//   peak_mfma_kernel  every wave issues independent chains of bf16
//                     32x32x16 MFMAs on register operands (no memory in the
//                     loop) and records its core-clock and constant-clock
//                     ticks, which give the clock the MFMAs ran at;
//   peak_copy_kernel  a grid-stride copy with 16-byte nontemporal loads and
//                     stores;
//   peak_read_kernel  a grid-stride read with 16-byte loads.
//
// None of them is part of the attention path.
#include "attn_common.h"

namespace cattn {
namespace {

constexpr int PEAK_CHAINS = 8;  // independent accumulators per wave

// out[wg * 256 + thread] = the lane's accumulator sum (keeps the chains
// live); ticks[2 * wg] = core-clock ticks and ticks[2 * wg + 1] = 100 MHz
// constant-clock ticks of the workgroup's wave 0 over its loop.
__global__ __launch_bounds__(256) void peak_mfma_kernel(float* __restrict__ out,
                                                        long long* __restrict__ ticks, int iters) {
    const int lane = threadIdx.x & 63;
    const bf16 x = (bf16)(1.0f + 0.0078125f * (float)(lane & 7));
    const bf16 y = (bf16)(0.0009765625f * (float)((lane >> 3) + 1));
    const bf16x8 a = {x, y, x, y, x, y, x, y};
    const bf16x8 b = {y, x, y, x, y, x, y, x};
    f32x16 acc[PEAK_CHAINS];
#pragma unroll
    for (int c = 0; c < PEAK_CHAINS; ++c) acc[c] = zero16();
    const long long t0 = __builtin_amdgcn_s_memtime();
    const long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < PEAK_CHAINS; ++c) acc[c] = mfma32(a, b, acc[c]);
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    const long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < PEAK_CHAINS; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    out[(long long)blockIdx.x * 256 + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        ticks[2LL * blockIdx.x] = t1 - t0;
        ticks[2LL * blockIdx.x + 1] = r1 - r0;
    }
}

constexpr int PEAK_GRID = 8192;  // workgroups of the copy and read probes (at most)

// dst[i] = src[i] for n 16-byte elements, four per thread per pass, with
// nontemporal loads and stores (the data is touched once).
__global__ __launch_bounds__(256) void peak_copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, long long n) {
    const long long stride = (long long)gridDim.x * 256;
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

// out[workgroup] = XOR of every word the workgroup read (keeps the loads
// live); reads n 16-byte elements, four per thread per pass.
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ src,
                                                        unsigned int* __restrict__ out,
                                                        long long n) {
    __shared__ unsigned int part[4];
    const long long stride = (long long)gridDim.x * 256;
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    unsigned int acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const u32x4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= (unsigned int)__shfl_xor((int)acc, m, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

unsigned int probe_grid(long long n) {
    const long long want = (n + 4LL * 256 - 1) / (4LL * 256);
    return (unsigned int)(want < PEAK_GRID ? (want > 0 ? want : 1) : PEAK_GRID);
}

}  // namespace

long long peak_mfma_flops_per_wg(int iters) {
    return 4LL * iters * PEAK_CHAINS * 32 * 32 * 16 * 2;  // 4 waves per workgroup
}

hipError_t launch_peak_mfma(float* out, long long* ticks, int n_wg, int iters,
                            hipStream_t stream) {
    hipLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)n_wg), dim3(256), 0, stream, out, ticks,
                       iters);
    return hipGetLastError();
}

hipError_t launch_peak_copy(const void* src, void* dst, long long bytes, hipStream_t stream) {
    const long long n = bytes / 16;
    hipLaunchKernelGGL(peak_copy_kernel, dim3(probe_grid(n)), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return hipGetLastError();
}

int peak_read_slots() { return PEAK_GRID; }

hipError_t launch_peak_read(const void* src, long long bytes, unsigned int* out,
                            hipStream_t stream) {
    const long long n = bytes / 16;
    hipLaunchKernelGGL(peak_read_kernel, dim3(probe_grid(n)), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), out, n);
    return hipGetLastError();
}

}  // namespace cattn
