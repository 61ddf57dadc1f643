// Decode attention, bf16 storage, fp32 arithmetic (gfx950).
//
// One new token per (batch, head) attends to the keys and values of all T
// cached positions (its own included, so no mask): the generation loop the
// pages describe as possible but not tuned for inference ("Let's reproduce
// GPT-2 (124M)", chapter list, 00:37:02 on sampling; the llm.c page, FAQ on
// inference). Per (b, h):
//   s_j = q . k_j / sqrt(d),  O = sum_j softmax(s)_j v_j,  LSE = ln sum_j exp(s_j)
//
// The work is a pass over the cache with 2 d flops per byte pair, so it is
// bound by HBM and runs on the vector ALUs, not MFMA. Flash decoding: the T
// keys of a head are split over several workgroups so that every CU streams;
// each workgroup keeps an online softmax (running max, sum and V-weighted sum)
// per group of 8 lanes, one key per group per step, each lane owning 8 of the
// 64 channels (16-byte loads, a 128-byte row per group), merges its 32 groups
// through LDS and writes one partial (m, l, acc[64]); a second kernel merges
// the partials of each head in a fixed order (deterministic, no atomics).
#include "attn_common.h"

namespace cattn {
namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_GROUPS = DEC_THREADS / 8;  // keys per step
constexpr int DEC_PART = 2 + HEAD_DIM;       // floats per partial: m, l, acc[64]

struct DecodeArgs {
    const bf16* q;
    long long q_bs;  // elements between batch rows of q
    const bf16* k;
    const bf16* v;
    long long row_stride, batch_stride;  // cache elements between positions / batch rows
    int T, H, n_split, keys_per_split;
    float c_log2;  // scale * log2 e
};

// Partials of split `blockIdx.x` of head blockIdx.y; base-2 logits.
__global__ __launch_bounds__(DEC_THREADS) void decode_partial_kernel(DecodeArgs a, float* ws) {
    __shared__ float red[DEC_GROUPS][DEC_PART];
    const int tid = threadIdx.x, grp = tid >> 3, part = tid & 7;  // part: channels 8p .. 8p+7
    const int bh = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
    const int t0 = blockIdx.x * a.keys_per_split;
    const int t1 = min(t0 + a.keys_per_split, a.T);

    float q[8];
    {
        const bf16x8 qv = *reinterpret_cast<const bf16x8*>(a.q + b * a.q_bs + h * HEAD_DIM + 8 * part);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (float)qv[e] * a.c_log2;
    }
    const long long base = b * a.batch_stride + h * HEAD_DIM + 8 * part;
    float m = -INFINITY, l = 0.0f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    // One key per group per step (more keys per step, with their loads
    // issued together, measured slower), online update of (m, l, acc).
    for (int t = t0 + grp; t < t1; t += DEC_GROUPS) {
        const long long off = base + (long long)t * a.row_stride;
        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(a.k + off);
        const bf16x8 vv = *reinterpret_cast<const bf16x8*>(a.v + off);
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(q[e], (float)kv[e], s);
        s += __shfl_xor(s, 1, 8);
        s += __shfl_xor(s, 2, 8);
        s += __shfl_xor(s, 4, 8);
        const float m_new = fmaxf(m, s);
        const float alpha = exp2f(m - m_new);  // 0 on the first key (m = -inf)
        const float p = exp2f(s - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, (float)vv[e], acc[e] * alpha);
        m = m_new;
    }
    // Merge the groups: each group's m, l (lane 0 of the group) and acc.
    if (part == 0) {
        red[grp][0] = m;
        red[grp][1] = l;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[grp][2 + 8 * part + e] = acc[e];
    __syncthreads();
    float* out = ws + ((long long)bh * a.n_split + blockIdx.x) * DEC_PART;
    if (tid < HEAD_DIM) {
        float mx = -INFINITY;
        for (int g = 0; g < DEC_GROUPS; ++g) mx = fmaxf(mx, red[g][0]);
        float lt = 0.0f, at = 0.0f;
        if (mx != -INFINITY) {
            for (int g = 0; g < DEC_GROUPS; ++g) {
                const float w = exp2f(red[g][0] - mx);  // 0 for groups that saw no key
                lt = fmaf(red[g][1], w, lt);
                at = fmaf(red[g][2 + tid], w, at);
            }
        }
        out[2 + tid] = at;
        if (tid == 0) {
            out[0] = mx;
            out[1] = lt;
        }
    }
}

// Merge the n_split partials of each head in split order; O = acc / l,
// LSE = ln 2 (m + log2 l).
__global__ __launch_bounds__(HEAD_DIM) void decode_combine_kernel(const float* ws, bf16* out,
                                                                  float* lse, int H, int n_split) {
    const int bh = blockIdx.x, d = threadIdx.x;
    const float* p = ws + (long long)bh * n_split * DEC_PART;
    float mx = -INFINITY;
    for (int s = 0; s < n_split; ++s) mx = fmaxf(mx, p[s * DEC_PART]);
    float lt = 0.0f, at = 0.0f;
    for (int s = 0; s < n_split; ++s) {
        const float w = p[s * DEC_PART] == -INFINITY ? 0.0f : exp2f(p[s * DEC_PART] - mx);
        lt = fmaf(p[s * DEC_PART + 1], w, lt);
        at = fmaf(p[s * DEC_PART + 2 + d], w, at);
    }
    const int b = bh / H, h = bh - b * H;
    out[(long long)b * H * HEAD_DIM + h * HEAD_DIM + d] = (bf16)(at / lt);
    if (d == 0) lse[bh] = (mx + log2f(lt)) * LN2;
}

}  // namespace

// Splits per head: enough workgroups to cover the chip (about 2048), each
// with at least 64 keys.
int decode_splits(int BH, int T) {
    long long n = (2048LL + BH - 1) / (BH > 0 ? BH : 1);
    const long long max_n = (T + 63LL) / 64;
    if (n > max_n) n = max_n;
    return n < 1 ? 1 : (int)n;
}

long long decode_workspace_floats(int B, int T, int H) {
    const long long BH = (long long)B * H;
    return BH * decode_splits((int)(BH > 0x7fffffff ? 0x7fffffff : BH), T) * DEC_PART;
}

hipError_t launch_attn_decode_bf16(const void* q, long long q_bs, const void* k, const void* v,
                                   long long row_stride, long long batch_stride, void* out,
                                   float* lse, float* ws, int B, int T, int H, hipStream_t stream) {
    const int BH = B * H;
    const int n_split = decode_splits(BH, T);
    const DecodeArgs a{static_cast<const bf16*>(q), q_bs, static_cast<const bf16*>(k),
                       static_cast<const bf16*>(v), row_stride, batch_stride, T, H, n_split,
                       (T + n_split - 1) / n_split, LOG2E / 8.0f};
    hipLaunchKernelGGL(decode_partial_kernel, dim3((unsigned)n_split, (unsigned)BH),
                       dim3(DEC_THREADS), 0, stream, a, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)BH), dim3(HEAD_DIM), 0, stream, ws,
                       static_cast<bf16*>(out), lse, H, n_split);
    return hipGetLastError();
}

}  // namespace cattn
