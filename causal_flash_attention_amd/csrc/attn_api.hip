// C ABI of the causal attention library: argument checks, then kernel
// launches on the caller's stream. Declared in include/causal_attn.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "causal_attn.h"

namespace cattn {
hipError_t launch_attn_fwd_bf16(const void*, void*, float*, int, int, int, hipStream_t);
hipError_t launch_attn_bwd_pre_bf16(const void*, const void*, const float*, float*, int, int, int,
                                    hipStream_t);
hipError_t launch_attn_bwd_dkdv_bf16(const void*, const void*, const float*, void*, int, int, int,
                                     hipStream_t);
hipError_t launch_attn_bwd_dq_bf16(const void*, const void*, const float*, void*, int, int, int,
                                   hipStream_t);
hipError_t launch_attn_fwd_unfused_bf16(const void*, void*, float*, void*, void*, int, int, int,
                                        hipStream_t);
hipError_t launch_attn_bwd_unfused_bf16(const void*, const void*, const void*, void*, void*, int,
                                        int, int, hipStream_t);
int unfused_max_T();
long long decode_workspace_floats(int B, int T, int H);
hipError_t launch_attn_decode_bf16(const void*, long long, const void*, const void*, long long,
                                   long long, void*, float*, float*, int, int, int, hipStream_t);
long long unfused_row_stride(int T);
hipError_t launch_attn_bwd_dq_pre_bf16(const void*, const void*, const void*, const float*, float*,
                                       void*, int, int, int, hipStream_t);
long long fp8_buffer_bytes(int B, int T, int H);
long long block_workspace_floats(int B, int T, int H);
long long fp8_bwd_buffer_bytes(int B, int T, int H);
hipError_t launch_attn_quantize_bwd_fp8(const void*, const void*, const void*, const float*, void*,
                                        int, int, int, hipStream_t);
hipError_t launch_attn_bwd_fp8(const void*, const void*, void*, int, int, int, hipStream_t);
hipError_t launch_attn_block_fwd_bf16(const void*, const void*, const void*, const void*,
                                      const void*, void*, void*, float*, void*, int, int, int,
                                      hipStream_t);
hipError_t launch_attn_block_bwd_bf16(const void*, const void*, const void*, const void*,
                                      const void*, const void*, const float*, void*, void*, void*,
                                      float*, float*, float*, float*, float*, int, int, int,
                                      hipStream_t);
hipError_t launch_attn_quantize_fp8(const void*, void*, int, int, int, hipStream_t);
hipError_t launch_attn_fwd_fp8(const void*, void*, float*, int, int, int, hipStream_t);
hipError_t launch_attn_fwd_f32(const float*, float*, float*, int, int, int, hipStream_t);
hipError_t launch_attn_bwd_pre_f32(const float*, const float*, const float*, float*, int, int, int,
                                   hipStream_t);
hipError_t launch_attn_bwd_dkdv_f32(const float*, const float*, const float*, const float*, float*,
                                    int, int, int, hipStream_t);
hipError_t launch_attn_bwd_dq_f32(const float*, const float*, const float*, const float*, float*,
                                  int, int, int, hipStream_t);
long long peak_mfma_flops_per_wg(int iters);
hipError_t launch_peak_mfma(float*, long long*, int, int, hipStream_t);
hipError_t launch_peak_copy(const void*, void*, long long, hipStream_t);
int peak_read_slots();
hipError_t launch_peak_read(const void*, long long, unsigned int*, hipStream_t);
}  // namespace cattn

namespace {

constexpr int kVersion = 10000;  // 1.0.0
constexpr int kHeadDim = 64;
constexpr long long kMaxBytes = 1LL << 62;
constexpr long long kMaxBlocks = 0x7fffffffLL;

thread_local char g_last_error[256];

int fail(int status, const char* what) {
    snprintf(g_last_error, sizeof g_last_error, "%s", what);
    return status;
}

int fail_hip(hipError_t e, const char* where) {
    snprintf(g_last_error, sizeof g_last_error, "%s: %s", where, hipGetErrorString(e));
    return ATTN_ERR_HIP;
}

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
    const char* name;
};

bool overlaps(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

// Shape checks shared by every entry point. Sets *empty when there is
// nothing to compute.
constexpr long long kMaxChannels = 1LL << 23;  // 64 rows * 3C * 2 bytes < 2^32
constexpr int kMaxT = 1 << 30;

int check_shape(int B, int T, int H, int d, int elem, bool* empty) {
    if (B < 0 || T < 0 || H < 0 || d <= 0) return fail(ATTN_ERR_BAD_SHAPE, "B, T, n_head must be >= 0 and head_dim > 0");
    if (d != kHeadDim) return fail(ATTN_ERR_UNSUPPORTED, "head_dim must be 64");
    *empty = (B == 0 || T == 0 || H == 0);
    if (*empty) return ATTN_OK;
    // Tile counts are rounded up from T in 32-bit arithmetic.
    if (T > kMaxT) return fail(ATTN_ERR_TOO_LARGE, "T exceeds 2^30");
    // Largest tensor: qkv / dqkv with B*T*3*H*d elements; grid: B*H*ceil(T/64).
    const long long bt = (long long)B * T;
    const long long c3 = 3LL * H * d;
    if (bt > kMaxBytes / c3 / elem) return fail(ATTN_ERR_TOO_LARGE, "B*T*3*n_head*head_dim overflows");
    const long long blocks = (long long)B * H * (((long long)T + 63) / 64);
    if (blocks > kMaxBlocks) return fail(ATTN_ERR_TOO_LARGE, "launch grid exceeds 2^31-1 workgroups");
    // the preprocess grid: 16 rows of (b, t, h) per workgroup in float32, plus
    // one thread per padded workspace row entry
    const long long tp = ((long long)T + 63) / 64 * 64;
    if (((long long)B * T * H + 15) / 16 + ((long long)B * H * tp + 255) / 256 > kMaxBlocks)
        return fail(ATTN_ERR_TOO_LARGE, "launch grid exceeds 2^31-1 workgroups");
    // Tile loads address 64 packed qkv rows with 32-bit byte offsets.
    if ((long long)H * d > kMaxChannels) return fail(ATTN_ERR_TOO_LARGE, "n_head*head_dim exceeds 2^23");
    return ATTN_OK;
}

int check_aligned(const void* p, uintptr_t a, const char* name) {
    if (reinterpret_cast<uintptr_t>(p) % a != 0) return fail(ATTN_ERR_MISALIGNED, name);
    return ATTN_OK;
}

// Outputs may not overlap any input or any other output.
int check_disjoint(const Span* outs, int n_out, const Span* ins, int n_in) {
    thread_local char msg[128];
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j)
            if (overlaps(outs[i], ins[j])) {
                snprintf(msg, sizeof msg, "%s overlaps %s", outs[i].name, ins[j].name);
                return fail(ATTN_ERR_ALIAS, msg);
            }
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(outs[i], outs[j])) {
                snprintf(msg, sizeof msg, "%s overlaps %s", outs[i].name, outs[j].name);
                return fail(ATTN_ERR_ALIAS, msg);
            }
    }
    return ATTN_OK;
}

Span span(const void* p, long long bytes, const char* name) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, lo + (uintptr_t)bytes, name};
}

struct Sizes {
    // bytes of qkv, of a (B,T,C) tensor, of (B,H,T) fp32, of the backward workspace
    long long qkv, bt_c, rows, ws;
};

long long workspace_floats(int B, int T, int H) {
    const long long tp = ((long long)T + 63) / 64 * 64;
    return 10LL * B * H * tp;  // D, LSE*log2 e, then 32 bytes of MFMA terms per row
}

Sizes sizes(int B, int T, int H, int elem) {
    const long long n = (long long)B * T * H * kHeadDim;
    return Sizes{3 * n * elem, n * elem, (long long)B * H * T * 4, workspace_floats(B, T, H) * 4};
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int fwd_common(const void* qkv, void* out, float* lse, int B, int T, int H, int d, void* stream,
               int elem) {
    g_last_error[0] = '\0';
    bool empty = false;
    if (!(B == 0 || T == 0 || H == 0) && (!qkv || !out || !lse))
        return fail(ATTN_ERR_NULL_PTR, !qkv ? "qkv is NULL" : !out ? "out is NULL" : "lse is NULL");
    int st = check_shape(B, T, H, d, elem, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_aligned(qkv, 16, "qkv must be 16-byte aligned")) != ATTN_OK) return st;
    if ((st = check_aligned(out, 16, "out must be 16-byte aligned")) != ATTN_OK) return st;
    if ((st = check_aligned(lse, 4, "lse must be 4-byte aligned")) != ATTN_OK) return st;
    const Sizes z = sizes(B, T, H, elem);
    const Span ins[] = {span(qkv, z.qkv, "qkv")};
    const Span outs[] = {span(out, z.bt_c, "out"), span(lse, z.rows, "lse")};
    if ((st = check_disjoint(outs, 2, ins, 1)) != ATTN_OK) return st;
    hipError_t e = elem == 2
        ? cattn::launch_attn_fwd_bf16(qkv, out, lse, B, T, H, as_stream(stream))
        : cattn::launch_attn_fwd_f32(static_cast<const float*>(qkv), static_cast<float*>(out), lse,
                                     B, T, H, as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_fwd launch");
}

enum Stage { kPre = 1, kDkdv = 2, kDq = 4, kAll = 7 };

// Backward argument checks and launches. Stage kPre reads dout, out, lse and
// writes the workspace; kDkdv / kDq read dout, qkv and the workspace (the
// float32 kernels also lse) and write dqkv.
int bwd_common(const void* dout, const void* qkv, const void* out, const float* lse, void* dqkv,
               float* ws, int B, int T, int H, int d, void* stream, int elem, int stages) {
    g_last_error[0] = '\0';
    const bool grad = (stages & (kDkdv | kDq)) != 0;
    const bool need_lse = (stages & kPre) || elem == 4;
    const bool nonempty = !(B == 0 || T == 0 || H == 0);
    if (nonempty) {
        if (!dout) return fail(ATTN_ERR_NULL_PTR, "dout is NULL");
        if (grad && !qkv) return fail(ATTN_ERR_NULL_PTR, "qkv is NULL");
        if ((stages & kPre) && !out) return fail(ATTN_ERR_NULL_PTR, "out is NULL");
        if (need_lse && !lse) return fail(ATTN_ERR_NULL_PTR, "lse is NULL");
        if (grad && !dqkv) return fail(ATTN_ERR_NULL_PTR, "dqkv is NULL");
        if (!ws) return fail(ATTN_ERR_NULL_PTR, "delta (workspace) is NULL");
    }
    bool empty = false;
    int st = check_shape(B, T, H, d, elem, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_aligned(dout, 16, "dout must be 16-byte aligned")) != ATTN_OK) return st;
    if (grad && (st = check_aligned(qkv, 16, "qkv must be 16-byte aligned")) != ATTN_OK) return st;
    if ((stages & kPre) && (st = check_aligned(out, 16, "out must be 16-byte aligned")) != ATTN_OK) return st;
    if (need_lse && (st = check_aligned(lse, 4, "lse must be 4-byte aligned")) != ATTN_OK) return st;
    if (grad && (st = check_aligned(dqkv, 16, "dqkv must be 16-byte aligned")) != ATTN_OK) return st;
    if ((st = check_aligned(ws, 16, "delta (workspace) must be 16-byte aligned")) != ATTN_OK) return st;

    const Sizes z = sizes(B, T, H, elem);
    Span ins[5];
    int n_in = 0;
    ins[n_in++] = span(dout, z.bt_c, "dout");
    if (grad) ins[n_in++] = span(qkv, z.qkv, "qkv");
    if (need_lse) ins[n_in++] = span(lse, z.rows, "lse");
    if (stages & kPre) ins[n_in++] = span(out, z.bt_c, "out");
    Span outs[2];
    int n_out = 0;
    if (grad) outs[n_out++] = span(dqkv, z.qkv, "dqkv");
    // The workspace is written by the preprocess stage and read by the others.
    if (stages & kPre) outs[n_out++] = span(ws, z.ws, "delta");
    else ins[n_in++] = span(ws, z.ws, "delta");
    if ((st = check_disjoint(outs, n_out, ins, n_in)) != ATTN_OK) return st;

    const hipStream_t s = as_stream(stream);
    hipError_t e = hipSuccess;
    if (elem == 2 && (stages & kPre) && (stages & kDq)) {
        // The dQ kernel computes the workspace for its own rows on the way
        // (same values as the preprocess stage); dK/dV then reads it.
        e = cattn::launch_attn_bwd_dq_pre_bf16(qkv, dout, out, lse, ws, dqkv, B, T, H, s);
        if (e != hipSuccess) return fail_hip(e, "attn_bwd dQ launch");
        if (stages & kDkdv) {
            e = cattn::launch_attn_bwd_dkdv_bf16(qkv, dout, ws, dqkv, B, T, H, s);
            if (e != hipSuccess) return fail_hip(e, "attn_bwd dK/dV launch");
        }
    } else if (elem == 2) {
        if (stages & kPre) {
            e = cattn::launch_attn_bwd_pre_bf16(dout, out, lse, ws, B, T, H, s);
            if (e != hipSuccess) return fail_hip(e, "attn_bwd preprocess launch");
        }
        if (stages & kDkdv) {
            e = cattn::launch_attn_bwd_dkdv_bf16(qkv, dout, ws, dqkv, B, T, H, s);
            if (e != hipSuccess) return fail_hip(e, "attn_bwd dK/dV launch");
        }
        if (stages & kDq) {
            e = cattn::launch_attn_bwd_dq_bf16(qkv, dout, ws, dqkv, B, T, H, s);
            if (e != hipSuccess) return fail_hip(e, "attn_bwd dQ launch");
        }
    } else {
        const float* f_dout = static_cast<const float*>(dout);
        const float* f_qkv = static_cast<const float*>(qkv);
        float* f_dqkv = static_cast<float*>(dqkv);
        if (stages & kPre) {
            e = cattn::launch_attn_bwd_pre_f32(f_dout, static_cast<const float*>(out), lse, ws, B,
                                               T, H, s);
            if (e != hipSuccess) return fail_hip(e, "attn_bwd_f32 preprocess launch");
        }
        if (stages & kDkdv) {
            e = cattn::launch_attn_bwd_dkdv_f32(f_qkv, f_dout, lse, ws, f_dqkv, B, T, H, s);
            if (e != hipSuccess) return fail_hip(e, "attn_bwd_f32 dK/dV launch");
        }
        if (stages & kDq) {
            e = cattn::launch_attn_bwd_dq_f32(f_qkv, f_dout, lse, ws, f_dqkv, B, T, H, s);
            if (e != hipSuccess) return fail_hip(e, "attn_bwd_f32 dQ launch");
        }
    }
    return ATTN_OK;
}

// ---------------------------------------------------------------------------
// The workspace of attn_bwd_noalloc: one file-scope device array, of which
// every GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is looked up once per device (with that device
// current) and only that address is passed to kernels.
// ---------------------------------------------------------------------------
constexpr long long kNoallocWsFloats = 8LL << 20;  // 32 MiB
constexpr int kMaxDevices = 64;

__device__ __align__(256) float scratch[kNoallocWsFloats];

std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream).
int scratch_for_stream(hipStream_t stream, float** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail_hip(e, "attn_bwd_noalloc: hipGetDevice");
    int dev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return fail_hip(e, "attn_bwd_noalloc: hipStreamGetDevice");
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_ERR_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return fail_hip(e, "attn_bwd_noalloc: hipSetDevice");
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess && r != hipSuccess) e = r;
        }
        if (e != hipSuccess) return fail_hip(e, "attn_bwd_noalloc: hipGetSymbolAddress");
        if (p == nullptr) return fail(ATTN_ERR_HIP, "attn_bwd_noalloc: no device address");
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    return ATTN_OK;
}

// Extra limits of the materialising path: rows of up to unfused_max_T()
// keys held in one wave's registers by the row kernels, and one grid row per
// head in its matrix products.
int check_unfused(int B, int T, int H) {
    if (T > cattn::unfused_max_T())
        return fail(ATTN_ERR_UNSUPPORTED, "the materialising path takes T <= 4096");
    if ((long long)B * H > 65535) return fail(ATTN_ERR_TOO_LARGE, "B*n_head exceeds 65535");
    return ATTN_OK;
}

// Extra limit of the FP8 path: one head's codes (64 * round_up(T, 64) bytes)
// are addressed with 32-bit buffer offsets.
int check_fp8(int T) {
    if (((long long)T + 63) / 64 * 64 * 64 > 0xffffffffLL)
        return fail(ATTN_ERR_TOO_LARGE, "the FP8 path takes round_up(T, 64) * 64 < 2^32");
    return ATTN_OK;
}

// Extra limit of the attention block: its column sums run one grid row per
// 256 token rows.
int check_block(int B, int T) {
    if ((long long)B * T > 65535LL * 256)
        return fail(ATTN_ERR_TOO_LARGE, "the attention block takes B*T <= 16776960");
    return ATTN_OK;
}

int check_all_aligned(const void* const* ptrs, int n, uintptr_t a, const char* what) {
    for (int i = 0; i < n; ++i)
        if (reinterpret_cast<uintptr_t>(ptrs[i]) % a != 0) return fail(ATTN_ERR_MISALIGNED, what);
    return ATTN_OK;
}

long long unfused_ws_bytes(int B, int T, int H) {
    return 6LL * B * H * T * cattn::unfused_row_stride(T);
}

// Size queries answer -1 for a negative argument and for a size past 2^62
// bytes (which no call accepts); the bound is computed in 128 bits before any
// 64-bit size arithmetic runs.
typedef __int128 i128;

bool past_limit(i128 bytes) { return bytes > (i128)kMaxBytes; }

i128 round_up(i128 x, int m) { return (x + m - 1) / m * m; }

}  // namespace

extern "C" {

int attn_fwd(const void* qkv, void* out, float* lse, int B, int T, int n_head, int head_dim,
             void* stream) {
    return fwd_common(qkv, out, lse, B, T, n_head, head_dim, stream, 2);
}

int attn_bwd(const void* dout, const void* qkv, const void* out, const float* lse, void* dqkv,
             float* delta, int B, int T, int n_head, int head_dim, void* stream) {
    return bwd_common(dout, qkv, out, lse, dqkv, delta, B, T, n_head, head_dim, stream, 2, kAll);
}

int attn_bwd_noalloc(const void* dout, const void* qkv, const void* out, const float* lse,
                     void* dqkv, int B, int T, int n_head, int head_dim, void* stream) {
    g_last_error[0] = '\0';
    if (!(B == 0 || T == 0 || n_head == 0) && (!dout || !qkv || !out || !lse || !dqkv))
        return fail(ATTN_ERR_NULL_PTR, "attn_bwd_noalloc: a tensor pointer is NULL");
    bool empty = false;
    int st = check_shape(B, T, n_head, head_dim, 2, &empty);
    if (st != ATTN_OK || empty) return st;
    if (workspace_floats(B, T, n_head) > kNoallocWsFloats)
        return fail(ATTN_ERR_TOO_LARGE, "attn_bwd_noalloc: the workspace of this shape exceeds "
                                        "attn_bwd_noalloc_max_floats()");
    float* ws = nullptr;
    if ((st = scratch_for_stream(as_stream(stream), &ws)) != ATTN_OK) return st;
    return bwd_common(dout, qkv, out, lse, dqkv, ws, B, T, n_head, head_dim, stream, 2, kAll);
}

long long attn_bwd_noalloc_max_floats(void) { return kNoallocWsFloats; }

int attn_bwd_preprocess(const void* dout, const void* out, const float* lse, float* delta, int B,
                        int T, int n_head, int head_dim, void* stream) {
    return bwd_common(dout, nullptr, out, lse, nullptr, delta, B, T, n_head, head_dim, stream, 2,
                      kPre);
}

int attn_bwd_dq_preprocess(const void* dout, const void* qkv, const void* out, const float* lse,
                           void* dqkv, float* delta, int B, int T, int n_head, int head_dim,
                           void* stream) {
    return bwd_common(dout, qkv, out, lse, dqkv, delta, B, T, n_head, head_dim, stream, 2,
                      kPre | kDq);
}

int attn_bwd_dkdv(const void* dout, const void* qkv, const float* delta, void* dqkv, int B, int T,
                  int n_head, int head_dim, void* stream) {
    return bwd_common(dout, qkv, nullptr, nullptr, dqkv, const_cast<float*>(delta), B, T, n_head,
                      head_dim, stream, 2, kDkdv);
}

int attn_bwd_dq(const void* dout, const void* qkv, const float* delta, void* dqkv, int B, int T,
                int n_head, int head_dim, void* stream) {
    return bwd_common(dout, qkv, nullptr, nullptr, dqkv, const_cast<float*>(delta), B, T, n_head,
                      head_dim, stream, 2, kDq);
}

long long attn_unfused_workspace_bytes(int B, int T, int n_head) {
    if (B < 0 || T < 0 || n_head < 0) return -1;
    if (B == 0 || T == 0 || n_head == 0) return 0;
    if (past_limit((i128)6 * B * n_head * T * round_up(T, 8))) return -1;
    return unfused_ws_bytes(B, T, n_head);
}

int attn_fwd_unfused(const void* qkv, void* out, float* lse, void* probs, void* ws, int B, int T,
                     int n_head, int head_dim, void* stream) {
    g_last_error[0] = '\0';
    const int H = n_head;
    if (!(B == 0 || T == 0 || H == 0) && (!qkv || !out || !lse || !probs || !ws))
        return fail(ATTN_ERR_NULL_PTR, "qkv, out, lse, probs and ws must not be NULL");
    bool empty = false;
    int st = check_shape(B, T, H, head_dim, 2, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_unfused(B, T, H)) != ATTN_OK) return st;
    const void* al16[] = {qkv, out, probs, ws};
    for (const void* p : al16)
        if ((st = check_aligned(p, 16, "qkv, out, probs and ws must be 16-byte aligned")) != ATTN_OK)
            return st;
    if ((st = check_aligned(lse, 4, "lse must be 4-byte aligned")) != ATTN_OK) return st;
    const Sizes z = sizes(B, T, H, 2);
    const long long tt = (long long)B * H * T * cattn::unfused_row_stride(T);
    const Span ins[] = {span(qkv, z.qkv, "qkv")};
    const Span outs[] = {span(out, z.bt_c, "out"), span(lse, z.rows, "lse"),
                         span(probs, tt * 2, "probs"), span(ws, tt * 4, "ws")};
    if ((st = check_disjoint(outs, 4, ins, 1)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_attn_fwd_unfused_bf16(qkv, out, lse, probs, ws, B, T, H,
                                                             as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_fwd_unfused launch");
}

int attn_bwd_unfused(const void* dout, const void* qkv, const void* probs, void* dqkv, void* ws,
                     int B, int T, int n_head, int head_dim, void* stream) {
    g_last_error[0] = '\0';
    const int H = n_head;
    if (!(B == 0 || T == 0 || H == 0) && (!dout || !qkv || !probs || !dqkv || !ws))
        return fail(ATTN_ERR_NULL_PTR, "dout, qkv, probs, dqkv and ws must not be NULL");
    bool empty = false;
    int st = check_shape(B, T, H, head_dim, 2, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_unfused(B, T, H)) != ATTN_OK) return st;
    const void* al16[] = {dout, qkv, probs, dqkv, ws};
    for (const void* p : al16)
        if ((st = check_aligned(p, 16, "dout, qkv, probs, dqkv and ws must be 16-byte aligned")) !=
            ATTN_OK)
            return st;
    const Sizes z = sizes(B, T, H, 2);
    const long long tt = (long long)B * H * T * cattn::unfused_row_stride(T);
    const Span ins[] = {span(dout, z.bt_c, "dout"), span(qkv, z.qkv, "qkv"),
                        span(probs, tt * 2, "probs")};
    const Span outs[] = {span(dqkv, z.qkv, "dqkv"), span(ws, unfused_ws_bytes(B, T, H), "ws")};
    if ((st = check_disjoint(outs, 2, ins, 3)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_attn_bwd_unfused_bf16(dout, qkv, probs, dqkv, ws, B, T, H,
                                                             as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_bwd_unfused launch");
}

long long attn_decode_workspace_floats(int B, int T, int n_head) {
    if (B < 0 || T < 0 || n_head < 0) return -1;
    if (B == 0 || T == 0 || n_head == 0) return 0;
    // at most one split per cache row, each of a few hundred bytes
    if (past_limit((i128)B * n_head * T * 1024)) return -1;
    return cattn::decode_workspace_floats(B, T, n_head);
}

int attn_decode(const void* q, long long q_batch_stride, const void* k_cache, const void* v_cache,
                long long cache_row_stride, long long cache_batch_stride, void* out, float* lse,
                float* ws, int B, int T, int n_head, int head_dim, void* stream) {
    g_last_error[0] = '\0';
    const int H = n_head;
    if (!(B == 0 || T == 0 || H == 0) && (!q || !k_cache || !v_cache || !out || !lse || !ws))
        return fail(ATTN_ERR_NULL_PTR, "q, k_cache, v_cache, out, lse and ws must not be NULL");
    bool empty = false;
    int st = check_shape(B, T, H, head_dim, 2, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((long long)B * H > 65535) return fail(ATTN_ERR_TOO_LARGE, "B*n_head exceeds 65535");
    const long long C = (long long)H * head_dim;
    if (q_batch_stride < C || cache_row_stride < C ||
        (B > 1 && cache_batch_stride < (long long)(T - 1) * cache_row_stride + C))
        return fail(ATTN_ERR_BAD_SHAPE, "strides smaller than the rows they step over");
    if (q_batch_stride % 8 || cache_row_stride % 8 || cache_batch_stride % 8)
        return fail(ATTN_ERR_MISALIGNED, "strides must be multiples of 8 elements");
    const long long max_elems = (long long)1 << 61;
    if (cache_batch_stride > max_elems / (B > 0 ? B : 1) || cache_row_stride > max_elems / T ||
        q_batch_stride > max_elems / B)
        return fail(ATTN_ERR_TOO_LARGE, "cache extent overflows");
    const void* al16[] = {q, k_cache, v_cache, out, ws};
    for (const void* p : al16)
        if ((st = check_aligned(p, 16, "q, k_cache, v_cache, out and ws must be 16-byte aligned")) !=
            ATTN_OK)
            return st;
    if ((st = check_aligned(lse, 4, "lse must be 4-byte aligned")) != ATTN_OK) return st;
    const long long cache_elems = (long long)(B - 1) * cache_batch_stride +
                                  (long long)(T - 1) * cache_row_stride + C;
    const Span ins[] = {span(q, ((long long)(B - 1) * q_batch_stride + C) * 2, "q"),
                        span(k_cache, cache_elems * 2, "k_cache"),
                        span(v_cache, cache_elems * 2, "v_cache")};
    const Span outs[] = {span(out, (long long)B * C * 2, "out"),
                         span(lse, (long long)B * H * 4, "lse"),
                         span(ws, cattn::decode_workspace_floats(B, T, H) * 4, "ws")};
    if ((st = check_disjoint(outs, 3, ins, 3)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_attn_decode_bf16(q, q_batch_stride, k_cache, v_cache,
                                                        cache_row_stride, cache_batch_stride, out,
                                                        lse, ws, B, T, H, as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_decode launch");
}

long long attn_block_workspace_bytes(int B, int T, int n_head) {
    if (B < 0 || T < 0 || n_head < 0) return -1;
    if (B == 0 || T == 0 || n_head == 0) return 0;
    // beyond the shapes attn_block_bwd accepts (B * T <= 16776960 and
    // n_head * 64 <= 2^23) the answer is -1
    if ((long long)B * T > 65535LL * 256 || (long long)n_head * kHeadDim > kMaxChannels) return -1;
    const i128 C = (i128)n_head * kHeadDim;
    if (past_limit(4 * ((i128)10 * B * n_head * round_up(T, 64) + 64 * C * 3 * C))) return -1;
    return 4 * cattn::block_workspace_floats(B, T, n_head);
}

int attn_block_fwd(const void* x, const void* w_attn, const void* b_attn, const void* w_proj,
                   const void* b_proj, void* qkv, void* att, float* lse, void* y, int B, int T,
                   int n_head, int head_dim, void* stream) {
    g_last_error[0] = '\0';
    const int H = n_head;
    if (!(B == 0 || T == 0 || H == 0) &&
        (!x || !w_attn || !b_attn || !w_proj || !b_proj || !qkv || !att || !lse || !y))
        return fail(ATTN_ERR_NULL_PTR, "attn_block_fwd: an argument pointer is NULL");
    bool empty = false;
    int st = check_shape(B, T, H, head_dim, 2, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_block(B, T)) != ATTN_OK) return st;
    const void* al16[] = {x, w_attn, w_proj, qkv, att, y};
    if ((st = check_all_aligned(al16, 6, 16, "x, weights, qkv, att and y must be 16-byte aligned")) != ATTN_OK)
        return st;
    const void* al2[] = {b_attn, b_proj};
    if ((st = check_all_aligned(al2, 2, 2, "biases must be 2-byte aligned")) != ATTN_OK) return st;
    if ((st = check_aligned(lse, 4, "lse must be 4-byte aligned")) != ATTN_OK) return st;
    const Sizes z = sizes(B, T, H, 2);
    const long long C = (long long)H * head_dim;
    const Span ins[] = {span(x, z.bt_c, "x"), span(w_attn, C * 3 * C * 2, "w_attn"),
                        span(b_attn, 3 * C * 2, "b_attn"), span(w_proj, C * C * 2, "w_proj"),
                        span(b_proj, C * 2, "b_proj")};
    const Span outs[] = {span(qkv, z.qkv, "qkv"), span(att, z.bt_c, "att"), span(lse, z.rows, "lse"),
                         span(y, z.bt_c, "y")};
    if ((st = check_disjoint(outs, 4, ins, 5)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_attn_block_fwd_bf16(x, w_attn, b_attn, w_proj, b_proj, qkv,
                                                           att, lse, y, B, T, H, as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_block_fwd launch");
}

int attn_block_bwd(const void* dy, const void* x, const void* w_attn, const void* w_proj,
                   const void* qkv, const void* att, const float* lse, void* datt, void* dqkv,
                   void* dx, float* dw_attn, float* db_attn, float* dw_proj, float* db_proj,
                   float* ws, int B, int T, int n_head, int head_dim, void* stream) {
    g_last_error[0] = '\0';
    const int H = n_head;
    if (!(B == 0 || T == 0 || H == 0) &&
        (!dy || !x || !w_attn || !w_proj || !qkv || !att || !lse || !datt || !dqkv || !dx ||
         !dw_attn || !db_attn || !dw_proj || !db_proj || !ws))
        return fail(ATTN_ERR_NULL_PTR, "attn_block_bwd: an argument pointer is NULL");
    bool empty = false;
    int st = check_shape(B, T, H, head_dim, 2, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_block(B, T)) != ATTN_OK) return st;
    const void* al16[] = {dy, x, w_attn, w_proj, qkv, att, datt, dqkv, dx, ws};
    if ((st = check_all_aligned(al16, 10, 16,
                                "matrices, weights and ws must be 16-byte aligned")) != ATTN_OK)
        return st;
    const void* al4[] = {lse, dw_attn, db_attn, dw_proj, db_proj};
    if ((st = check_all_aligned(al4, 5, 4, "lse and the float32 gradients must be 4-byte aligned")) !=
        ATTN_OK)
        return st;
    const Sizes z = sizes(B, T, H, 2);
    const long long C = (long long)H * head_dim;
    const Span ins[] = {span(dy, z.bt_c, "dy"), span(x, z.bt_c, "x"),
                        span(w_attn, C * 3 * C * 2, "w_attn"), span(w_proj, C * C * 2, "w_proj"),
                        span(qkv, z.qkv, "qkv"), span(att, z.bt_c, "att"), span(lse, z.rows, "lse")};
    const Span outs[] = {span(datt, z.bt_c, "datt"), span(dqkv, z.qkv, "dqkv"),
                         span(dx, z.bt_c, "dx"), span(dw_attn, C * 3 * C * 4, "dw_attn"),
                         span(db_attn, 3 * C * 4, "db_attn"), span(dw_proj, C * C * 4, "dw_proj"),
                         span(db_proj, C * 4, "db_proj"),
                         span(ws, 4 * cattn::block_workspace_floats(B, T, H), "ws")};
    if ((st = check_disjoint(outs, 8, ins, 7)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_attn_block_bwd_bf16(
        dy, x, w_attn, w_proj, qkv, att, lse, datt, dqkv, dx, dw_attn, db_attn, dw_proj, db_proj,
        ws, B, T, H, as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_block_bwd launch");
}

long long attn_fp8_bwd_buffer_bytes(int B, int T, int n_head) {
    if (B < 0 || T < 0 || n_head < 0) return -1;
    if (B == 0 || T == 0 || n_head == 0) return 0;
    if (round_up(T, 64) * 64 > 0xffffffffLL) return -1;  // beyond the FP8 path's limit
    // five 64-byte code rows plus 18 side bytes per padded position
    if (past_limit((i128)B * n_head * round_up(T, 64) * 512)) return -1;
    return cattn::fp8_bwd_buffer_bytes(B, T, n_head);
}

int attn_quantize_bwd_fp8(const void* dout, const void* qkv, const void* out, const float* lse,
                          void* fp8_bwd, int B, int T, int n_head, int head_dim, void* stream) {
    g_last_error[0] = '\0';
    const int H = n_head;
    if (!(B == 0 || T == 0 || H == 0) && (!dout || !qkv || !out || !lse || !fp8_bwd))
        return fail(ATTN_ERR_NULL_PTR, "dout, qkv, out, lse and fp8_bwd must not be NULL");
    bool empty = false;
    int st = check_shape(B, T, H, head_dim, 2, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_fp8(T)) != ATTN_OK) return st;
    const void* al16[] = {dout, qkv, out, fp8_bwd};
    if ((st = check_all_aligned(al16, 4, 16, "dout, qkv, out and fp8_bwd must be 16-byte aligned")) != ATTN_OK)
        return st;
    if ((st = check_aligned(lse, 4, "lse must be 4-byte aligned")) != ATTN_OK) return st;
    const Sizes z = sizes(B, T, H, 2);
    const Span ins[] = {span(dout, z.bt_c, "dout"), span(qkv, z.qkv, "qkv"), span(out, z.bt_c, "out"),
                        span(lse, z.rows, "lse")};
    const Span outs[] = {span(fp8_bwd, cattn::fp8_bwd_buffer_bytes(B, T, H), "fp8_bwd")};
    if ((st = check_disjoint(outs, 1, ins, 4)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_attn_quantize_bwd_fp8(dout, qkv, out, lse, fp8_bwd, B, T, H,
                                                             as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_quantize_bwd_fp8 launch");
}

int attn_bwd_fp8(const void* fp8, const void* fp8_bwd, void* dqkv, int B, int T, int n_head,
                 int head_dim, void* stream) {
    g_last_error[0] = '\0';
    const int H = n_head;
    if (!(B == 0 || T == 0 || H == 0) && (!fp8 || !fp8_bwd || !dqkv))
        return fail(ATTN_ERR_NULL_PTR, "fp8, fp8_bwd and dqkv must not be NULL");
    bool empty = false;
    int st = check_shape(B, T, H, head_dim, 2, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_fp8(T)) != ATTN_OK) return st;
    const void* al16[] = {fp8, fp8_bwd, dqkv};
    if ((st = check_all_aligned(al16, 3, 16, "fp8, fp8_bwd and dqkv must be 16-byte aligned")) != ATTN_OK)
        return st;
    const Sizes z = sizes(B, T, H, 2);
    const Span ins[] = {span(fp8, cattn::fp8_buffer_bytes(B, T, H), "fp8"),
                        span(fp8_bwd, cattn::fp8_bwd_buffer_bytes(B, T, H), "fp8_bwd")};
    const Span outs[] = {span(dqkv, z.qkv, "dqkv")};
    if ((st = check_disjoint(outs, 1, ins, 2)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_attn_bwd_fp8(fp8, fp8_bwd, dqkv, B, T, H, as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_bwd_fp8 launch");
}

long long attn_fp8_buffer_bytes(int B, int T, int n_head) {
    if (B < 0 || T < 0 || n_head < 0) return -1;
    if (B == 0 || T == 0 || n_head == 0) return 0;
    if (round_up(T, 64) * 64 > 0xffffffffLL) return -1;  // beyond the FP8 path's limit
    // three 64-byte code rows plus 6 exponent bytes per padded position
    if (past_limit((i128)B * n_head * round_up(T, 64) * 512)) return -1;
    return cattn::fp8_buffer_bytes(B, T, n_head);
}

int attn_quantize_fp8(const void* qkv, void* fp8, int B, int T, int n_head, int head_dim,
                      void* stream) {
    g_last_error[0] = '\0';
    const int H = n_head;
    if (!(B == 0 || T == 0 || H == 0) && (!qkv || !fp8))
        return fail(ATTN_ERR_NULL_PTR, !qkv ? "qkv is NULL" : "fp8 is NULL");
    bool empty = false;
    int st = check_shape(B, T, H, head_dim, 2, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_fp8(T)) != ATTN_OK) return st;
    if ((st = check_aligned(qkv, 16, "qkv must be 16-byte aligned")) != ATTN_OK) return st;
    if ((st = check_aligned(fp8, 16, "fp8 must be 16-byte aligned")) != ATTN_OK) return st;
    const Sizes z = sizes(B, T, H, 2);
    const Span ins[] = {span(qkv, z.qkv, "qkv")};
    const Span outs[] = {span(fp8, cattn::fp8_buffer_bytes(B, T, H), "fp8")};
    if ((st = check_disjoint(outs, 1, ins, 1)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_attn_quantize_fp8(qkv, fp8, B, T, H, as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_quantize_fp8 launch");
}

int attn_fwd_fp8(const void* fp8, void* out, float* lse, int B, int T, int n_head, int head_dim,
                 void* stream) {
    g_last_error[0] = '\0';
    const int H = n_head;
    if (!(B == 0 || T == 0 || H == 0) && (!fp8 || !out || !lse))
        return fail(ATTN_ERR_NULL_PTR, !fp8 ? "fp8 is NULL" : !out ? "out is NULL" : "lse is NULL");
    bool empty = false;
    int st = check_shape(B, T, H, head_dim, 2, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_fp8(T)) != ATTN_OK) return st;
    if ((st = check_aligned(fp8, 16, "fp8 must be 16-byte aligned")) != ATTN_OK) return st;
    if ((st = check_aligned(out, 16, "out must be 16-byte aligned")) != ATTN_OK) return st;
    if ((st = check_aligned(lse, 4, "lse must be 4-byte aligned")) != ATTN_OK) return st;
    const Sizes z = sizes(B, T, H, 2);
    const Span ins[] = {span(fp8, cattn::fp8_buffer_bytes(B, T, H), "fp8")};
    const Span outs[] = {span(out, z.bt_c, "out"), span(lse, z.rows, "lse")};
    if ((st = check_disjoint(outs, 2, ins, 1)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_attn_fwd_fp8(fp8, out, lse, B, T, H, as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_fwd_fp8 launch");
}

long long attn_bwd_workspace_floats(int B, int T, int n_head) {
    if (B < 0 || T < 0 || n_head < 0) return -1;
    if (B == 0 || T == 0 || n_head == 0) return 0;
    if (past_limit((i128)40 * B * n_head * round_up(T, 64))) return -1;
    return workspace_floats(B, T, n_head);
}

int attn_fwd_f32(const float* qkv, float* out, float* lse, int B, int T, int n_head, int head_dim,
                 void* stream) {
    return fwd_common(qkv, out, lse, B, T, n_head, head_dim, stream, 4);
}

int attn_bwd_f32(const float* dout, const float* qkv, const float* out, const float* lse,
                 float* dqkv, float* delta, int B, int T, int n_head, int head_dim, void* stream) {
    return bwd_common(dout, qkv, out, lse, dqkv, delta, B, T, n_head, head_dim, stream, 4, kAll);
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_NULL_PTR: return "ATTN_ERR_NULL_PTR";
        case ATTN_ERR_BAD_SHAPE: return "ATTN_ERR_BAD_SHAPE";
        case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
        case ATTN_ERR_TOO_LARGE: return "ATTN_ERR_TOO_LARGE";
        case ATTN_ERR_MISALIGNED: return "ATTN_ERR_MISALIGNED";
        case ATTN_ERR_ALIAS: return "ATTN_ERR_ALIAS";
        case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
        default: return "ATTN_ERR_UNKNOWN";
    }
}

const char* attn_last_error(void) { return g_last_error; }

int attn_version(void) { return kVersion; }

constexpr int kPeakMax = 1 << 20;

long long attn_peak_mfma_flops(int n_wg, int iters) {
    if (n_wg < 1 || n_wg > kPeakMax || iters < 1 || iters > kPeakMax) return -1;
    return (long long)n_wg * cattn::peak_mfma_flops_per_wg(iters);
}

int attn_peak_mfma(float* out, long long* ticks, int n_wg, int iters, void* stream) {
    g_last_error[0] = '\0';
    if (!out || !ticks) return fail(ATTN_ERR_NULL_PTR, "attn_peak_mfma: out or ticks is NULL");
    if (n_wg < 1 || n_wg > kPeakMax || iters < 1 || iters > kPeakMax)
        return fail(ATTN_ERR_BAD_SHAPE, "attn_peak_mfma: n_wg and iters must lie in [1, 2^20]");
    int st;
    if ((st = check_aligned(out, 4, "out must be 4-byte aligned")) != ATTN_OK) return st;
    if ((st = check_aligned(ticks, 8, "ticks must be 8-byte aligned")) != ATTN_OK) return st;
    const Span outs[1] = {{(uintptr_t)out, (uintptr_t)(out + 256LL * n_wg), "out"}};
    const Span ins[1] = {{(uintptr_t)ticks, (uintptr_t)(ticks + 2LL * n_wg), "ticks"}};
    if ((st = check_disjoint(outs, 1, ins, 1)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_peak_mfma(out, ticks, n_wg, iters, as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_peak_mfma launch");
}

int attn_peak_copy(const void* src, void* dst, long long bytes, void* stream) {
    g_last_error[0] = '\0';
    if (bytes == 0) return ATTN_OK;
    if (!src || !dst) return fail(ATTN_ERR_NULL_PTR, "attn_peak_copy: src or dst is NULL");
    if (bytes < 0 || bytes % 16 != 0)
        return fail(ATTN_ERR_BAD_SHAPE, "attn_peak_copy: bytes must be a non-negative multiple of 16");
    if (bytes > kMaxBytes) return fail(ATTN_ERR_TOO_LARGE, "attn_peak_copy: bytes too large");
    int st;
    if ((st = check_aligned(src, 16, "src must be 16-byte aligned")) != ATTN_OK) return st;
    if ((st = check_aligned(dst, 16, "dst must be 16-byte aligned")) != ATTN_OK) return st;
    const Span outs[1] = {{(uintptr_t)dst, (uintptr_t)dst + (uintptr_t)bytes, "dst"}};
    const Span ins[1] = {{(uintptr_t)src, (uintptr_t)src + (uintptr_t)bytes, "src"}};
    if ((st = check_disjoint(outs, 1, ins, 1)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_peak_copy(src, dst, bytes, as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_peak_copy launch");
}

int attn_peak_read_slots(void) { return cattn::peak_read_slots(); }

int attn_peak_read(const void* src, long long bytes, unsigned int* out, void* stream) {
    g_last_error[0] = '\0';
    if (bytes == 0) return ATTN_OK;
    if (!src || !out) return fail(ATTN_ERR_NULL_PTR, "attn_peak_read: src or out is NULL");
    if (bytes < 0 || bytes % 16 != 0)
        return fail(ATTN_ERR_BAD_SHAPE, "attn_peak_read: bytes must be a non-negative multiple of 16");
    if (bytes > kMaxBytes) return fail(ATTN_ERR_TOO_LARGE, "attn_peak_read: bytes too large");
    int st;
    if ((st = check_aligned(src, 16, "src must be 16-byte aligned")) != ATTN_OK) return st;
    if ((st = check_aligned(out, 4, "out must be 4-byte aligned")) != ATTN_OK) return st;
    const Span outs[1] = {{(uintptr_t)out, (uintptr_t)(out + cattn::peak_read_slots()), "out"}};
    const Span ins[1] = {{(uintptr_t)src, (uintptr_t)src + (uintptr_t)bytes, "src"}};
    if ((st = check_disjoint(outs, 1, ins, 1)) != ATTN_OK) return st;
    const hipError_t e = cattn::launch_peak_read(src, bytes, out, as_stream(stream));
    return e == hipSuccess ? ATTN_OK : fail_hip(e, "attn_peak_read launch");
}

}  // extern "C"
