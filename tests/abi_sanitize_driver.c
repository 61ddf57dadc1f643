/*
 * Host-side sweep of the C ABI for the address and undefined-behaviour
 * sanitizers (built by tests/test_abi_sanitized.py with the library's host
 * code only). Every entry point and size query is called over a grid of
 * shape values from INT_MIN to INT_MAX, with NULL, misaligned, overlapping
 * and well-formed (fake, far apart) pointers. Only argument validation and
 * size arithmetic run: the process has no GPU, so a call that passes
 * validation fails at its launch with ATTN_ERR_HIP. The sanitizers abort on
 * the first fault; the driver itself checks a few status codes and that
 * every call returns a known one.
 */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "causal_attn.h"

/* From the HIP runtime (plain C declaration): the sweep's fake addresses must
 * never reach a kernel, so the driver refuses to run where a GPU is visible. */
extern int hipGetDeviceCount(int* count);

static const int kShapes[] = {INT_MIN, -1, 0, 1, 2, 63, 64, 65, 1000, 4096, 1 << 17, 1 << 20, 1 << 24, INT_MAX};
static const int kDims[] = {64, 32, 0, -64, INT_MAX};
#define N_SHAPES (int)(sizeof kShapes / sizeof kShapes[0])
#define N_DIMS (int)(sizeof kDims / sizeof kDims[0])

/* Fake device addresses: 16-byte aligned, 2^40 bytes apart, never dereferenced. */
static void* P(int i) { return (void*)(uintptr_t)(((uint64_t)(i + 1)) << 40); }
static void* MIS(int i) { return (void*)((uintptr_t)P(i) + 2); }

static long calls = 0;

static void check(int st, const char* what) {
    ++calls;
    if (st > 0 || st < -7) {
        fprintf(stderr, "%s returned unknown status %d\n", what, st);
        exit(2);
    }
    (void)attn_status_string(st);
    (void)attn_last_error();
}

static void expect(int st, int want, const char* what) {
    check(st, what);
    if (st != want) {
        fprintf(stderr, "%s returned %d, expected %d (%s)\n", what, st, want, attn_last_error());
        exit(3);
    }
}

/* Pointer sets: 0 = all well-formed, 1 = first NULL, 2 = first misaligned,
 * 3 = second equal to the first (overlap). */
static void* ptr(int set, int i) {
    if (i == 0 && set == 1) return NULL;
    if (i == 0 && set == 2) return MIS(0);
    if (i == 1 && set == 3) return P(0);
    return P(i);
}

int main(void) {
    int devices = 0;
    if (hipGetDeviceCount(&devices) == 0 && devices > 0) {
        printf("a GPU is visible: the sweep runs on machines without one\n");
        return 77;
    }
    for (int a = 0; a < N_SHAPES; ++a)
        for (int b = 0; b < N_SHAPES; ++b)
            for (int c = 0; c < N_SHAPES; ++c) {
                const int B = kShapes[a], T = kShapes[b], H = kShapes[c];
                (void)attn_bwd_workspace_floats(B, T, H);
                (void)attn_unfused_workspace_bytes(B, T, H);
                (void)attn_decode_workspace_floats(B, T, H);
                (void)attn_block_workspace_bytes(B, T, H);
                (void)attn_fp8_buffer_bytes(B, T, H);
                (void)attn_fp8_bwd_buffer_bytes(B, T, H);
                calls += 6;
                for (int e = 0; e < N_DIMS; ++e)
                    for (int s = 0; s < 4; ++s) {
                        const int d = kDims[e];
#define p(i) ptr(s, i)
                        check(attn_fwd(p(0), p(1), p(2), B, T, H, d, NULL), "attn_fwd");
                        check(attn_bwd(p(0), p(1), p(2), p(3), p(4), p(5), B, T, H, d, NULL), "attn_bwd");
                        check(attn_bwd_noalloc(p(0), p(1), p(2), p(3), p(4), B, T, H, d, NULL),
                              "attn_bwd_noalloc");
                        check(attn_bwd_preprocess(p(0), p(1), p(2), p(3), B, T, H, d, NULL), "attn_bwd_preprocess");
                        check(attn_bwd_dq_preprocess(p(0), p(1), p(2), p(3), p(4), p(5), B, T, H, d, NULL),
                              "attn_bwd_dq_preprocess");
                        check(attn_bwd_dkdv(p(0), p(1), p(2), p(3), B, T, H, d, NULL), "attn_bwd_dkdv");
                        check(attn_bwd_dq(p(0), p(1), p(2), p(3), B, T, H, d, NULL), "attn_bwd_dq");
                        check(attn_fwd_f32(p(0), p(1), p(2), B, T, H, d, NULL), "attn_fwd_f32");
                        check(attn_bwd_f32(p(0), p(1), p(2), p(3), p(4), p(5), B, T, H, d, NULL), "attn_bwd_f32");
                        check(attn_fwd_unfused(p(0), p(1), p(2), p(3), p(4), B, T, H, d, NULL), "attn_fwd_unfused");
                        check(attn_bwd_unfused(p(0), p(1), p(2), p(3), p(4), B, T, H, d, NULL), "attn_bwd_unfused");
                        check(attn_decode(p(0), 768, p(1), p(2), 768, 1LL << 30, p(3), p(4), p(5), B, T,
                                          H, d, NULL),
                              "attn_decode");
                        check(attn_block_fwd(p(0), p(1), p(2), p(3), p(4), p(5), p(6), p(7), p(8), B, T, H, d,
                                             NULL), "attn_block_fwd");
                        check(attn_block_bwd(p(0), p(1), p(2), p(3), p(4), p(5), p(6), p(7), p(8), p(9),
                                             p(10), p(11), p(12), p(13), p(14), B, T, H, d, NULL),
                              "attn_block_bwd");
                        check(attn_quantize_fp8(p(0), p(1), B, T, H, d, NULL), "attn_quantize_fp8");
                        check(attn_fwd_fp8(p(0), p(1), p(2), B, T, H, d, NULL), "attn_fwd_fp8");
                        check(attn_quantize_bwd_fp8(p(0), p(1), p(2), p(3), p(4), B, T, H, d, NULL),
                              "attn_quantize_bwd_fp8");
                        check(attn_bwd_fp8(p(0), p(1), p(2), B, T, H, d, NULL), "attn_bwd_fp8");
#undef p
                    }
            }
    for (int a = 0; a < N_SHAPES; ++a)
        for (int b = 0; b < N_SHAPES; ++b) {
            (void)attn_peak_mfma_flops(kShapes[a], kShapes[b]);
            check(attn_peak_mfma(P(0), P(1), kShapes[a], kShapes[b], NULL), "attn_peak_mfma");
            const long long bytes = (long long)kShapes[a] * 16;
            check(attn_peak_copy(P(0), P(1), bytes, NULL), "attn_peak_copy");
            check(attn_peak_read(P(0), bytes, P(1), NULL), "attn_peak_read");
            calls += 1;
        }
    check(attn_peak_copy(P(0), P(1), LLONG_MAX - 15, NULL), "attn_peak_copy");
    check(attn_peak_read(P(0), LLONG_MIN, P(1), NULL), "attn_peak_read");

    /* A few fixed expectations (the same as the ctypes tests). */
    expect(attn_fwd(NULL, P(1), P(2), 1, 64, 2, 64, NULL), ATTN_ERR_NULL_PTR, "attn_fwd NULL");
    expect(attn_fwd(P(0), P(1), P(2), -1, 64, 2, 64, NULL), ATTN_ERR_BAD_SHAPE, "attn_fwd B<0");
    expect(attn_fwd(P(0), P(1), P(2), 1, 64, 2, 128, NULL), ATTN_ERR_UNSUPPORTED, "attn_fwd d=128");
    expect(attn_fwd(P(0), P(1), P(2), INT_MAX, INT_MAX, 1 << 17, 64, NULL), ATTN_ERR_TOO_LARGE,
           "attn_fwd huge");
    expect(attn_fwd(MIS(0), P(1), P(2), 1, 64, 2, 64, NULL), ATTN_ERR_MISALIGNED, "attn_fwd misaligned");
    expect(attn_fwd(P(0), P(0), P(2), 1, 64, 2, 64, NULL), ATTN_ERR_ALIAS, "attn_fwd alias");
    expect(attn_fwd(P(0), P(1), P(2), 1, 64, 2, 64, NULL), ATTN_ERR_HIP, "attn_fwd without a GPU");
    expect(attn_fwd(NULL, NULL, NULL, 0, 64, 2, 64, NULL), ATTN_OK, "attn_fwd empty");
    if (attn_bwd_workspace_floats(-1, 1, 1) != -1 || attn_block_workspace_bytes(1, -1, 1) != -1) {
        fprintf(stderr, "size queries must return -1 for negative shapes\n");
        return 4;
    }
    printf("abi sweep: %ld calls, no sanitizer report\n", calls);
    return 0;
}
