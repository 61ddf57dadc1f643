/*
 * causal_attn.h -- C ABI of the MI355X (gfx950) causal multi-head
 * self-attention library, forward and backward, FlashAttention style.
 *
 * The operation (the plain definition the kernels reproduce, up to rounding):
 * for every batch row b and head h, with Q, K, V the (T, d) slices of the
 * packed qkv tensor and scale = 1/sqrt(d),
 *
 *     S = scale * Q K^T, masked to -inf where key j > query i
 *     P = row softmax of S,   O = P V,   LSE[i] = ln sum_j exp(S[i, j])
 *
 * and, for an upstream gradient G = dL/dO,
 *
 *     D[i] = sum_k G[i, k] O[i, k],   dS = P * (G V^T - D)
 *     dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T G.
 *
 * Source: flash attention is attention computed without ever keeping the full
 * T x T attention matrix in GPU memory, used in every training step of GPT-2
 * (theprofessional.online summary of "Let's reproduce GPT-2 (124M)",
 * glossary table, row "flash attention"; "Andrej Karpathy - Lets reproduce
 * GPT 2 124M", chapter list, 02:00:18); the model predicts the next token,
 * so the attention is causal (same glossary, row "loss"); the formula is the
 * scaled dot-product attention of "Attention is All You Need", linked from
 * the same chapter list. The pages give no equations: the mask includes the
 * diagonal, the scale is fixed at 1/sqrt(head_dim) and LSE is the natural
 * log of the sum over the scaled logits.
 *
 * Layouts (all contiguous, row-major, C = n_head * head_dim):
 *   qkv   (B, T, 3C)  [Q | K | V] along the last axis; head h occupies
 *                     columns h*d .. h*d+d-1 of each of the three blocks
 *   out   (B, T, C)   same head placement as one block of qkv
 *   lse   (B, n_head, T) float32
 *   dout  (B, T, C)   gradient of the loss with respect to out
 *   dqkv  (B, T, 3C)  [dQ | dK | dV], mirrors qkv; overwritten, never
 *                     accumulated into
 *   delta         float32 workspace of attn_bwd_workspace_floats(B, T, n_head)
 *                 = 10 * B * n_head * Tp floats, Tp = T rounded up to a
 *                 multiple of 64, with R = B * n_head * Tp padded rows and
 *                 row index r = (b * n_head + h) * Tp + t:
 *                   floats [0, R):   D[b, h, t] = sum_k dout * out (0 for t >= T)
 *                   floats [R, 2R):  LSE * log2(e) (+inf for t >= T)
 *                   bytes from 8R:   32 bytes per row in groups of 32 rows
 *                                    (1 KB each): the group's 32 m chunks,
 *                                    eight bf16 [m1 m2 m3 0 0 0 0 0] each,
 *                                    then its 32 D chunks [d1 d2 d3 0 0 0 0
 *                                    0]; m1 + m2 + m3 splits m = 8 * LSE and
 *                                    d1 + d2 + d3 splits D into three bf16
 *                                    terms of decreasing size (for t >= T:
 *                                    m1 = the largest finite bf16, the rest 0)
 *                 written by the backward's preprocess work and read by its
 *                 other stages
 * Element types: the unsuffixed calls take bf16 (IEEE binary32 upper half,
 * passed as void*), accumulate in float32 and round results to nearest-even
 * bf16; the _f32 calls take and produce float32 throughout.
 *
 * Ownership and synchronisation: every pointer is device memory owned by the
 * caller. The library never allocates, frees or synchronises: each call
 * validates its arguments, enqueues its kernels on `stream` (a hipStream_t
 * passed as void*; NULL is the default stream) and returns. ATTN_OK means
 * "validated and enqueued"; a fault inside a kernel surfaces at the caller's
 * next synchronisation. The library holds no state, so calls on different
 * streams may run concurrently as long as their buffers do not overlap.
 *
 * Shapes: head_dim must be 64. B, T and n_head may be any non-negative value
 * with T <= 2^30, n_head * head_dim <= 2^23, whose tensors fit in 2^62 bytes and whose
 * launch grids fit in 2^31 - 1 workgroups; a call with B, T or n_head equal to 0 has nothing to compute
 * and returns ATTN_OK without touching memory (its pointers may then be
 * NULL). qkv, out, dout, dqkv and delta must start on a 16-byte boundary,
 * lse on a 4-byte boundary. Outputs may not overlap inputs or each other.
 *
 * Errors: every call returns a status code and never throws. Argument checks
 * run before any HIP call, in this order: NULL pointer, shape, unsupported
 * head_dim, size overflow, alignment, overlap.
 */
#ifndef CAUSAL_ATTN_H
#define CAUSAL_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL_PTR = -1,     /* a required pointer is NULL */
    ATTN_ERR_BAD_SHAPE = -2,    /* B, T or n_head negative, head_dim <= 0 */
    ATTN_ERR_UNSUPPORTED = -3,  /* head_dim other than 64 */
    ATTN_ERR_TOO_LARGE = -4,    /* a tensor or the launch grid would overflow */
    ATTN_ERR_MISALIGNED = -5,   /* a pointer is not aligned as required */
    ATTN_ERR_ALIAS = -6,        /* an output overlaps an input or another output */
    ATTN_ERR_HIP = -7           /* the HIP runtime refused a launch */
};

/* ---------------------------------------------------------------- bf16 ---- */

/* Forward: out = attention(qkv), lse = per-row log-sum-exp. One kernel. */
int attn_fwd(const void* qkv, void* out, float* lse,
             int B, int T, int n_head, int head_dim, void* stream);

/* Backward: dqkv = gradients of sum(dout * out) with respect to qkv, given
 * the out and lse written by attn_fwd for the same qkv. Runs
 * attn_bwd_dq_preprocess and then attn_bwd_dkdv on `stream` (two kernels);
 * `delta` is the caller's workspace (layout above). */
int attn_bwd(const void* dout, const void* qkv, const void* out, const float* lse,
             void* dqkv, float* delta,
             int B, int T, int n_head, int head_dim, void* stream);

/* The stages of attn_bwd, exported so that each kernel can be launched and
 * timed on its own.
 *   attn_bwd_preprocess:    D = rowsum(dout * out) and LSE * log2(e) into delta
 *   attn_bwd_dkdv:          writes the dK and dV blocks of dqkv (reads delta)
 *   attn_bwd_dq:            writes the dQ block of dqkv (reads delta)
 *   attn_bwd_dq_preprocess: one kernel doing the work of attn_bwd_preprocess
 *                           and attn_bwd_dq (each row's D and LSE * log2(e)
 *                           are computed where its dQ is, and written to
 *                           delta); same arguments as attn_bwd
 * attn_bwd is attn_bwd_dq_preprocess followed by attn_bwd_dkdv. The staged
 * sequence preprocess, dkdv, dq gives the same dqkv and delta bit for bit.
 * dkdv and dq must follow the stage that writes delta on the stream; they
 * write disjoint columns of dqkv and may run in either order. */
int attn_bwd_preprocess(const void* dout, const void* out, const float* lse, float* delta,
                        int B, int T, int n_head, int head_dim, void* stream);
int attn_bwd_dq_preprocess(const void* dout, const void* qkv, const void* out,
                           const float* lse, void* dqkv, float* delta,
                           int B, int T, int n_head, int head_dim, void* stream);
int attn_bwd_dkdv(const void* dout, const void* qkv, const float* delta, void* dqkv,
                  int B, int T, int n_head, int head_dim, void* stream);
int attn_bwd_dq(const void* dout, const void* qkv, const float* delta, void* dqkv,
                int B, int T, int n_head, int head_dim, void* stream);

/* Number of floats the backward workspace `delta` must hold for this shape:
 * 10 * B * n_head * round_up(T, 64). Like every size query here it returns
 * -1 if an argument is negative or the size would pass 2^62 bytes. */
long long attn_bwd_workspace_floats(int B, int T, int n_head);

/* attn_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * same kernels and results as attn_bwd (bit for bit), with the workspace in
 * an array the library keeps in each GPU's memory until the process ends
 * (attn_bwd_noalloc_max_floats() floats, 32 MiB) instead of a `delta`
 * argument; the call itself allocates nothing. Arguments, layouts and
 * errors as attn_bwd, plus ATTN_ERR_TOO_LARGE when
 * attn_bwd_workspace_floats(B, T, n_head) exceeds that size (B 64, T 1024,
 * 12 heads fits). The array is found on the device that runs `stream` (the
 * current device for NULL); the first call on a device looks its address up.
 * Every call on one GPU shares that GPU's array: calls ordered on one stream
 * are safe, calls that may overlap on one GPU (other streams, other threads)
 * race on it and must not be issued. Nothing in it needs to start at zero:
 * the first kernel writes every element the second reads. */
int attn_bwd_noalloc(const void* dout, const void* qkv, const void* out, const float* lse,
                     void* dqkv, int B, int T, int n_head, int head_dim, void* stream);
long long attn_bwd_noalloc_max_floats(void);

/* --------------------------------------------------------------- fp32 ---- */

/* Same operations in float32 storage and arithmetic (same workspace). */
int attn_fwd_f32(const float* qkv, float* out, float* lse,
                 int B, int T, int n_head, int head_dim, void* stream);
int attn_bwd_f32(const float* dout, const float* qkv, const float* out,
                 const float* lse, float* dqkv, float* delta,
                 int B, int T, int n_head, int head_dim, void* stream);

/* ------------------------------------------------ materialising (bf16) ---- */

/* The same attention computed the way a framework does without flash
 * attention, kept as the reference point for it (the pages credit flash
 * attention with a GPT-2 124M step going from 130 ms to 96 ms: "Let's
 * reproduce GPT-2 (124M)", chapter list, 01:48:15 to 02:00:18). Every
 * product runs over the whole T x T square and the scores and
 * probabilities go through HBM:
 *   attn_fwd_unfused: S = QK^T / sqrt(d) as float32 into ws; P =
 *     softmax_rows(causal mask(S)) as bf16 into probs (B, n_head, T, Tp8),
 *     Tp8 = T rounded up to a multiple of 8, with P = 0 above the diagonal
 *     and in the padding columns; lse as for attn_fwd; out = P V.
 *   attn_bwd_unfused: dP = dout V^T as float32 into ws, then dS = P (dP -
 *     rowsum(P dP)) as bf16 after it; dQ = dS K / sqrt(d), dK = dS^T Q /
 *     sqrt(d), dV = P^T dout into dqkv. probs must come from
 *     attn_fwd_unfused on the same qkv.
 * Same layouts, dtypes, status codes and ownership rules as attn_fwd /
 * attn_bwd; ws is a caller-owned device buffer of
 * attn_unfused_workspace_bytes(B, T, n_head) = 6 * B * n_head * T * Tp8
 * bytes. Extra limits: T <= 4096 (ATTN_ERR_UNSUPPORTED) and
 * B * n_head <= 65535 (ATTN_ERR_TOO_LARGE). */
long long attn_unfused_workspace_bytes(int B, int T, int n_head);
int attn_fwd_unfused(const void* qkv, void* out, float* lse, void* probs, void* ws,
                     int B, int T, int n_head, int head_dim, void* stream);
int attn_bwd_unfused(const void* dout, const void* qkv, const void* probs, void* dqkv,
                     void* ws, int B, int T, int n_head, int head_dim, void* stream);

/* ---------------------------------------------------------- decode (bf16) ---- */

/* One new query per (batch, head) against the keys and values of T cached
 * positions, its own included (so no mask): the token-by-token sampling
 * loop ("Let's reproduce GPT-2 (124M)", chapter list, 00:37:02). Per (b, h):
 * O = sum_t softmax_t(q . k_t / sqrt(d)) v_t and LSE = ln sum_t exp(q . k_t /
 * sqrt(d)), in float32 arithmetic.
 *   q        bf16; element (b, h, k) at q[b * q_batch_stride + h * head_dim + k]
 *   k_cache, v_cache
 *            bf16; element (b, t, h, k) at
 *            cache[b * cache_batch_stride + t * cache_row_stride + h * head_dim + k]
 *            for t = 0 .. T-1 (position T-1 is the new token, appended by
 *            the caller). Strides count elements and are multiples of 8. The
 *            packed qkv of attn_fwd can serve directly: k_cache = qkv + C,
 *            v_cache = qkv + 2C, row stride 3C, batch stride T_max * 3C.
 *   out      (B, C) bf16
 *   lse      (B, n_head) float32
 *   ws       float32 workspace of attn_decode_workspace_floats(B, T, n_head)
 * Two kernels on `stream` (split over the cache, then a fixed-order merge;
 * the result does not depend on anything but the inputs). Limits:
 * B * n_head <= 65535; q_batch_stride and cache_row_stride >= C; for B > 1,
 * cache_batch_stride >= (T - 1) * cache_row_stride + C. */
long long attn_decode_workspace_floats(int B, int T, int n_head);
int attn_decode(const void* q, long long q_batch_stride,
                const void* k_cache, const void* v_cache,
                long long cache_row_stride, long long cache_batch_stride,
                void* out, float* lse, float* ws,
                int B, int T, int n_head, int head_dim, void* stream);

/* ------------------------------------------------- attention block (bf16) ---- */

/* The attention layer of GPT-2 around the fused attention ("Let's reproduce
 * GPT-2 (124M)", chapter list, 00:13:47 for the layer, 01:48:15 and 02:00:18
 * for fusing and flash attention): with x (B, T, C), weights stored (in, out)
 * and C = n_head * head_dim,
 *   attn_block_fwd: qkv = x W_attn + b_attn (the packed layout of attn_fwd,
 *     bias added in the product's epilogue); att, lse = attn_fwd(qkv);
 *     y = att W_proj + b_proj (att read in place as the product's operand).
 *   attn_block_bwd: datt = dy W_proj^T; dW_proj = att^T dy;
 *     db_proj = sum over rows of dy; dqkv = attn_bwd(datt, qkv, att, lse);
 *     dx = dqkv W_attn^T; dW_attn = x^T dqkv; db_attn = sum over rows of dqkv.
 * bf16, row-major: x, y, att, dy, datt, dx (B, T, C); qkv, dqkv (B, T, 3C);
 * w_attn (C, 3C); w_proj (C, C); b_attn (3C); b_proj (C). float32: lse
 * (B, n_head, T); dw_attn (C, 3C), db_attn (3C), dw_proj (C, C), db_proj (C),
 * overwritten. qkv, att and lse must come from attn_block_fwd on the same x
 * and weights; datt and dqkv are written by attn_block_bwd (the gradients
 * the layer passes through). ws: caller-owned float32 workspace of
 * attn_block_workspace_bytes(B, T, n_head) bytes (the attention backward's
 * delta, then K-split partial sums of the weight and bias gradients, added
 * in a fixed order: the result does not depend on anything but the inputs).
 * All launches go on `stream`; nothing is allocated. Matrices, weights and ws
 * must be 16-byte aligned, biases 2-byte, float32 gradients and lse 4-byte;
 * no output may overlap an input or another output. Extra limit:
 * B * T <= 16776960 (ATTN_ERR_TOO_LARGE); attn_block_workspace_bytes
 * returns -1 beyond it, for n_head * 64 > 2^23 and for negative arguments. */
long long attn_block_workspace_bytes(int B, int T, int n_head);
int attn_block_fwd(const void* x, const void* w_attn, const void* b_attn, const void* w_proj,
                   const void* b_proj, void* qkv, void* att, float* lse, void* y, int B, int T,
                   int n_head, int head_dim, void* stream);
int attn_block_bwd(const void* dy, const void* x, const void* w_attn, const void* w_proj,
                   const void* qkv, const void* att, const float* lse, void* datt, void* dqkv,
                   void* dx, float* dw_attn, float* db_attn, float* dw_proj, float* db_proj,
                   float* ws, int B, int T, int n_head, int head_dim, void* stream);

/* ------------------------------------------------------------ FP8 (MXFP8) ---- */

/* Causal attention forward with FP8 operands. The llm.c page ("Réimplémenter
 * à bas coût le modèle GPT-2 avec llm.c", FAQ) has BF16 training today and
 * FP8 planned, without a recipe; this is the variant defined here:
 *   - OCP E4M3 elements (round to nearest even) sharing, per block of 32, an
 *     E8M0 scale 2^e with e the smallest integer such that the block's
 *     largest magnitude is <= 448 * 2^e (no element saturates; an all-zero
 *     block takes e = -127). Q and K blocks run along channels, V blocks
 *     along positions (32 aligned positions of one channel, zero past T).
 *   - z = log2(e) * Q^ K^T / sqrt(d) (dequantized operands, causal); per row
 *     an integer reference m = ceil(max z); weights P^ = E4M3(2^(z - m + 8))
 *     * 2^-8; O = P^ V^ / rowsum(P^) in bf16; LSE = ln 2 (m + log2 rowsum(P^))
 *     in float32, the log-normaliser of the weights O uses.
 * attn_quantize_fp8 reads the packed bf16 qkv of attn_fwd and writes the FP8
 * buffer `fp8` (caller-owned device memory of attn_fp8_buffer_bytes(B, T,
 * n_head) bytes, 16-byte aligned). With BH = B * n_head, Tp = round_up(T, 64)
 * and NT = Tp / 64 its layout is
 *   [0, 64 BH Tp)          Q codes, [BH][Tp][64]
 *   [64 BH Tp, 128 BH Tp)  K codes, [BH][Tp][64]
 *   [128 BH Tp, 192 BH Tp) V codes, [BH][64][Tp] (channel-major)
 *   then BH * NT tiles of 384 exponent bytes (e + 127): per tile of 64
 *   positions, bytes [0, 128) hold Q's (position p, channel block c at
 *   2p + c), [128, 256) K's likewise, [256, 384) V's (position block c of the
 *   tile, channel k at 64c + k); positions in [T, Tp) are zero codes with
 *   exponent byte 0.
 * attn_fwd_fp8 reads that buffer and writes out (B, T, C) bf16 and lse
 * (B, n_head, T) float32 as attn_fwd does. Both are single kernels on
 * `stream`, allocate nothing and return the status codes above; extra limit
 * round_up(T, 64) * 64 < 2^32 (ATTN_ERR_TOO_LARGE). The forward assumes
 * |q . k| / sqrt(d) * log2(e) < 2^22 for every score (far beyond attention
 * logits in practice); larger scores can give NaN. The FP8 matrix products
 * sum their 64 exact products with about 14 significant bits (measured), so
 * the results differ from an exact evaluation of the definition where a
 * weight's argument lies within that error of an E4M3 rounding midpoint. */
/* attn_fp8_buffer_bytes and attn_fp8_bwd_buffer_bytes return -1 for negative
 * arguments and beyond the FP8 path's limit on T. */
long long attn_fp8_buffer_bytes(int B, int T, int n_head);
int attn_quantize_fp8(const void* qkv, void* fp8, int B, int T, int n_head, int head_dim,
                      void* stream);
int attn_fwd_fp8(const void* fp8, void* out, float* lse, int B, int T, int n_head, int head_dim,
                 void* stream);

/* FP8 backward: the gradients of L = sum(dout * out) for the FP8 forward,
 * with every product on MXFP8 operands blocked along its own contraction
 * (channels for S = Q K^T and dP = dout V^T; positions for dV = P^T dout,
 * dK = dS^T Q / sqrt(d) and dQ = dS K / sqrt(d)). P = exp(S - lse) enters dV
 * on the forward's fixed grid E4M3(2^8 P) 2^-8; D = rowsum(dout * out);
 * dS = P (dP - D) is quantized per block of 32 queries (for dK) or 32 keys
 * (for dQ) with the forward's block-scale rule.
 * attn_quantize_bwd_fp8 reads dout and out (B, T, C) bf16, qkv, and lse
 * (B, n_head, T) float32 from attn_fwd_fp8, and writes the backward buffer
 * fp8_bwd (caller-owned, attn_fp8_bwd_buffer_bytes(B, T, n_head) bytes,
 * 16-byte aligned). With BH, Tp, NT as above and n = 64 BH Tp:
 *   [0, n) V codes in channel blocks [BH][Tp][64]; [n, 2n) dout likewise;
 *   [2n, 3n) Q codes in position blocks [BH][64][Tp]; [3n, 4n) K likewise;
 *   [4n, 5n) dout likewise; then BH * NT tiles of 1152 bytes per 64
 *   positions: exponent bytes of V (channel blocks, 2 per position), K
 *   (position blocks, 64 per block of 32 positions), dout (channel blocks),
 *   Q and dout (position blocks), 128 bytes each; then the tile's
 *   LSE * log2(e) (+inf past T) and D (0 past T), 64 floats each.
 * attn_bwd_fp8 reads the forward buffer fp8 (attn_quantize_fp8 on the same
 * qkv) and fp8_bwd, and overwrites dqkv (B, T, 3C) bf16: two kernels on
 * `stream`, no atomics (deterministic), nothing allocated; the limits of the
 * forward apply. */
long long attn_fp8_bwd_buffer_bytes(int B, int T, int n_head);
int attn_quantize_bwd_fp8(const void* dout, const void* qkv, const void* out, const float* lse,
                          void* fp8_bwd, int B, int T, int n_head, int head_dim, void* stream);
int attn_bwd_fp8(const void* fp8, const void* fp8_bwd, void* dqkv, int B, int T, int n_head,
                 int head_dim, void* stream);

/* -------------------------------------------------------- measurement ---- */

/* Probes of the two rates the kernels are priced against, measured on the
 * GPU the library runs on; not part of the attention path. They read the
 * chip's sustained rates under load next to its specification (dense bf16
 * MFMA 2516.6 TFLOP/s, HBM3E 8 TB/s).
 *
 * attn_peak_mfma: n_wg workgroups of four waves; each wave runs `iters`
 * rounds of eight independent bf16 32x32x16 MFMAs on register operands
 * (attn_peak_mfma_flops(n_wg, iters) FLOPs in all, -1 for arguments out of
 * range). out: n_wg * 256 floats of the accumulators' sums (meaningless
 * values that keep the work live); ticks: 2 * n_wg int64, the core-clock
 * ticks (s_memtime) and 100 MHz constant-clock ticks (s_memrealtime) of each
 * workgroup's first wave over its loop, whose ratio gives the clock the
 * MFMAs ran at. n_wg and iters lie in [1, 2^20] (else ATTN_ERR_BAD_SHAPE);
 * out 4-byte and ticks 8-byte aligned, not overlapping.
 *
 * attn_peak_copy: copies `bytes` (a multiple of 16) from src to dst with
 * 16-byte nontemporal loads and stores; both 16-byte aligned, not
 * overlapping. bytes = 0 does nothing. Errors as for the attention calls.
 *
 * attn_peak_read: reads `bytes` (a multiple of 16) from src with 16-byte
 * loads; out (4-byte aligned, attn_peak_read_slots() uint32, not overlapping
 * src) receives one XOR of the data per workgroup, which keeps the loads
 * live. bytes = 0 does nothing. */
long long attn_peak_mfma_flops(int n_wg, int iters);
int attn_peak_mfma(float* out, long long* ticks, int n_wg, int iters, void* stream);
int attn_peak_copy(const void* src, void* dst, long long bytes, void* stream);
int attn_peak_read_slots(void);
int attn_peak_read(const void* src, long long bytes, unsigned int* out, void* stream);

/* ------------------------------------------------------------- status ---- */

/* Static, human-readable name of a status code (never NULL). */
const char* attn_status_string(int status);

/* Detail of the last failing call on the calling thread (argument name or
 * HIP error text); "" if none. Valid until the thread's next library call. */
const char* attn_last_error(void);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CAUSAL_ATTN_H */
