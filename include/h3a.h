/*
 * h3a.h -- C ABI of the rotated-int8 ("kvi8r") K/V store and token-chunked
 * long-sequence attention library for AMD Instinct MI355X (gfx950).
 *
 * What the calls compute follows three pages:
 *   [P1] "H3 Streamed Blocks (exact low-VRAM, alpha)" node page:
 *        "How it works" and the Inputs table (rows q_chunk, kv_chunk, kv_block,
 *        kv_store, exact_av_rows).
 *   [P2] "Low VRAM, low RAM: the de-rope on a 16 GB card" page:
 *        "The K/V store options" (table and rotation paragraph),
 *        "What is exact, and what is not" and "What is next".
 *   [P3] "H3-Optimizations" extension page: "Nodes" (H3 Sparse Attention,
 *        H3 Sparse Attention (Advanced) and the routed-geometry paragraph).
 *
 * Conventions shared by every call
 *   - Every tensor pointer is device memory owned by the caller, and must stay
 *     valid until the work queued on `stream` has finished.  Exceptions:
 *     h3a_attention_routed's exact_spans (host memory, read during the call)
 *     and h3a_attention_host_kv's store (pinned host memory).  The library keeps
 *     no pointer after a call returns and allocates no device memory; scratch
 *     space comes only through the `workspace` argument.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     GPU work is queued asynchronously on it, in call order.
 *   - Arguments are checked before anything is queued.  A failed check returns
 *     a negative status, queues nothing, and leaves a one-line reason in
 *     h3a_last_error().  Device pointers are checked to lie inside one device
 *     allocation large enough for the access the call will make.
 *   - No fallback: a request the library cannot serve is an error, never a
 *     silent substitute [P3, Nodes: explicit selections are hard requirements].
 *   - head_dim must be 128: the width of the fixed Hadamard basis [P1 kv_store].
 *   - Token-major tensors are [tokens, n_heads, 128] with the 128 values of a
 *     (token, head) row contiguous.
 *   - The attention calls take 1 <= n_heads <= 65536, 0 <= s_kv < 2^31 and
 *     0 <= s_q <= 2^31; other sizes are H3A_EINVAL.
 */
#ifndef H3A_H
#define H3A_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3A_ABI_VERSION 1
#define H3A_HEAD_DIM 128
#define H3A_TILE 64 /* 64Q x 64KV routing granularity [P3] */

/* Status codes. */
#define H3A_OK 0
#define H3A_EINVAL (-1)       /* an argument is out of range, null, misaligned or too small */
#define H3A_EUNSUPPORTED (-2) /* a valid request this library does not implement (e.g. head_dim != 128) */
#define H3A_EHIP (-3)         /* the HIP runtime reported an error (text in h3a_last_error) */
#define H3A_EWORKSPACE (-4)   /* workspace missing or smaller than h3a_attention_workspace_bytes */

/* K/V store kinds, named after the kv_store choices they implement [P1 kv_store]. */
#define H3A_MODE_EXACT_BF16 0 /* "bf16 (exact)": K/V kept as bf16, stock attention math */
#define H3A_MODE_KVI8R 1      /* "kvi8r": rotated int8 K/V with one fp16 scale per (token, head) row */
#define H3A_MODE_KVI8R32 2    /* "kvi8r32": the same with one fp16 scale per 32 rotated values [P2 What is next] */

/* Flag OR-ed into mode (with a tile_mask only): every dropped KV tile still
 * contributes, as one pseudo-key -- its block-mean key with its block-mean value,
 * counted as many times as the tile has keys -- instead of being left out of the
 * softmax (the Sol arm, which stands in for rejected tiles with block-mean K and
 * block-sum V [P3 Nodes, routed geometry]). */
#define H3A_SOL 0x100

/* Flag OR-ed into H3A_MODE_KVI8R or H3A_MODE_KVI8R32: `out` is fp16 instead of
 * bf16.  kvi8r attention runs in fp16 [P1 kv_store; P2 "The K/V store options":
 * why fp16 and not bf16 inside kvi8r], and fp16 keeps that precision in the
 * output: rounding the exact result to fp16 costs about 2e-4 relative (RMS)
 * against about 1.7e-3 for bf16, whose half-ulp above 2.0 alone is 7.8e-3.
 * The row is un-rotated in fp32 and rounded once, to fp16 here or to bf16
 * without the flag, so the two outputs are two roundings of one value.  With
 * the exact store it is H3A_EINVAL (that output is bf16). */
#define H3A_OUT_F16 0x200

/* ABI version of the loaded library; callers compare it with H3A_ABI_VERSION. */
int32_t h3a_abi_version(void);

/* One line describing the last failed check on the calling thread ("" if none). */
const char* h3a_last_error(void);

/*
 * h3a_kv_quantize -- build one kv_chunk of the kvi8r store [P1 kv_chunk, kv_store].
 *
 * For every (token, head) row x of the chunk (128 bf16 values):
 *   y = x H, H the orthonormal 128x128 Sylvester Hadamard basis (natural order,
 *     entries +-1/sqrt(128));
 *   scale = fp16(max|y| / 127), rounded to nearest-even from the exact value;
 *     0 for a zero row; saturates at 65504;
 *   code_i = clamp(round-half-even(y_i / scale), -127, 127) as int8, against
 *     the stored (rounded) scale.  y_i / scale is evaluated in fp32 (butterflies,
 *     then one product with an fp32 reciprocal of the scale), so where it lies
 *     within that evaluation's rounding error of a half-step (about 1e-4 of a
 *     step for Gaussian rows) the code may be either neighbour.
 *
 * x:               bf16 [n_tokens, n_heads, 128]; token t, head h starts at
 *                  element t * x_token_stride + h * 128.  16-byte aligned.
 * x_token_stride:  elements between consecutive tokens; >= n_heads * 128 and a
 *                  multiple of 8 (so a slice of a fused QKV buffer can be passed).
 * token_offset:    first store row written; token_offset + n_tokens <= s_total.
 * s_total:         rows per head of the whole store.
 * codes:           int8  [n_heads, s_total, 128] (head-major), 16-byte aligned.
 * scales_f16:      fp16  [n_heads, s_total] (head-major), 2-byte aligned.
 * Rows [token_offset, token_offset + n_tokens) of every head are written;
 * nothing else is touched, so a store can be built chunk by chunk and the
 * result equals one call over all tokens.  n_tokens == 0 is a no-op.
 * Inputs must be finite (a non-finite row gets unspecified codes and scale).
 */
int32_t h3a_kv_quantize(const void* x, int64_t x_token_stride, int64_t n_tokens, int32_t n_heads,
                        int32_t head_dim, int64_t token_offset, int64_t s_total, int8_t* codes,
                        void* scales_f16, void* stream);

/*
 * h3a_kv_quantize_g32 -- build one kv_chunk of the kvi8r32 store: the
 * per-32-value scale variant of kvi8r [P2 "What is next": finer than per row].
 *
 * As h3a_kv_quantize, except that each rotated row y is cut into four groups
 * of 32 consecutive values (y_0..y_31, y_32..y_63, y_64..y_95, y_96..y_127) and
 * every group g gets its own scale_g = fp16(max|y in g| / 127), its codes taken
 * against scale_g in the same way.
 *
 * scales_f16:      fp16 [n_heads, s_total, 4] (head-major, the four group
 *                  scales of a row together), 8-byte aligned.
 */
int32_t h3a_kv_quantize_g32(const void* x, int64_t x_token_stride, int64_t n_tokens, int32_t n_heads,
                            int32_t head_dim, int64_t token_offset, int64_t s_total, int8_t* codes,
                            void* scales_f16, void* stream);

/*
 * h3a_kv_quantize_pair -- h3a_kv_quantize of K and V of one kv_chunk in one
 * launch: the projection produces a chunk's K and V together [P1 kv_chunk:
 * the K/V buffers are built chunk by chunk], and one launch over both keeps
 * the GPU streaming twice as long between launch ramps.
 *
 * k, v:            bf16 [n_tokens, n_heads, 128], both with the same
 *                  x_token_stride (e.g. two slices of a fused QKV buffer).
 * k_codes, v_codes: int8 [n_heads, s_total, 128] each, distinct buffers.
 * scales_f16:      fp16 [2, n_heads, s_total]: K scales, then V scales, the
 *                  layout h3a_attention takes.
 * Every other argument, the result and the errors are those of two
 * h3a_kv_quantize calls (bitwise the same codes and scales).
 */
int32_t h3a_kv_quantize_pair(const void* k, const void* v, int64_t x_token_stride, int64_t n_tokens, int32_t n_heads,
                             int32_t head_dim, int64_t token_offset, int64_t s_total, int8_t* k_codes,
                             int8_t* v_codes, void* scales_f16, void* stream);

/*
 * h3a_attention_workspace_bytes -- bytes of workspace h3a_attention needs.
 * sparse != 0 when a tile_mask will be passed; mode as passed to h3a_attention
 * (including H3A_SOL).  Returns 0 when none is needed or the arguments are
 * invalid.
 */
size_t h3a_attention_workspace_bytes(int64_t s_q, int64_t s_kv, int32_t n_heads, int32_t head_dim,
                                     int64_t q_chunk, int32_t mode, int32_t sparse);

/*
 * h3a_attention -- token-chunked full (non-causal) attention of every head
 * against a whole-sequence K/V store [P1 "How it works", q_chunk, kv_block,
 * kv_store; P2 "The K/V store options"; P3 Nodes for tile_mask].
 *
 *   O[t, h, :] = sum_j softmax_j(softmax_scale * q[t,h,:] . k[j,h,:]) v[j,h,:]
 *
 * mode is H3A_MODE_EXACT_BF16, H3A_MODE_KVI8R or H3A_MODE_KVI8R32, optionally OR-ed
 * with H3A_SOL and (kvi8r stores) H3A_OUT_F16.
 * mode H3A_MODE_EXACT_BF16: k_store / v_store are bf16 [s_kv, n_heads, 128]
 *   (token-major), scales must be NULL.  Inputs feed bf16 matrix cores, fp32
 *   accumulation.  The output is bitwise identical for every q_chunk and
 *   kv_block (each row's arithmetic depends only on s_kv).
 * mode H3A_MODE_KVI8R: k_store / v_store are the int8 codes [n_heads, s_kv, 128]
 *   written by h3a_kv_quantize, scales is fp16 [2, n_heads, s_kv] (K scales,
 *   then V scales).  Each query chunk is rotated into the Hadamard basis
 *   (rounded to fp16), attends the K/V rows dequantised on the fly as one
 *   int8 -> fp16 cast times the row scale, with fp16 matrix-core products and
 *   fp32 accumulation, and the output is rotated back once per row.
 * mode H3A_MODE_KVI8R32: as H3A_MODE_KVI8R over the store written by
 *   h3a_kv_quantize_g32; scales is fp16 [2, n_heads, s_kv, 4], 8-byte aligned.
 *   Each K and V row is dequantised group by group (code * group scale,
 *   rounded to fp16) before the fp16 matrix-core products.  The rotated query
 *   is multiplied by softmax_scale * log2(e) before its one rounding to fp16,
 *   so this mode takes softmax_scale * log2(e) <= 1 in fp32, i.e. softmax_scale
 *   up to ln 2 (larger is H3A_EINVAL).
 *
 * q:          bf16 [s_q, n_heads, 128], 16-byte aligned.
 * out:        bf16 [s_q, n_heads, 128] (fp16 with H3A_OUT_F16), 16-byte
 *             aligned; must not alias inputs.
 * q_chunk:    query tokens per pass (>= 1; a multiple of 64 when tile_mask is
 *             given).  Query chunks are attended one after another on `stream`.
 * kv_block:   K/V block length of the online-softmax (log-sum-exp) combine:
 *             0 (mode default) or a positive multiple of 64.  The softmax state
 *             is carried in registers across blocks, so the result does not
 *             depend on it.
 * tile_mask:  NULL for dense attention, else uint8 [n_heads, ceil(s_q/64),
 *             ceil(s_kv/64)]: entry != 0 keeps the 64-query x 64-key tile, 0
 *             drops it from the softmax (hard arm).  A query row with no kept
 *             key gets an all-zero output, as does every row when s_kv == 0.
 *             With mode | H3A_SOL, a dropped tile t of n_t keys adds one
 *             pseudo-key instead: the mean of its keys, with the mean of its
 *             values, at softmax weight n_t * exp(scale * q . mean key).  The
 *             means are taken once per call over the dequantised store in fp32
 *             and rounded to the matrix-core input type (fp16 for kvi8r, bf16
 *             for exact); the mean key is first scaled by a power of two, an
 *             exact step that keeps it inside the fp16 range.  A query row whose
 *             tiles are all dropped attends the pseudo-keys alone.  H3A_SOL
 *             without a tile_mask, or with s_kv > 2^30 - 64, is H3A_EINVAL.
 * workspace:  at least h3a_attention_workspace_bytes(...) bytes of device
 *             memory, 256-byte aligned (may be NULL when that is 0).
 */
int32_t h3a_attention(const void* q, const void* k_store, const void* v_store, const void* scales,
                      int64_t s_q, int64_t s_kv, int32_t n_heads, int32_t head_dim, float softmax_scale,
                      int64_t q_chunk, int64_t kv_block, int32_t mode, const uint8_t* tile_mask,
                      void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * h3a_attention_noalloc -- h3a_attention for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 *
 * Same arguments, checks, kernels and results as h3a_attention (bitwise), with
 * no workspace argument: the scratch it needs (rotated query chunk, rotated
 * output, tile lists, tile means) lives in a device array inside the library,
 * H3A_NOALLOC_SCRATCH_BYTES bytes on every GPU it runs on, held until the
 * process ends.  The call makes no hipMalloc / hipFree and calls no allocating
 * routine.  The caller still owns q, the store, tile_mask and out.
 *
 * A call whose h3a_attention_workspace_bytes(...) exceeds
 * H3A_NOALLOC_SCRATCH_BYTES returns H3A_EWORKSPACE and queues nothing.  The
 * output does not depend on q_chunk, so a smaller q_chunk gives the same
 * result with less scratch (kvi8r modes need 768 bytes per query row and
 * head of a chunk: q_chunk 8192 at 32 heads fits).
 *
 * Every call on one GPU uses that GPU's one array, which keeps whatever the
 * last call left there; every kernel writes the scratch it reads within the
 * same call, so nothing needs clearing.  Calls that overlap on one GPU (queued
 * on different streams without ordering between them) race on the array: order
 * them on one stream, or use h3a_attention with a workspace each.
 */
#define H3A_NOALLOC_SCRATCH_BYTES (256u << 20) /* 256 MiB per GPU */
int32_t h3a_attention_noalloc(const void* q, const void* k_store, const void* v_store, const void* scales,
                              int64_t s_q, int64_t s_kv, int32_t n_heads, int32_t head_dim, float softmax_scale,
                              int64_t q_chunk, int64_t kv_block, int32_t mode, const uint8_t* tile_mask,
                              void* out, void* stream);

/*
 * h3a_attention_routed -- h3a_attention over two stores of the same K/V, chosen
 * per query row [P1 Inputs table, exact_av_rows row: text and audio rows attend
 * a retained bf16 K/V exactly, the other rows the quantised store].
 *
 * Rows inside one of the n_spans [begin, end) spans of exact_spans get exact
 * attention over k_bf16 / v_bf16 (bf16 [s_kv, n_heads, 128], as
 * H3A_MODE_EXACT_BF16); every other row gets kvi8r attention over k_codes /
 * v_codes / scales (as H3A_MODE_KVI8R).  Each row's output is bitwise the one
 * h3a_attention gives it in that mode.  Rows are attended in increasing
 * order, each stretch of one mode in passes of at most q_chunk rows.
 *
 * out:         bf16 [s_q, n_heads, 128] for every row (no H3A_OUT_F16 here:
 *              both stores' rows go to one bf16 tensor).
 * exact_spans: HOST memory, n_spans pairs of int64 (begin, end) with
 *              0 <= begin <= end <= s_q, increasing and disjoint
 *              (end_i <= begin_{i+1}); NULL when n_spans == 0.  Read during
 *              the call only.
 * workspace:   h3a_attention_workspace_bytes(s_q, s_kv, n_heads, 128, q_chunk,
 *              H3A_MODE_KVI8R, 0) bytes.
 * Other arguments as for h3a_attention.  Dense only (no tile_mask).
 */
int32_t h3a_attention_routed(const void* q, const void* k_bf16, const void* v_bf16, const void* k_codes,
                             const void* v_codes, const void* scales, int64_t s_q, int64_t s_kv, int32_t n_heads,
                             int32_t head_dim, float softmax_scale, int64_t q_chunk, int64_t kv_block,
                             const int64_t* exact_spans, int32_t n_spans, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * h3a_attention_host_kv_workspace_bytes -- device workspace of
 * h3a_attention_host_kv.  Returns 0 when none is needed or the arguments are
 * invalid.
 */
size_t h3a_attention_host_kv_workspace_bytes(int64_t s_q, int64_t s_kv, int32_t n_heads, int32_t head_dim,
                                             int64_t q_chunk, int64_t kv_block, int32_t mode);

/*
 * h3a_attention_host_kv -- h3a_attention (dense, no tile_mask) with the K/V
 * store in pinned host memory, brought to the GPU one kv_block at a time
 * [P1 Inputs table, kv_block row: K/V attended in blocks with a log-sum-exp
 * combine, kept for a host-staged K/V store].
 *
 * For every query chunk, the store is copied block by block (kv_block tokens,
 * 0 = 16384) into one of two device buffers in the workspace, on a copy
 * stream of the library's own, while the previous block is attended on
 * `stream`.  Each block's launch resumes every query row's running max, row
 * sum and output accumulators from the workspace and leaves them there for
 * the next block; the last block writes the output.  The output is bitwise the
 * one h3a_attention gives for the same store resident on the GPU.
 *
 * k_host, v_host, scales_host: the store of `mode` (as for h3a_attention) in
 *              PINNED host memory (hipHostMalloc), 16-byte aligned; pageable
 *              memory is H3A_EINVAL.  Must stay valid and unchanged until the
 *              work queued on `stream` has finished.
 * mode:        a store kind as for h3a_attention, optionally OR-ed with
 *              H3A_OUT_F16 (kvi8r stores; no H3A_SOL: dense only).
 * q, out:      device memory, as for h3a_attention.
 * workspace:   h3a_attention_host_kv_workspace_bytes(...) bytes of device
 *              memory (two K/V blocks, one query chunk's state).
 * The copy stream waits for the work queued on `stream` before the call, and
 * `stream` waits for every copy it uses, so the call is ordered on `stream`
 * like any other.
 */
int32_t h3a_attention_host_kv(const void* q, const void* k_host, const void* v_host, const void* scales_host,
                              int64_t s_q, int64_t s_kv, int32_t n_heads, int32_t head_dim, float softmax_scale,
                              int64_t q_chunk, int64_t kv_block, int32_t mode, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * h3a_rotate_rows -- y = fp16(x H) for n_rows rows of 128 bf16 values (the
 * query rotation of the kvi8r mode [P1 kv_store]; the same kernel that
 * h3a_attention runs).  x bf16 [n_rows, 128], y fp16 [n_rows, 128], both
 * 16-byte aligned.
 */
int32_t h3a_rotate_rows(const void* x_bf16, void* y_f16, int64_t n_rows, void* stream);

/*
 * h3a_unrotate_rows -- y = bf16(x H^T) for n_rows rows of 128 fp32 values (the
 * single output un-rotation of the kvi8r mode [P2, rotation paragraph]; the
 * same kernel that h3a_attention runs).  x fp32 [n_rows, 128], y bf16
 * [n_rows, 128], both 16-byte aligned.
 */
int32_t h3a_unrotate_rows(const float* x_f32, void* y_bf16, int64_t n_rows, void* stream);

/*
 * Kernel timing for measurement.  While enabled, the attention entry points
 * bracket every launch of their attention kernel, and of the query rotation and
 * output un-rotation of the kvi8r stores, and the store-build entry points
 * (h3a_kv_quantize, h3a_kv_quantize_g32, h3a_kv_quantize_pair) their launch,
 * with a pair of HIP events recorded on the call's stream.
 * h3a_timing_collect_kernel(kind, ...) waits for the events recorded for that
 * kernel kind, returns their summed time (ms) and the number of launches since
 * the last collect of that kind, and clears that record; an unknown kind
 * returns H3A_EINVAL.  h3a_timing_collect is the attention kind.  Disabled by
 * default.
 */
#define H3A_TIMING_ATTENTION 0
#define H3A_TIMING_ROTATE_Q 1
#define H3A_TIMING_UNROTATE_O 2
#define H3A_TIMING_KV_QUANTIZE 3
int32_t h3a_timing_enable(int32_t on);
int32_t h3a_timing_collect(double* attn_ms, int64_t* attn_launches);
int32_t h3a_timing_collect_kernel(int32_t kind, double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* H3A_H */
