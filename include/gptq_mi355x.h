/*
 * gptq_mi355x.h -- C ABI of the GPTQ one-shot layer quantizer for MI355X
 * (gfx950).
 *
 * The library computes the three stages of the GPTQ layer path:
 *   1. H (+)= 2 X^T X              gptq_hessian_accumulate
 *   2. U = chol((H + lambda I)^-1)  gptq_prepare_hinv     (upper factor)
 *   3. the fixed-order column sweep with OBS compensation, lazy blocks,
 *      per-group min-max scale/zero and packed b-bit codes
 *                                   gptq_quantize_layer (+ gptq_pack_codes)
 *
 * Conventions shared by every entry point
 *   - Pointers named as device pointers refer to GPU memory the caller
 *     allocated (for instance with torch). The library never allocates,
 *     frees or retains caller memory.
 *   - Process-wide state (created on first use, kept until the process
 *     ends, never freed): gptq_prepare_hinv keeps, per device, two
 *     auxiliary streams (default priority) and a small set of events for its
 *     look-ahead, and serializes its own enqueueing with a host mutex, so
 *     concurrent factor calls on different streams share those auxiliary
 *     streams and their device work overlaps less; while a caller captures a
 *     factor call into a graph, no other thread may call gptq_prepare_hinv
 *     on that device (the shared auxiliary streams are then part of the
 *     capture). gptq_quantize_layer_noalloc uses one static scratch array
 *     per device (see there). The packed product caches the occupancy per
 *     kernel, taken on the first device it runs on. Nothing else is kept
 *     between calls.
 *   - All matrices are row-major and contiguous unless a leading dimension
 *     is given.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on that stream and returns; nothing is
 *     synchronized. Results are valid once the stream has reached them.
 *   - Argument errors are reported synchronously, before anything is
 *     enqueued, as a gptq_status. A failed kernel launch returns
 *     GPTQ_E_HIP. Numerical breakdown of the factorization is reported on
 *     the device through `info`.
 *   - `ws`/`ws_bytes`: device scratch the caller provides, at least the size
 *     the matching *_workspace_size function returns; its contents on entry
 *     do not matter and on exit are unspecified. Two calls that may run at
 *     the same time need separate workspaces.
 *   - Sizes are int64_t; a size of 0 is allowed where stated and then does
 *     nothing.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_E_INVALID_ARG = 1, /* a size, pointer or parameter is out of range   */
  GPTQ_E_UNSUPPORTED = 2, /* valid for the method but not implemented here  */
  GPTQ_E_WORKSPACE = 3,   /* ws_bytes smaller than the required size         */
  GPTQ_E_HIP = 4,         /* a HIP launch or runtime call failed             */
  GPTQ_E_TOO_LARGE = 5    /* beyond the static scratch of the allocation-free
                             entry point                                     */
} gptq_status;

/* Largest layer gptq_quantize_layer_noalloc takes: d_row * d_col weights
   and d_row rows (its static scratch holds an fp32 working copy of W). */
#define GPTQ_NOALLOC_MAX_WEIGHTS (1 << 24)
#define GPTQ_NOALLOC_MAX_ROWS 65536

typedef enum { GPTQ_F16 = 0, GPTQ_F32 = 1 } gptq_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char* gptq_status_string(int status);

/* Library version as "major.minor.patch" (static storage). */
const char* gptq_version(void);

/* ------------------------------------------------------------------------
 * Stage 1 -- Hessian of the layer objective.
 *
 * Defines: H = 2 * sum over tokens t of x_t x_t^T (aiqz.cc "GPTQ：一键量化
 * 大模型压缩", section 二阶信息; compassingai.com "GPTQ", section 3, H = 2XX^T
 * with samples as columns). Here X holds one token per row, so H = 2 X^T X.
 *
 *   X          device, n_tokens x d, element type xdtype (GPTQ_F16 or
 *              GPTQ_F32), row stride ldx >= d elements.
 *   H          device fp32 d x d; both triangles are written.
 *   accumulate 0: H = 2 X^T X.  1: H += 2 X^T X (calibration in chunks).
 * The products of fp16 inputs are exact in fp32; partial sums are fp32
 * and are combined in a fixed order, so the result is deterministic.
 * n_tokens = 0 writes zeros (accumulate = 0) or leaves H unchanged.
 * Errors: d < 1, n_tokens < 0, ldx < d, NULL X (with n_tokens > 0) or H,
 * unknown dtype -> GPTQ_E_INVALID_ARG.
 * ---------------------------------------------------------------------- */
size_t gptq_hessian_workspace_size(int64_t n_tokens, int64_t d, int xdtype);
int gptq_hessian_accumulate(const void* X, int xdtype, int64_t n_tokens, int64_t d, int64_t ldx,
                            float* H, int accumulate, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 2 -- the rows of the inverse Hessian that the sweep uses.
 *
 * Defines: with mild damping, a Cholesky factorization precomputes the
 * needed rows of H^-1 (astro-blog LLM quantization survey, section 2.3
 * item 3; xuzou.cn reading card of the GPTQ paper, section 方法适配).
 * Computes lambda = damp * mean(diag H) (damp is the relative fraction),
 * H_d = H + lambda I, and U: upper triangular with positive diagonal and
 * H_d^-1 = U^T U. Row q of U, times U_qq, is row q of the inverse of the
 * trailing sub-Hessian H_d[q:, q:].
 *
 *   H          device fp32 d x d, symmetric (only the lower triangle is
 *              read); not modified.
 *   U          device fp32 d x d; the strictly lower triangle is zeroed.
 *   lambda_out device fp32 scalar, may be NULL.
 *   info       device int32 scalar: 0 on success; k > 0 if H_d is not
 *              numerically positive definite, k - 1 being the column (in H's
 *              indexing) where the factorization broke down. U is then
 *              unspecified.
 * The factorization runs in fp64 on the device. Part of its work runs on
 * per-device auxiliary streams that are forked from and joined back to
 * `stream` by events within the call, so the call keeps the usual stream
 * semantics and can be captured into a HIP graph. Errors: d < 1, NULL H, U
 * or info, damp < 0 or not finite -> GPTQ_E_INVALID_ARG.
 * ---------------------------------------------------------------------- */
size_t gptq_prepare_hinv_workspace_size(int64_t d);
int gptq_prepare_hinv(const float* H, int64_t d, double damp, float* U, float* lambda_out,
                      int32_t* info, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 3 -- fixed-order GPTQ column sweep.
 *
 * Defines: columns in natural order, shared by all rows; each rounded
 * column's error is spread over the row's remaining columns through the
 * inverse Hessian (aiqz.cc, section 误差补偿; astro-blog survey, sections
 * 2.2-2.3); blocks of `block` columns whose update of later columns is
 * deferred to the end of the block (xuzou.cn, section 方法适配);
 * per-group asymmetric min-max scale and zero (aiqz.cc, section 分组方案;
 * astro-blog survey, section 1.2); codes packed into 32-bit words
 * (mcipr.com "一文读懂GPTQ", section 三). For every row and column q:
 *   at a group start: xmin = min(0, min of the group's current values),
 *     xmax = max(0, ...) ([-1, 1] if both are 0); s = (xmax - xmin)/maxq,
 *     z = rint(-xmin / s); group_size = -1 takes one group per row from
 *     the original row.
 *   code = clamp(rint(w_q / s) + z, 0, maxq), what = s (code - z),
 *   err = w_q - what, e = err / U_qq, w_j -= e U_qj for j > q,
 *   loss += err^2 / (2 U_qq^2)            (maxq = 2^bits - 1)
 * Arithmetic is fp32 (code decisions included) with the loss in fp64.
 *
 *   W          device, d_row x d_col, wdtype GPTQ_F16 or GPTQ_F32; read only.
 *   U          device fp32 d_col x d_col from gptq_prepare_hinv (only the
 *              upper triangle is read).
 *   bits       2, 3, 4 or 8.
 *   group_size -1, or a multiple of 16 with block % group_size == 0 or
 *              group_size % block == 0.
 *   block      the lazy-batch width B (xuzou.cn, section 方法适配: updates
 *              of later columns wait until a block of B columns is done):
 *              a power of two up to 128, or a multiple of 128 up to 1024;
 *              other widths -> UNSUPPORTED. Lazy batches are exact, and the
 *              kernels apply every element's fp32 updates in the same order
 *              for every width, so all widths give the same outputs to the
 *              bit; 128 is the fastest (it is the kernels' own block).
 *   symmetric  0: the min-max grid above. 1: the symmetric grid (astro-blog
 *              survey, section 1.2: z = 0, signed values clamped to
 *              [-2^(bits-1), 2^(bits-1) - 1]; aiqz.cc demo scale): s =
 *              max|x| / (2^(bits-1) - 1) over the group (max|x| = 1 for an
 *              all-zero group), stored as code = signed + 2^(bits-1), so
 *              zeros holds 2^(bits-1). Other values -> INVALID_ARG.
 *   codes      device uint8 d_row x d_col (code per weight).
 *   scales     device fp32 d_row x n_groups, zeros device int32 d_row x
 *              n_groups, n_groups = 1 if group_size == -1 else
 *              ceil(d_col / group_size).
 *   packed     device uint32 d_row x ceil(d_col * bits / 32): per row an
 *              LSB-first bitstream, code j in bits [bits j, bits j + bits),
 *              zero padded.
 *   loss       device fp64 scalar (sum over rows and columns).
 *   row_loss   device fp32 d_row, may be NULL.
 * Errors: sizes < 1, NULL outputs (row_loss excepted), bad bits or group,
 * block < 1 -> GPTQ_E_INVALID_ARG; a block width outside the set above, or
 * a group that is not a multiple of 16 -> GPTQ_E_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
size_t gptq_quantize_layer_workspace_size(int64_t d_row, int64_t d_col, int bits,
                                          int64_t group_size, int64_t block);
int gptq_quantize_layer(const void* W, int wdtype, int64_t d_row, int64_t d_col, const float* U,
                        int bits, int64_t group_size, int64_t block, int symmetric,
                        uint8_t* codes, float* scales, int32_t* zeros, uint32_t* packed,
                        double* loss, float* row_loss, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 3 without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 *
 * Same operation, arguments, outputs and kernels as gptq_quantize_layer,
 * minus ws/ws_bytes: the fp32 working copy of W and the loss partials live
 * in one static device array of the library (64 MiB + 64 KiB), which each
 * GPU the library runs on holds from the library's load until the process
 * ends. The call allocates nothing (no hipMalloc, no allocating library
 * routine); it takes the array's device address once per device with
 * hipGetSymbolAddress. Nothing in the array needs clearing between calls.
 *   Limits: d_row * d_col <= GPTQ_NOALLOC_MAX_WEIGHTS and d_row <=
 *   GPTQ_NOALLOC_MAX_ROWS, else GPTQ_E_TOO_LARGE (checked before anything
 *   is enqueued).
 *   stream     must belong to the current device (else GPTQ_E_INVALID_ARG).
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (other streams, other threads) race and give undefined results;
 * serialize them, or use gptq_quantize_layer with separate workspaces.
 * Errors: as gptq_quantize_layer, plus GPTQ_E_TOO_LARGE.
 * ---------------------------------------------------------------------- */
int gptq_quantize_layer_noalloc(const void* W, int wdtype, int64_t d_row, int64_t d_col,
                                const float* U, int bits, int64_t group_size, int64_t block,
                                int symmetric, uint8_t* codes, float* scales, int32_t* zeros,
                                uint32_t* packed, double* loss, float* row_loss, void* stream);

/* ------------------------------------------------------------------------
 * Dequantize the packed layer (for running the quantized layer, e.g. to
 * propagate calibration activations to the next layer).
 *
 * Defines: astro-blog survey, section 1.2 (dequantization s (x_q - z));
 * xuzou.cn reading card, section 计算设置 (the quantized block is run to
 * produce the next block's inputs).
 *   out[r][c] = s[r][g(c)] * (code[r][c] - zeros[r][g(c)]), the product in
 *   fp32, then rounded to nearest even in the output type.
 *   packed, scales, zeros   as for gptq_quantize_layer.
 *   group_size -1 or >= 1; out_dtype GPTQ_F16 or GPTQ_F32; out device,
 *   d_row x d_col, row stride ld_out >= d_col.
 * Runs on `stream`; nothing is allocated. Errors: sizes < 1, NULL pointers,
 * ld_out < d_col, bad bits, group or dtype -> GPTQ_E_INVALID_ARG.
 * ---------------------------------------------------------------------- */
int gptq_dequantize(const uint32_t* packed, const float* scales, const int32_t* zeros, int64_t d_row,
                    int64_t d_col, int bits, int64_t group_size, void* out, int out_dtype, int64_t ld_out,
                    void* stream);

/* ------------------------------------------------------------------------
 * Running the quantized layer on token batches (the calibration pipeline's
 * propagation to the next layer).
 *
 * Defines: xuzou.cn reading card of the GPTQ paper, section 计算设置 (each
 * quantized block is run on the calibration tokens to give the next block's
 * inputs) and section 方法适配, last paragraph (the quantized matrix is used
 * with dequantization on the fly); What = s (code - z) per group (astro-blog
 * survey, section 1.2), held as fp16 to run. For t < n_tokens, r < d_out:
 *   Y[t][r] = act(sum_c X[t][c] * W16[r][c]),
 *   W16[r][c] = fp16(fp32(scales[r][g(c)] * (code[r][c] - zeros[r][g(c)]))),
 * act = ReLU when relu = 1 (identity when 0), Y rounded to fp16 (nearest
 * even). The products of fp16 values are exact in fp32 and the sums are
 * fp32, on the fp16 MFMA (the weights are dequantized inside the kernel,
 * never written out).
 *   packed, scales, zeros   as for gptq_quantize_layer (d_out rows, d_in
 *              columns; bits 2, 3, 4 or 8).
 *   X          device fp16, n_tokens rows of d_in values, row stride ldx.
 *   Y          device fp16, n_tokens x d_out, row stride ldy >= d_out.
 *   ws         device workspace of gptq_dequant_gemm_workspace_size(d_out,
 *              d_in, n_tokens) bytes, or NULL. With a workspace and d_in a
 *              multiple of 128, the weights are dequantized once into it
 *              (K-major fp16, the same values) and X is copied K-major beside
 *              them; the product then runs on both from there (the form for
 *              large token batches). Without one, or for other d_in, the
 *              weights are dequantized inside the product kernel per token
 *              tile. Both use the same fp16 weights; their fp32 sums run in
 *              different orders inside each 16-K MFMA step.
 * Runs on `stream`; nothing is allocated; n_tokens = 0 does nothing.
 * Errors: sizes < 1, NULL pointers, ldx < d_in, ldy < d_out, bad bits,
 * group_size 0 or < -1, relu not 0 or 1 -> GPTQ_E_INVALID_ARG; d_in not a
 * multiple of 32, group_size not -1 or a multiple of 64, X not 16-byte
 * aligned or ldx not a multiple of 8 -> GPTQ_E_UNSUPPORTED; ws given with
 * ws_bytes below the size query -> GPTQ_E_WORKSPACE.
 * ---------------------------------------------------------------------- */
int gptq_dequant_gemm(const uint32_t* packed, const float* scales, const int32_t* zeros, int64_t d_out,
                      int64_t d_in, int bits, int64_t group_size, const void* X, int64_t n_tokens,
                      int64_t ldx, void* Y, int64_t ldy, int relu, void* ws, size_t ws_bytes, void* stream);
size_t gptq_dequant_gemm_workspace_size(int64_t d_out, int64_t d_in, int64_t n_tokens);

/* ------------------------------------------------------------------------
 * Column order: act-order permutation.
 *
 * Defines: mcipr.com "一文读懂GPTQ", section 四 (the desc_act flag of the
 * method's library configuration; the page gives no formula). Reading: the
 * columns are quantized in order of descending diag(H); equal values keep
 * ascending column order, NaN values come last, -0 equals +0. The layer is
 * then the fixed-order method on W[:, perm] with H[perm][:, perm] (gather
 * both with gptq_gather, then gptq_prepare_hinv and gptq_quantize_layer);
 * groups are consecutive in the permuted order, so group k of the outputs
 * covers the original columns perm[k g .. k g + g - 1].
 *   H        device fp32, d x d, row stride ldh >= d; only the diagonal is read.
 *   perm     device int32 [d]: perm[q] = original column quantized q-th.
 *   invperm  device int32 [d]: invperm[perm[q]] = q (also the rank buffer).
 * Runs on `stream`; nothing is allocated. Errors: d < 1, d > 65535 * 256, ldh < d,
 * NULL pointers -> GPTQ_E_INVALID_ARG.
 * ---------------------------------------------------------------------- */
int gptq_act_order_perm(const float* H, int64_t d, int64_t ldh, int32_t* perm, int32_t* invperm,
                        void* stream);

/* ------------------------------------------------------------------------
 * Row and column gather (moves a layer into or out of a column order).
 *
 * Defines: the permuted layer of the act-order reading above (mcipr.com
 * "一文读懂GPTQ", section 四): W[:, perm], H[perm][:, perm], the codes back
 * in original order (codes_p[:, invperm]) and activations in the permuted
 * order (x[:, perm]) for the packed product.
 *   dst[i][q] = src[row_idx[i]][col_idx[q]], i < rows, q < cols; a NULL
 *   index array means the identity.
 *   src      device, src_rows x src_cols elements of elem_bytes (1, 2 or 4)
 *            bytes, row stride ld_src >= src_cols (elements).
 *   dst      device, rows x cols, row stride ld_dst >= cols; must not
 *            overlap src.
 *   info     device int32 or NULL: set to 0, then to 1 if any index lies
 *            outside the source; such elements are written as 0.
 * Runs on `stream`; nothing is allocated. Errors: sizes < 1, NULL src or
 * dst, ld_src < src_cols, ld_dst < cols, elem_bytes not 1, 2 or 4 ->
 * GPTQ_E_INVALID_ARG.
 * ---------------------------------------------------------------------- */
int gptq_gather(const void* src, int elem_bytes, int64_t src_rows, int64_t src_cols, int64_t ld_src,
                const int32_t* row_idx, int64_t rows, const int32_t* col_idx, int64_t cols, void* dst,
                int64_t ld_dst, int32_t* info, void* stream);

/* ------------------------------------------------------------------------
 * Use of the packed layer: quantized matrix x full-precision vectors.
 *
 * Defines: xuzou.cn reading card of the GPTQ paper, section 方法适配 (last
 * paragraph) and section 瓶颈: the inference kernel multiplies the
 * quantized matrix by full-precision activation vectors and dequantizes the
 * weights on the fly, so that batch-1 generation reads the low-bit words.
 * Dequantization What = s (code - z) per group (astro-blog survey, section
 * 1.2). For b < batch, r < d_row:
 *   y[b][r] = sum_c x[b][c] * scales[r][g(c)] * (code[r][c] - zeros[r][g(c)])
 * with code[r][c] read from `packed` (layout of gptq_quantize_layer) and
 * g(c) = c / group_size (0 if group_size == -1).
 *   packed     device uint32 d_row x ceil(d_col * bits / 32).
 *   scales     device fp32, zeros device int32, d_row x n_groups.
 *   bits       2, 3, 4 or 8.
 *   group_size -1, or a multiple of 8.
 *   x          device fp16, batch rows of d_col values, row stride ldx >= d_col.
 *   y          device fp32, batch x d_row, row-major.
 * fp32 accumulation of exact codes times fp16 activations; the per-row sum
 * has a fixed order, so results are deterministic. When group_size is -1 or
 * a multiple of 32 and x rows are 16-byte aligned (ldx % 8 == 0, x 16-byte
 * aligned), a faster kernel runs (two codes per instruction, several rows
 * per wave); with 3 or more vectors, d_col a multiple of 128 and groups of
 * 128-column multiples (or -1), up to 16 vectors go through fp16 MFMAs per
 * pass; other layouts take a per-code kernel. Runs on `stream` (NULL: the
 * default stream); nothing is allocated. Errors: sizes < 1, NULL pointers,
 * ldx < d_col, bad bits or group -> GPTQ_E_INVALID_ARG; a failed launch or
 * device query -> GPTQ_E_HIP.
 * ---------------------------------------------------------------------- */
int gptq_dequant_matvec(const uint32_t* packed, const float* scales, const int32_t* zeros,
                        int64_t d_row, int64_t d_col, int bits, int64_t group_size, const void* x,
                        int64_t batch, int64_t ldx, float* y, void* stream);

/* ------------------------------------------------------------------------
 * Packing of existing codes (the same device routine the sweep uses).
 *
 * Defines: b-bit codes stored in 32-bit integer arrays (mcipr.com
 * "一文读懂GPTQ", section 三); layout as for `packed` above. Codes are
 * masked to their low `bits` bits.
 *   codes  device uint8 d_row x d_col;  packed device uint32 d_row x
 *   ceil(d_col * bits / 32).
 * Errors: sizes < 1, NULL pointers, bits not in {2,3,4,8}
 * -> GPTQ_E_INVALID_ARG.
 * ---------------------------------------------------------------------- */
int gptq_pack_codes(const uint8_t* codes, int64_t d_row, int64_t d_col, int bits,
                    uint32_t* packed, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
