/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 W4A4 library, libnvfp4.so.
 *
 * The format ("LongLive-2.0: An NVFP4 Parallel Infrastructure for Long Video
 * Generation", architecture walkthrough page, section "NVFP4 Training",
 * paragraphs "NVFP4 numeric format", "Hierarchical scaling" and
 * "Quantization rule for a tensor block"):
 *
 *     Xhat = X_FP4 * alpha_FP8 * alpha_FP32
 *
 * X_FP4 is a 4-bit E2M1 code per element (values 0, +-0.5, +-1, +-1.5, +-2,
 * +-3, +-4, +-6), alpha_FP8 an E4M3 scale shared by a block of 16 elements
 * (or a 16x16 tile for weights, "NVFP4 training recipe"), alpha_FP32 one
 * float per tensor.  The block scale maps the block max to 6, or -- rule
 * NVFP4_RULE_4OVER6, the pages' "Four Over Six" scale search of section
 * "NVFP4 Inference" -- to 4 when that reconstructs the block with a smaller
 * squared error.
 *
 * Exact arithmetic of every step (fp32 evaluation order, rounding, ties,
 * saturation) is fixed by this library as follows; the pages state the rule
 * in real numbers only:
 *   alpha   = amax / 2688 in fp32 (2688 = 448 * 6); alpha = 1 if amax == 0
 *   mu      = m / alpha, m the block's max |x|
 *   s_c     = E4M3(mu / c), c in {6, 4}: nearest, ties to even, subnormals
 *             kept, saturating at 448
 *   code    = E2M1(x * (1 / (s_c * alpha))): nearest, ties to even,
 *             saturating at 6, sign of x kept (-0.0 -> code 0x8); s_c == 0
 *             gives +-0 codes
 *   xhat    = (q * s) * alpha                    (two fp32 multiplies)
 *   error_c = per block row, fma chain e = fma(d, d, e) over the row's 16
 *             elements in index order, d = fma(-(q * s), alpha, x) (the
 *             exact residual, rounded once); rows added in order;
 *             4 is chosen only if error_4 < error_6.
 *
 * Layouts (row-major, element 2j in the LOW nibble of byte j, scales are
 * E4M3FN bytes):
 *   NVFP4_ROW16  x [rows][cols], blocks of 16 along cols (activations,
 *                gradients, KV).  codes [rows][cols/2], scales [rows][cols/16].
 *   NVFP4_TILE16 x [rows][cols], 16x16 tiles (weights).
 *                codes [rows][cols/2], scales [rows/16][cols/16].
 *   NVFP4_COL16  x [rows][cols], blocks of 16 along ROWS (the contraction
 *                dimension of the weight-gradient GEMM); stored transposed so
 *                that dimension is contiguous: codes [cols][rows/2], scales
 *                [cols][rows/16].  This is exactly the ROW16 packing of x^T.
 *   alpha        one float (device memory).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates or frees device memory and keeps no state
 *     between calls, except the static scratch array of
 *     nvfp4_linear_no_alloc (see there).  Work is enqueued on `stream`
 *     (0 = null stream) and is asynchronous; buffers must stay alive until
 *     the stream reaches it.
 *   - Inputs must not alias outputs or the workspace.
 *   - Arguments are validated before anything is enqueued; on any error
 *     nothing is enqueued and outputs are untouched.  Launch failures are
 *     reported as NVFP4_ERR_LAUNCH.  No C++ exception crosses the ABI.
 *   - Alignment: codes, scales and workspaces 16-byte aligned.  Inputs read
 *     and outputs written in 16-byte vectors (ROW16/TILE16 quantize input,
 *     ROW16/TILE16 dequantize output, nvfp4_linear's x) need a 16-byte
 *     aligned pointer and a leading dimension that is a multiple of 8
 *     elements; every other tensor (COL16 input, GEMM output, ...) only
 *     needs element alignment.  Leading dimensions are >= the row length.
 *   - Sizes: every dimension below 2^31.  Entry points that run the GEMM
 *     (nvfp4_gemm, nvfp4_linear, nvfp4_linear_lora, nvfp4_wgrad and the
 *     DGRAD use of nvfp4_linear) also need each packed operand below 4 GiB
 *     (rows * k / 2 < 2^32 for both A and B) and fewer than 2^23 output
 *     tiles of 128 x 128 (about 2^37 output elements).  The quantize,
 *     dequantize, transpose and smoothed-key entry points launch one lane
 *     per 16-element block and a dispatch counts lanes in 32 bits: at most
 *     2^36 - 2^20 elements per call.  Larger calls return NVFP4_ERR_SHAPE.
 *   - Numeric contract: inputs finite and amax == 0 or amax >= 2^-96;
 *     otherwise results are unspecified, but no call faults.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 1

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
    NVFP4_ERR_SHAPE = 2,       /* a size is negative, too large or not a multiple of 16 where required */
    NVFP4_ERR_ALIGN = 3,       /* pointer or leading dimension misaligned */
    NVFP4_ERR_DTYPE = 4,       /* unknown dtype / block / rule enum value */
    NVFP4_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
    NVFP4_ERR_LAUNCH = 6,      /* a kernel launch failed (hipGetLastError) */
    NVFP4_ERR_SCRATCH = 7      /* nvfp4_linear_no_alloc: the call needs more than
                                  NVFP4_NO_ALLOC_SCRATCH_BYTES of scratch */
} nvfp4_status_t;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype_t;
typedef enum { NVFP4_RULE_STATIC6 = 0, NVFP4_RULE_4OVER6 = 1 } nvfp4_rule_t;
typedef enum { NVFP4_ROW16 = 0, NVFP4_TILE16 = 1, NVFP4_COL16 = 2 } nvfp4_block_t;

/* Scale layout of a packed GEMM operand (see nvfp4_gemm). */
typedef enum { NVFP4_SCALE_1D = 0, NVFP4_SCALE_2D = 1 } nvfp4_scale_layout_t;

int nvfp4_abi_version(void);
const char *nvfp4_status_string(nvfp4_status_t status);

/* Bytes of workspace nvfp4_quantize / nvfp4_kv_quantize need (amax partial
 * maxima).  Never more than 4 KiB (currently 1 KiB). */
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols);

/* The same figure under the name of the scope table's helper list: the
 * workspace of one single-tensor quantize call (nvfp4_quantize,
 * nvfp4_kv_quantize).  The fused and chunked calls have their own size
 * helpers. */
size_t nvfp4_workspace_size(int64_t rows, int64_t cols);

/*
 * nvfp4_quantize -- quantize x [rows][cols] (row stride ldx elements,
 * dtype NVFP4_F32 or NVFP4_BF16) into NVFP4.
 *   block  NVFP4_ROW16 (cols % 16 == 0), NVFP4_TILE16 (rows, cols % 16 == 0)
 *          or NVFP4_COL16 (rows % 16 == 0).
 *   rule   NVFP4_RULE_STATIC6 (block max -> 6) or NVFP4_RULE_4OVER6.
 *   amax   NULL: the tensor's max |x| is computed on the device (one extra
 *          read of x).  Otherwise a device pointer to a precomputed amax
 *          (e.g. the same tensor's max used for another packing of it).
 *   codes, scales, alpha: outputs as in the layout table above.
 *   workspace: >= nvfp4_quantize_workspace_size(rows, cols) bytes (unused
 *          when amax != NULL, may then be NULL).
 * Source of the operation: "Hierarchical scaling" and "Quantization rule for a
 * tensor block" (NVFP4 Training section) and "Scale-search mechanism" (NVFP4
 * Inference section) of the architecture walkthrough page.
 */
nvfp4_status_t nvfp4_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                              int block, int rule, const float *amax,
                              uint8_t *codes, uint8_t *scales, float *alpha,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_dequantize -- y = (q * s) * alpha for a tensor packed by
 * nvfp4_quantize with the same (rows, cols, block).  y is [rows][cols] in the
 * ORIGINAL orientation (also for COL16), row stride ldy, dtype NVFP4_F32 or
 * NVFP4_BF16 (bf16 = round-to-nearest-even of the fp32 value).
 * Source: the "Hierarchical scaling" equation.
 */
nvfp4_status_t nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *alpha,
                                int64_t rows, int64_t cols, int block,
                                void *y, int y_dtype, int64_t ldy, hipStream_t stream);

/*
 * nvfp4_gemm -- C[m][n] = alpha_A * alpha_B * sum_k Ahat[m][k] * Bhat[n][k]
 * (both operands K-contiguous, "NT"), fp32 accumulation, fp32 or bf16 out.
 *   A: codes [m][k/2], scales 1D [m][k/16] or 2D [m/16][k/16], alpha.
 *   B: codes [n][k/2], scales 1D [n][k/16] or 2D [n/16][k/16], alpha.
 *   A ROW16 or TILE16 tensor of shape [r][k] is an operand as is; a COL16
 *   tensor of x [k][r] is the operand x^T [r][k] with 1D scales.
 *   k % 16 == 0; 2D scales need the operand's row count % 16 == 0.
 *   C [m][n], row stride ldc, dtype NVFP4_F32 or NVFP4_BF16.
 *   c_amax (optional, device, 4-byte aligned): receives max |C| over the
 *   stored values (after bf16 rounding for bf16 output) -- the amax a
 *   following nvfp4_quantize / nvfp4_kv_quantize of C needs, so that call
 *   can skip its own amax pass.  NULL: not computed.
 * The dequantized operands q*s are exact in fp16, so the contraction runs on
 * fp16 MFMA with fp32 accumulation; accumulation order is unspecified.
 * Source: "The three GEMMs of backpropagation" and "Quantization-
 * dequantization flow" (NVFP4 Training section).
 */
nvfp4_status_t nvfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                          int a_scale_layout,
                          const uint8_t *b_codes, const uint8_t *b_scales, const float *b_alpha,
                          int b_scale_layout,
                          int64_t m, int64_t n, int64_t k,
                          void *c, int c_dtype, int64_t ldc, float *c_amax, hipStream_t stream);

/*
 * nvfp4_kv_quantize -- quantize one K or V cache tensor of `vectors` rows of
 * head_dim elements (any leading-dimension order, e.g. [heads][tokens] or
 * [tokens][heads], contiguous, so vectors = heads * tokens), 16-element
 * blocks along head_dim, one alpha for the whole tensor.  Equivalent to
 * nvfp4_quantize(kv, dtype, vectors, head_dim, head_dim, NVFP4_ROW16, rule,
 * amax, ...).  head_dim % 16 == 0.  amax: NULL (computed, one extra read of
 * the tensor) or a device pointer to the tensor's max |x|, e.g. the c_amax
 * output of the GEMM that produced K or V (single pass over the tensor).
 * Source: "KV cache quantization" / "Chunkwise quantization procedure"
 * (NVFP4 Inference section of the architecture walkthrough page).
 */
nvfp4_status_t nvfp4_kv_quantize(const void *kv, int kv_dtype, int64_t vectors, int64_t head_dim,
                                 int rule, const float *amax, uint8_t *codes, uint8_t *scales, float *alpha,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace of nvfp4_linear: the packed activation (m*k*9/16 bytes) plus the
 * amax partials, rounded up. */
size_t nvfp4_linear_workspace_size(int64_t m, int64_t k);

/*
 * nvfp4_linear -- the W4A4 forward GEMM with activation quantization fused
 * into the call: quantize x [m][k] (ROW16, `rule`, amax computed on the
 * device) into the workspace, then y = nvfp4_gemm(x_packed, w).
 *   w: packed weight [n][k] (TILE16 -> NVFP4_SCALE_2D, ROW16 -> _1D).
 *   y_amax: optional max |y| output, as c_amax of nvfp4_gemm.
 * Source: "Quantization-dequantization flow" (FPROP: weight x activation ->
 * BF16 output).
 */
nvfp4_status_t nvfp4_linear(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, int rule,
                            const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                            int w_scale_layout, int64_t n,
                            void *y, int y_dtype, int64_t ldy, float *y_amax,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_linear_no_alloc -- nvfp4_linear for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation, kernels and results, with
 * the workspace taken from a static device array inside the library instead
 * of a caller buffer.  The call itself allocates nothing (no hipMalloc, no
 * allocating library routine).
 *   Scratch: NVFP4_NO_ALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the
 *   first call on that GPU until the process ends; the call uses the copy of
 *   the CURRENT device (the stream must belong to it).  A call needing more,
 *   i.e. nvfp4_linear_workspace_size(m, k) > NVFP4_NO_ALLOC_SCRATCH_BYTES
 *   (about 119 M activation elements, e.g. 32768 x 3072 fits), returns
 *   NVFP4_ERR_SCRATCH and enqueues nothing.
 *   Every call on a GPU shares that GPU's scratch and leaves its contents
 *   there: calls that can overlap on one GPU (two streams, two host threads
 *   without ordering) RACE and must be serialized by the caller.
 *   The first call on a device looks the array's address up
 *   (hipGetSymbolAddress); a failure there returns NVFP4_ERR_LAUNCH.
 * Other arguments, checks and errors as nvfp4_linear.
 */
#define NVFP4_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)

nvfp4_status_t nvfp4_linear_no_alloc(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, int rule,
                                     const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                                     int w_scale_layout, int64_t n,
                                     void *y, int y_dtype, int64_t ldy, float *y_amax, hipStream_t stream);

/*
 * nvfp4_linear_lora -- the W4A4 linear with a BF16 LoRA branch:
 *     y = nvfp4_linear(x, w) + lora_scale * U B^T,   U = bf16(x A^T)
 * x [m][k] bf16 (ld ldx, 16-byte aligned rows), lora_a A [rank][k] and
 * lora_b B [n][rank] bf16 contiguous, rank in {32, 64, 96, 128}, lora_scale
 * the adapter scale (alpha / rank).  lora_u: caller buffer [m][rank] bf16
 * that receives U (x A^T with fp32 accumulation, rounded once to bf16, as a
 * bf16 linear layer computes it).  The rank-r update runs on bf16 MFMA in the
 * same GEMM launch after the NVFP4 contraction; fp32 accumulation.  Both bf16
 * products run on the matrix cores, which flush fp32 subnormal products and
 * partial sums (below 2^-126) to zero: rows of x that are themselves near
 * the bottom of the bf16 range get U within k * 2^-126 of the exact sum,
 * not its rounding.  Other
 * arguments as nvfp4_linear; workspace >= nvfp4_linear_lora_workspace_size().
 * Source: "LoRA parameterization" (W ~ Dequant(Q(W0)) + (alpha/r) B A, rank
 * 128, alpha 128, BF16 adapters) and the NVFP4 Inference section (the
 * adapters kept as a separate BF16 branch on the quantized backbone) of the
 * architecture walkthrough page.
 */
/* Workspace of nvfp4_linear_lora: nvfp4_linear's plus the partial sums of
 * the down projection (at most 8 * m * rank floats) and up to 1024 partial
 * maxima of |x| (the down projection reads all of x and leaves them for the
 * activation quantizer, which then needs no amax pass of its own). */
size_t nvfp4_linear_lora_workspace_size(int64_t m, int64_t k, int rank);

nvfp4_status_t nvfp4_linear_lora(const void *x, int64_t m, int64_t k, int64_t ldx, int rule,
                                 const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                                 int w_scale_layout, int64_t n, const void *lora_a, const void *lora_b, int rank,
                                 float lora_scale, void *lora_u, void *y, int y_dtype, int64_t ldy, float *y_amax,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace of nvfp4_wgrad: both COL16-packed operands plus amax partials. */
size_t nvfp4_wgrad_workspace_size(int64_t tokens, int64_t n_out, int64_t k_in);

/*
 * nvfp4_wgrad -- weight gradient dW[n][k] = sum_t dY[t][n] * X[t][k] with
 * both operands quantized in 16-blocks along the token axis (NVFP4_COL16,
 * `rule`).  dy [tokens][n_out] (ld lddy), x [tokens][k_in] (ld ldx), same
 * dtype; tokens % 16 == 0.  dW [n_out][k_in] (ld lddw), fp32 or bf16.
 * rht_signs: -1 quantizes dY and X as they are; 0..0xFFFF first applies the
 * random Hadamard transform with these signs to both, along the tokens (see
 * nvfp4_quantize_col16_rht), so dW is computed from R dY and R X.
 * dy_amax, x_amax (optional, device, 4-byte aligned): the operands' max |.|,
 * each replacing that operand's amax pass (one read of the operand fewer).
 * The COL16 packing of X shares its global scale with the forward's ROW16
 * packing of the same X (same amax): hand in the amax the forward used,
 * e.g. the y_amax / c_amax output of the GEMM that produced X, or of the one
 * that produced dY.  With the transform the amax must be that of R dY / R X.
 * NULL: computed on the device.
 * Source: "The three GEMMs of backpropagation" (WGRAD: activation x output
 * gradient -> weight gradient) with 1D gradient blocks along the reduction
 * dimension ("NVFP4 training recipe"), and "Random Hadamard Transform (RHT)
 * for gradient stabilization" for the optional transform.
 */
nvfp4_status_t nvfp4_wgrad(const void *dy, const void *x, int dtype, int64_t tokens, int64_t n_out,
                           int64_t k_in, int64_t lddy, int64_t ldx, int rule, int rht_signs,
                           const float *dy_amax, const float *x_amax,
                           void *dw, int dw_dtype, int64_t lddw,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_quantize_col16_rht -- NVFP4_COL16 quantization of R x, where R applies
 * the random Hadamard transform to every 16-row block of every column (the
 * COL16 blocks): R = (1/4) H16 D, H16 the Sylvester Hadamard matrix
 * (H[i][j] = (-1)^popcount(i & j)), D = diag(-1 where bit i of rht_signs is
 * set, else +1), rht_signs in [0, 0xFFFF].  fp32 order of the transform:
 * sign flips, butterfly stages h = 1, 2, 4, 8 mapping (v[i], v[i+h]) with
 * i & h == 0 to (v[i] + v[i+h], v[i] - v[i+h]), then * 0.25.  alpha and the
 * codes are those of the transformed tensor; amax NULL computes its max |R x|
 * (one extra read of x), else a device pointer to it.  Other arguments and
 * layouts as nvfp4_quantize with NVFP4_COL16.  R is orthogonal, so a GEMM of
 * two operands transformed with the same signs contracts to the product of
 * the untransformed ones (up to quantization).
 * Source: "Random Hadamard Transform (RHT) for gradient stabilization"
 * (NVFP4 Training section of the architecture walkthrough page): both WGRAD
 * operands are multiplied by one fixed random Hadamard matrix before
 * quantization.  Size 16, aligned with the quantization blocks, and the
 * construction above are this library's reading (the pages give neither).
 */
nvfp4_status_t nvfp4_quantize_col16_rht(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                        int rule, int rht_signs, const float *amax,
                                        uint8_t *codes, uint8_t *scales, float *alpha,
                                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_transpose_tile16 -- the packed transpose W^T of a tensor W [rows][cols]
 * quantized with NVFP4_TILE16 blocks: codes_t [cols][rows/2], scales_t
 * [cols/16][rows/16] (one byte per 16x16 tile, unchanged), alpha_t = alpha.
 * Exact: no value is re-quantized, so dequantize(W^T) is the transpose of
 * dequantize(W) bit for bit.  rows % 16 == 0, cols % 16 == 0; codes, scales
 * and their transposes 16-byte aligned, must not overlap.
 * Use: the DGRAD GEMM dX = dY W contracts W over its rows (the layer's output
 * features); with Wt = nvfp4_transpose_tile16(W) it is
 * nvfp4_linear(dY, ..., Wt, NVFP4_SCALE_2D, ...), the same weight quantization
 * that FPROP uses.
 * Source: "NVFP4 training recipe" (2D 16x16 weight blocks) and "The three
 * GEMMs of backpropagation" (DGRAD: weight x output gradient -> activation
 * gradient), NVFP4 Training section of the architecture walkthrough page.
 */
nvfp4_status_t nvfp4_transpose_tile16(const uint8_t *codes, const uint8_t *scales, const float *alpha,
                                      int64_t rows, int64_t cols, uint8_t *codes_t, uint8_t *scales_t,
                                      float *alpha_t, hipStream_t stream);

/* ---------------------------------------- KV cache, one scale per chunk */

/* Workspace of nvfp4_kv_quantize_chunked (amax partial maxima): 4 KiB per
 * (tensor, chunk) unit. */
size_t nvfp4_kv_chunked_workspace_size(int64_t tensors, int64_t heads, int64_t tokens, int64_t head_dim,
                                       int64_t tokens_per_chunk);

/*
 * nvfp4_kv_quantize_chunked -- the KV quantizer with one FP32 global scale
 * per CHUNK of tokens of each tensor, all chunks (and e.g. a layer's K and V
 * as two tensors) in one call: two launches, the amax partials of every
 * (tensor, chunk) unit and then the quantizer; one launch when chunk_amax is
 * given.
 *   kv [tensors][heads][tokens][head_dim] (contiguous, 16-byte aligned, fp32
 *   or bf16); chunk c of tensor u holds tokens [c * tokens_per_chunk,
 *   min((c + 1) * tokens_per_chunk, tokens)) of every head of u, n_chunks =
 *   ceil(tokens / tokens_per_chunk).  Each unit is quantized exactly as
 *   nvfp4_kv_quantize would quantize that chunk of that tensor alone
 *   (16-blocks along head_dim, `rule`).
 *   codes [tensors][heads][tokens][head_dim/2], scales
 *   [tensors][heads][tokens][head_dim/16]: the ROW16 packing of the
 *   [tensors * heads * tokens][head_dim] view.
 *   alphas [tensors][n_chunks] (fp32, device): each unit's global scale.
 *   chunk_amax: NULL (computed, one extra read of the input) or a device
 *   array [tensors][n_chunks] of the units' max |x|.
 *   0 <= tensors, 1 <= heads <= 1024, head_dim % 16 == 0 and >= 16,
 *   tokens_per_chunk >= 1, tensors * n_chunks <= 65535; tensors == 0 or
 *   tokens == 0 enqueues nothing.
 *   workspace >= nvfp4_kv_chunked_workspace_size() (unused with chunk_amax).
 * Source: "Chunkwise quantization procedure" (a per-chunk, per-layer FP32
 * global scale for the keys and values of each chunk) and "KV cache
 * quantization" (16-element blocks along the head dimension), NVFP4 Inference
 * section of the architecture walkthrough page; the paper-notes page gives
 * the chunk size (8 latent frames).
 */
nvfp4_status_t nvfp4_kv_quantize_chunked(const void *kv, int kv_dtype, int64_t tensors, int64_t heads,
                                         int64_t tokens, int64_t head_dim, int64_t tokens_per_chunk, int rule,
                                         const float *chunk_amax, uint8_t *codes, uint8_t *scales,
                                         float *alphas, void *workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * nvfp4_kv_dequantize_chunked -- y = (q * s) * alpha_(u,c) for an input packed
 * by nvfp4_kv_quantize_chunked with the same (tensors, heads, tokens,
 * head_dim, tokens_per_chunk): alpha_(u,c) the scale of the element's tensor
 * and chunk.  y [tensors][heads][tokens][head_dim], contiguous, 16-byte
 * aligned, fp32 or bf16 (round to nearest even).
 * Source: the "Hierarchical scaling" equation with the per-chunk scale.
 */
nvfp4_status_t nvfp4_kv_dequantize_chunked(const uint8_t *codes, const uint8_t *scales, const float *alphas,
                                           int64_t tensors, int64_t heads, int64_t tokens, int64_t head_dim,
                                           int64_t tokens_per_chunk, void *y, int y_dtype, hipStream_t stream);

/* ------------------------------------------------ KV cache, consumer side */

/* Workspace of nvfp4_kv_quantize_smoothed (amax partials), at most 4 KiB. */
size_t nvfp4_kv_smooth_workspace_size(int64_t vectors, int64_t head_dim);

/*
 * nvfp4_kv_quantize_smoothed -- key smoothing, then the KV quantizer: every
 * key vector (head_dim elements, a power of two in [16, 1024]) loses its mean
 * over head_dim, and the smoothed keys are quantized as nvfp4_kv_quantize
 * does (16-blocks along head_dim, one alpha for the tensor -- call it once
 * per chunk for the per-chunk global scale).  means [vectors] (fp32, device)
 * receives each vector's mean, which nvfp4_kv_dequantize_window adds back.
 * fp32 order: per 16-element block a partial sum in index order, the
 * partials added in block order, mean = sum / head_dim, key - mean.
 * k: [vectors][head_dim] contiguous, 16-byte aligned; workspace >=
 * nvfp4_kv_smooth_workspace_size().  vectors == 0 writes only alpha (1.0,
 * the zero-amax value).
 * Source: "Key smoothing" (subtract the mean over the head dimension from
 * each key vector) and "Chunkwise quantization procedure" (per-chunk,
 * per-layer global scale), NVFP4 Inference section of the architecture
 * walkthrough page.  Keeping the means for the add-back is this library's
 * reading: without it each key's scores with a query change by mean * sum(q).
 */
nvfp4_status_t nvfp4_kv_quantize_smoothed(const void *k, int k_dtype, int64_t vectors, int64_t head_dim, int rule,
                                          uint8_t *codes, uint8_t *scales, float *alpha, float *means,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/* One cached chunk's contribution to an attention window: rows
 * [first, first + count) of a chunk quantized by nvfp4_kv_quantize (means
 * NULL) or nvfp4_kv_quantize_smoothed (means = its means array).  codes
 * [chunk rows][head_dim/2], scales [chunk rows][head_dim/16], alpha: device
 * pointers as the quantizer wrote them (codes and scales 16-byte aligned). */
typedef struct {
    const uint8_t *codes;
    const uint8_t *scales;
    const float *alpha;
    const float *means;
    int64_t first;
    int64_t count;
} nvfp4_kv_segment_t;

#define NVFP4_MAX_KV_SEGMENTS 32

/*
 * nvfp4_kv_dequantize_window -- rebuild an attention window from cached
 * chunks in ONE launch: the segments' rows, dequantized ((q * s) * alpha,
 * plus the vector's mean for smoothed keys, one fp32 add), written one after
 * another into out [sum of counts][head_dim] (row stride ldo elements, fp32 or
 * bf16 = round-to-nearest-even, 16-byte aligned rows).  segments: a HOST
 * array of n_segments <= NVFP4_MAX_KV_SEGMENTS entries, read during the call
 * (it can be reused as soon as the call returns).  The caller plans the
 * segments: global sink, shot sink and the sliding window of recent chunks,
 * with overlapping frames listed once.
 * Source: "Parallel CUDA dequantization kernel" (chunks of the active window
 * reconstructed together into the window buffer in one launch) and the
 * effective key/value set (global sink, shot-level sink, sliding window,
 * duplicates removed) of the Multi-Shot Attention Sink section of the
 * architecture walkthrough page.
 */
nvfp4_status_t nvfp4_kv_dequantize_window(const nvfp4_kv_segment_t *segments, int n_segments, int64_t head_dim,
                                          void *out, int out_dtype, int64_t ldo, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
