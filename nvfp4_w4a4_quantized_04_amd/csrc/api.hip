// C ABI of libnvfp4.so: argument validation, workspace carving and launches.
// Every entry point validates everything before enqueueing anything.
#include <nvfp4.h>

#include <mutex>

#include "internal.h"

using namespace nvfp4;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;     // kernels index rows/cols with 32-bit ints in places
constexpr size_t kAlignWs = 256;

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned_elem(const void *p, int dtype) { return ((uintptr_t)p & (dtype == NVFP4_BF16 ? 1u : 3u)) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool dtype_ok(int d) { return d == NVFP4_F32 || d == NVFP4_BF16; }
inline bool rule_ok(int r) { return r == NVFP4_RULE_STATIC6 || r == NVFP4_RULE_4OVER6; }
inline bool block_ok(int b) { return b == NVFP4_ROW16 || b == NVFP4_TILE16 || b == NVFP4_COL16; }
inline bool dims_ok(int64_t r, int64_t c) { return r >= 0 && c >= 0 && r < kMaxDim && c < kMaxDim; }
// The quantize, dequantize and transpose kernels launch up to one lane per
// 16-element block, and a dispatch counts work-items in 32 bits: at most
// 2^32 - 2^16 blocks, 2^36 - 2^20 elements (rows, cols < 2^31: no overflow).
inline bool lanes_fit(int64_t r, int64_t c) { return r * c / 16 <= ((int64_t)1 << 32) - ((int64_t)1 << 16); }
// The GEMM's producer waves address each packed operand ([rows][k/2] code
// bytes) with 32-bit byte offsets: both operands must stay below 4 GiB.  Its
// launch has 512 threads per output tile (at least 128 x 128) and a dispatch
// counts work-items in 32 bits: fewer than 2^23 tiles of 128 x 128.
inline bool gemm_operands_fit(int64_t m, int64_t n, int64_t k)
{
    const int64_t lim = (int64_t)1 << 32;
    const int64_t tiles = ((m + 127) / 128) * ((n + 127) / 128);
    return m * (k / 2) < lim && n * (k / 2) < lim && tiles < ((int64_t)1 << 23);
}

nvfp4_status_t launch_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH; }

// Shape rule of each block kind.
bool block_shape_ok(int block, int64_t rows, int64_t cols)
{
    if (block == NVFP4_ROW16) return cols % 16 == 0;
    if (block == NVFP4_TILE16) return rows % 16 == 0 && cols % 16 == 0;
    return rows % 16 == 0;
}

nvfp4_status_t check_quant_args(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int block,
                                int rule, const uint8_t *codes, const uint8_t *scales, const float *alpha)
{
    if (!dtype_ok(x_dtype) || !rule_ok(rule) || !block_ok(block))
        return NVFP4_ERR_DTYPE;
    if (!dims_ok(rows, cols) || !lanes_fit(rows, cols) || !block_shape_ok(block, rows, cols) || ldx < cols)
        return NVFP4_ERR_SHAPE;
    if (!alpha)
        return NVFP4_ERR_NULL;
    if (rows > 0 && cols > 0 && (!x || !codes || !scales))
        return NVFP4_ERR_NULL;
    // ROW16/TILE16 read x in 16-byte vectors; COL16 reads single elements
    const bool vec = block != NVFP4_COL16;
    if ((vec && (ldx % 8 != 0 || (x && !aligned16(x)))) || (x && !aligned_elem(x, x_dtype)) ||
        (codes && !aligned16(codes)) || (scales && !aligned16(scales)))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// Quantize with the amax pass when no amax is given; ws holds the partials.
// rht_signs >= 0: COL16 blocks go through the random Hadamard transform first
// (the amax pass then measures the transformed tensor).
nvfp4_status_t do_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int block, int rule,
                           const float *amax, uint8_t *codes, uint8_t *scales, float *alpha, float *partials,
                           hipStream_t stream, int rht_signs = -1)
{
    const float *src = amax;
    int n = 1;
    if (!amax) {
        n = amax_partials(rows, cols);
        hipError_t e = rht_signs >= 0
                           ? launch_amax_col16_rht(x, x_dtype, rows, cols, ldx, (uint32_t)rht_signs, partials, n,
                                                   stream)
                           : launch_amax(x, x_dtype, rows, cols, ldx, partials, n, stream);
        if (e != hipSuccess)
            return NVFP4_ERR_LAUNCH;
        src = partials;
    }
    return launch_status(launch_quantize(x, x_dtype, rows, cols, ldx, block, rule, src, n, codes, scales, alpha,
                                         stream, rht_signs));
}

inline bool signs_ok(int s) { return s >= -1 && s <= 0xFFFF; }

bool operand_ok(const uint8_t *codes, const uint8_t *scales, const float *alpha, int layout, int64_t rows,
                int64_t k)
{
    (void)k;
    if (layout != NVFP4_SCALE_1D && layout != NVFP4_SCALE_2D)
        return false;
    if (layout == NVFP4_SCALE_2D && rows % 16 != 0)
        return false;
    (void)codes; (void)scales; (void)alpha;
    return true;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char *nvfp4_status_string(nvfp4_status_t s)
{
    switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape";
    case NVFP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case NVFP4_ERR_DTYPE: return "invalid dtype, block or rule";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_LAUNCH: return "kernel launch failed";
    case NVFP4_ERR_SCRATCH: return "call needs more than the static scratch of the no-allocation entry point";
    }
    return "unknown status";
}

size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols)
{
    (void)rows; (void)cols;
    return kAmaxBytes;
}

size_t nvfp4_workspace_size(int64_t rows, int64_t cols) { return nvfp4_quantize_workspace_size(rows, cols); }

nvfp4_status_t nvfp4_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int block,
                              int rule, const float *amax, uint8_t *codes, uint8_t *scales, float *alpha,
                              void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    nvfp4_status_t st = check_quant_args(x, x_dtype, rows, cols, ldx, block, rule, codes, scales, alpha);
    if (st != NVFP4_OK)
        return st;
    if (!amax) {
        if (!workspace || workspace_bytes < nvfp4_quantize_workspace_size(rows, cols))
            return NVFP4_ERR_WORKSPACE;
        if (!aligned16(workspace))
            return NVFP4_ERR_ALIGN;
    }
    return do_quantize(x, x_dtype, rows, cols, ldx, block, rule, amax, codes, scales, alpha, (float *)workspace,
                       stream);
}

nvfp4_status_t nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t rows,
                                int64_t cols, int block, void *y, int y_dtype, int64_t ldy, hipStream_t stream)
{
    if (!dtype_ok(y_dtype) || !block_ok(block))
        return NVFP4_ERR_DTYPE;
    if (!dims_ok(rows, cols) || !lanes_fit(rows, cols) || !block_shape_ok(block, rows, cols) || ldy < cols)
        return NVFP4_ERR_SHAPE;
    if (rows > 0 && cols > 0 && (!codes || !scales || !alpha || !y))
        return NVFP4_ERR_NULL;
    const bool vec = block != NVFP4_COL16;       // ROW16/TILE16 write 16-byte vectors
    if ((vec && (ldy % 8 != 0 || (y && !aligned16(y)))) || (y && !aligned_elem(y, y_dtype)) ||
        (codes && !aligned16(codes)) || (scales && !aligned16(scales)))
        return NVFP4_ERR_ALIGN;
    return launch_status(launch_dequantize(codes, scales, alpha, rows, cols, block, y, y_dtype, ldy, stream));
}

nvfp4_status_t nvfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha, int a_scale_layout,
                          const uint8_t *b_codes, const uint8_t *b_scales, const float *b_alpha, int b_scale_layout,
                          int64_t m, int64_t n, int64_t k, void *c, int c_dtype, int64_t ldc, float *c_amax,
                          hipStream_t stream)
{
    if (!dtype_ok(c_dtype))
        return NVFP4_ERR_DTYPE;
    if (!operand_ok(a_codes, a_scales, a_alpha, a_scale_layout, m, k) ||
        !operand_ok(b_codes, b_scales, b_alpha, b_scale_layout, n, k))
        return (a_scale_layout != 0 && a_scale_layout != 1) || (b_scale_layout != 0 && b_scale_layout != 1)
                   ? NVFP4_ERR_DTYPE
                   : NVFP4_ERR_SHAPE;
    if (m < 0 || n < 0 || k < 0 || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim || k % 16 != 0 || ldc < n ||
        !gemm_operands_fit(m, n, k))
        return NVFP4_ERR_SHAPE;
    if (m > 0 && n > 0) {
        if (!c || !a_alpha || !b_alpha)
            return NVFP4_ERR_NULL;
        if (k > 0 && (!a_codes || !a_scales || !b_codes || !b_scales))
            return NVFP4_ERR_NULL;
    }
    if ((c && !aligned_elem(c, c_dtype)) || (a_codes && !aligned16(a_codes)) ||
        (b_codes && !aligned16(b_codes)) || (a_scales && !aligned16(a_scales)) ||
        (b_scales && !aligned16(b_scales)) || (c_amax && ((uintptr_t)c_amax & 3u) != 0))
        return NVFP4_ERR_ALIGN;
    GemmOperand A{a_codes, a_scales, a_alpha, a_scale_layout};
    GemmOperand B{b_codes, b_scales, b_alpha, b_scale_layout};
    return launch_status(launch_gemm(A, B, m, n, k, c, c_dtype, ldc, c_amax, stream));
}

nvfp4_status_t nvfp4_kv_quantize(const void *kv, int kv_dtype, int64_t vectors, int64_t head_dim, int rule,
                                 const float *amax, uint8_t *codes, uint8_t *scales, float *alpha,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (head_dim % 16 != 0)
        return NVFP4_ERR_SHAPE;
    return nvfp4_quantize(kv, kv_dtype, vectors, head_dim, head_dim, NVFP4_ROW16, rule, amax, codes, scales,
                          alpha, workspace, workspace_bytes, stream);
}

// workspace: [alpha 256 B][amax partials][codes m*k/2][scales m*k/16]
size_t nvfp4_linear_workspace_size(int64_t m, int64_t k)
{
    if (m < 0 || k < 0)
        return 0;
    return kAlignWs + round_up(kAmaxBytes, kAlignWs) + round_up((size_t)(m * k / 2), kAlignWs) +
           round_up((size_t)(m * k / 16), kAlignWs);
}

}  // extern "C"

namespace {

// The argument checks of nvfp4_linear other than the workspace's.
nvfp4_status_t check_linear_args(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, int rule,
                                 const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                                 int w_scale_layout, int64_t n, void *y, int y_dtype, int64_t ldy, float *y_amax)
{
    if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype) || !rule_ok(rule) ||
        (w_scale_layout != NVFP4_SCALE_1D && w_scale_layout != NVFP4_SCALE_2D))
        return NVFP4_ERR_DTYPE;
    if (!dims_ok(m, k) || !dims_ok(n, 1) || k % 16 != 0 || ldx < k || ldy < n || !gemm_operands_fit(m, n, k) ||
        (w_scale_layout == NVFP4_SCALE_2D && n % 16 != 0))
        return NVFP4_ERR_SHAPE;
    if (!w_alpha || (m > 0 && n > 0 && !y) || (m > 0 && k > 0 && !x) || (n > 0 && k > 0 && (!w_codes || !w_scales)))
        return NVFP4_ERR_NULL;
    if (ldx % 8 != 0 || (x && !aligned16(x)) || (y && !aligned_elem(y, y_dtype)) ||
        (y_amax && ((uintptr_t)y_amax & 3u) != 0) ||
        (w_codes && !aligned16(w_codes)) || (w_scales && !aligned16(w_scales)))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// The launches of nvfp4_linear on a checked, large enough workspace ws
// (device memory, 256-byte aligned): amax partials, activation quantize, GEMM.
nvfp4_status_t linear_launches(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, int rule,
                               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                               int w_scale_layout, int64_t n, void *y, int y_dtype, int64_t ldy, float *y_amax,
                               uint8_t *ws, hipStream_t stream)
{
    float *alpha = (float *)ws;
    float *partials = (float *)(ws + kAlignWs);
    uint8_t *codes = ws + kAlignWs + round_up(kAmaxBytes, kAlignWs);
    uint8_t *scales = codes + round_up((size_t)(m * k / 2), kAlignWs);
    nvfp4_status_t st = do_quantize(x, x_dtype, m, k, ldx, NVFP4_ROW16, rule, nullptr, codes, scales, alpha,
                                    partials, stream);
    if (st != NVFP4_OK)
        return st;
    GemmOperand A{codes, scales, alpha, NVFP4_SCALE_1D};
    GemmOperand B{w_codes, w_scales, w_alpha, w_scale_layout};
    return launch_status(launch_gemm(A, B, m, n, k, y, y_dtype, ldy, y_amax, stream));
}

// Scratch of nvfp4_linear_no_alloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  In host code its name
// is only a host-side stand-in; the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static_assert(NVFP4_NO_ALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[NVFP4_NO_ALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
uint8_t *g_scratch_ptr[kMaxScratchDevices];     // device address of `scratch` on each device, once looked up

// The current device's copy of the scratch array (its address looked up on
// the first call on that device).
nvfp4_status_t current_device_scratch(uint8_t **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
        (void)hipGetLastError();
        return NVFP4_ERR_LAUNCH;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();            // leave no sticky error for the caller's next call
            return NVFP4_ERR_LAUNCH;
        }
        g_scratch_ptr[dev] = (uint8_t *)p;
    }
    *out = g_scratch_ptr[dev];
    return NVFP4_OK;
}

}  // namespace

extern "C" {

nvfp4_status_t nvfp4_linear(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, int rule,
                            const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                            int w_scale_layout, int64_t n, void *y, int y_dtype, int64_t ldy, float *y_amax,
                            void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    nvfp4_status_t st = check_linear_args(x, x_dtype, m, k, ldx, rule, w_codes, w_scales, w_alpha, w_scale_layout,
                                          n, y, y_dtype, ldy, y_amax);
    if (st != NVFP4_OK)
        return st;
    if (!workspace || workspace_bytes < nvfp4_linear_workspace_size(m, k))
        return NVFP4_ERR_WORKSPACE;
    if (((uintptr_t)workspace % kAlignWs) != 0)
        return NVFP4_ERR_ALIGN;
    return linear_launches(x, x_dtype, m, k, ldx, rule, w_codes, w_scales, w_alpha, w_scale_layout, n, y, y_dtype,
                           ldy, y_amax, (uint8_t *)workspace, stream);
}

nvfp4_status_t nvfp4_linear_no_alloc(const void *x, int x_dtype, int64_t m, int64_t k, int64_t ldx, int rule,
                                     const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                                     int w_scale_layout, int64_t n, void *y, int y_dtype, int64_t ldy,
                                     float *y_amax, hipStream_t stream)
{
    nvfp4_status_t st = check_linear_args(x, x_dtype, m, k, ldx, rule, w_codes, w_scales, w_alpha, w_scale_layout,
                                          n, y, y_dtype, ldy, y_amax);
    if (st != NVFP4_OK)
        return st;
    if (nvfp4_linear_workspace_size(m, k) > (size_t)NVFP4_NO_ALLOC_SCRATCH_BYTES)
        return NVFP4_ERR_SCRATCH;
    uint8_t *ws = nullptr;
    st = current_device_scratch(&ws);
    if (st != NVFP4_OK)
        return st;
    // nothing in the scratch has to start at zero: the amax pass writes every
    // partial the quantizer reads, the quantizer writes alpha, codes and scales
    return linear_launches(x, x_dtype, m, k, ldx, rule, w_codes, w_scales, w_alpha, w_scale_layout, n, y, y_dtype,
                           ldy, y_amax, ws, stream);
}

size_t nvfp4_linear_lora_workspace_size(int64_t m, int64_t k, int rank)
{
    if (m < 0 || k < 0 || rank < 0)
        return 0;
    return nvfp4_linear_workspace_size(m, k) + round_up((size_t)kLoraMaxSlicesAbi * m * rank * 4, kAlignWs) +
           round_up((size_t)kMaxAmaxSrc * 4, kAlignWs);
}

nvfp4_status_t nvfp4_linear_lora(const void *x, int64_t m, int64_t k, int64_t ldx, int rule,
                                 const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                                 int w_scale_layout, int64_t n, const void *lora_a, const void *lora_b, int rank,
                                 float lora_scale, void *lora_u, void *y, int y_dtype, int64_t ldy, float *y_amax,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    // the NVFP4 part is nvfp4_linear's; the branch adds its own checks
    if (rank < 32 || rank > 128 || rank % 32 != 0 || !(lora_scale == lora_scale) || lora_scale == 0.0f ||
        __builtin_isinf(lora_scale))
        return NVFP4_ERR_SHAPE;
    if ((m > 0 && k > 0 && !lora_a) || (n > 0 && !lora_b) || (m > 0 && !lora_u))
        return NVFP4_ERR_NULL;
    if ((lora_a && !aligned16(lora_a)) || (lora_b && !aligned16(lora_b)) || (lora_u && !aligned16(lora_u)))
        return NVFP4_ERR_ALIGN;
    if (!dtype_ok(y_dtype) || !rule_ok(rule) || (w_scale_layout != NVFP4_SCALE_1D && w_scale_layout != NVFP4_SCALE_2D))
        return NVFP4_ERR_DTYPE;
    if (!dims_ok(m, k) || !dims_ok(n, 1) || k % 16 != 0 || ldx < k || ldy < n || !gemm_operands_fit(m, n, k) ||
        (w_scale_layout == NVFP4_SCALE_2D && n % 16 != 0))
        return NVFP4_ERR_SHAPE;
    if (!w_alpha || (m > 0 && n > 0 && !y) || (m > 0 && k > 0 && !x) || (n > 0 && k > 0 && (!w_codes || !w_scales)))
        return NVFP4_ERR_NULL;
    if (ldx % 8 != 0 || (x && !aligned16(x)) || (y && !aligned_elem(y, y_dtype)) ||
        (y_amax && ((uintptr_t)y_amax & 3u) != 0) || (w_codes && !aligned16(w_codes)) ||
        (w_scales && !aligned16(w_scales)))
        return NVFP4_ERR_ALIGN;
    static_assert(kLoraMaxSlicesAbi >= 1, "slices");
    if (!workspace || workspace_bytes < nvfp4_linear_lora_workspace_size(m, k, rank))
        return NVFP4_ERR_WORKSPACE;
    if (((uintptr_t)workspace % kAlignWs) != 0)
        return NVFP4_ERR_ALIGN;
    uint8_t *ws = (uint8_t *)workspace;
    float *alpha = (float *)ws;
    float *partials = (float *)(ws + kAlignWs);
    uint8_t *codes = ws + kAlignWs + round_up(kAmaxBytes, kAlignWs);
    uint8_t *scales = codes + round_up((size_t)(m * k / 2), kAlignWs);
    float *lora_part = (float *)(ws + nvfp4_linear_workspace_size(m, k));
    float *lora_amax = (float *)((uint8_t *)lora_part + round_up((size_t)kLoraMaxSlicesAbi * m * rank * 4, kAlignWs));
    nvfp4_status_t st;
    const int na = lora_amax_partials(m, k);
    if (na >= 1 && na <= kMaxAmaxSrc) {
        // U = x A^T in K-slice partials first: that kernel reads all of x and
        // also leaves one max |x| per workgroup, which stand in for the
        // quantizer's own amax pass; then the quantizer, then the sum into U
        st = launch_status(launch_lora_partial((const uint16_t *)x, ldx, m, k, (const uint16_t *)lora_a, rank,
                                               lora_part, lora_amax, stream));
        if (st != NVFP4_OK)
            return st;
        st = launch_status(launch_quantize(x, NVFP4_BF16, m, k, ldx, NVFP4_ROW16, rule, lora_amax, na, codes, scales,
                                           alpha, stream));
        if (st != NVFP4_OK)
            return st;
        st = launch_status(launch_lora_reduce(m, k, rank, lora_part, (uint16_t *)lora_u, stream));
    } else {
        st = do_quantize(x, NVFP4_BF16, m, k, ldx, NVFP4_ROW16, rule, nullptr, codes, scales, alpha, partials,
                         stream);
        if (st != NVFP4_OK)
            return st;
        // U = x A^T (an empty contraction gives zeros)
        st = launch_status(launch_lora_down((const uint16_t *)x, ldx, m, k, (const uint16_t *)lora_a, rank,
                                            (uint16_t *)lora_u, lora_part, stream));
    }
    if (st != NVFP4_OK)
        return st;
    GemmOperand A{codes, scales, alpha, NVFP4_SCALE_1D};
    GemmOperand B{w_codes, w_scales, w_alpha, w_scale_layout};
    LoraBranch lb{(const uint16_t *)lora_u, (const uint16_t *)lora_b, rank, lora_scale};
    return launch_status(launch_gemm(A, B, m, n, k, y, y_dtype, ldy, y_amax, stream, &lb));
}

// workspace: [alpha_dy][alpha_x] (256 B), [partials dy][partials x],
//            [dy^T codes][dy^T scales][x^T codes][x^T scales]
size_t nvfp4_wgrad_workspace_size(int64_t tokens, int64_t n_out, int64_t k_in)
{
    if (tokens < 0 || n_out < 0 || k_in < 0)
        return 0;
    return kAlignWs + 2 * round_up(kAmaxBytes, kAlignWs) + round_up((size_t)(n_out * tokens / 2), kAlignWs) +
           round_up((size_t)(n_out * tokens / 16), kAlignWs) + round_up((size_t)(k_in * tokens / 2), kAlignWs) +
           round_up((size_t)(k_in * tokens / 16), kAlignWs);
}

nvfp4_status_t nvfp4_wgrad(const void *dy, const void *x, int dtype, int64_t tokens, int64_t n_out, int64_t k_in,
                           int64_t lddy, int64_t ldx, int rule, int rht_signs, const float *dy_amax,
                           const float *x_amax, void *dw, int dw_dtype, int64_t lddw,
                           void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!dtype_ok(dtype) || !dtype_ok(dw_dtype) || !rule_ok(rule) || !signs_ok(rht_signs))
        return NVFP4_ERR_DTYPE;
    if (!dims_ok(tokens, n_out) || !dims_ok(k_in, 1) || tokens % 16 != 0 || lddy < n_out || ldx < k_in ||
        !gemm_operands_fit(n_out, k_in, tokens) ||
        lddw < k_in)
        return NVFP4_ERR_SHAPE;
    if ((n_out > 0 && k_in > 0 && !dw) || (tokens > 0 && ((n_out > 0 && !dy) || (k_in > 0 && !x))))
        return NVFP4_ERR_NULL;
    if ((dy && !aligned_elem(dy, dtype)) || (x && !aligned_elem(x, dtype)) || (dw && !aligned_elem(dw, dw_dtype)) ||
        ((uintptr_t)dy_amax & 3u) || ((uintptr_t)x_amax & 3u))
        return NVFP4_ERR_ALIGN;
    if (!workspace || workspace_bytes < nvfp4_wgrad_workspace_size(tokens, n_out, k_in))
        return NVFP4_ERR_WORKSPACE;
    if (((uintptr_t)workspace % kAlignWs) != 0)
        return NVFP4_ERR_ALIGN;
    uint8_t *ws = (uint8_t *)workspace;
    float *alpha_dy = (float *)ws;
    float *alpha_x = (float *)ws + 1;
    float *part_dy = (float *)(ws + kAlignWs);
    float *part_x = (float *)(ws + kAlignWs + round_up(kAmaxBytes, kAlignWs));
    uint8_t *c_dy = ws + kAlignWs + 2 * round_up(kAmaxBytes, kAlignWs);
    uint8_t *s_dy = c_dy + round_up((size_t)(n_out * tokens / 2), kAlignWs);
    uint8_t *c_x = s_dy + round_up((size_t)(n_out * tokens / 16), kAlignWs);
    uint8_t *s_x = c_x + round_up((size_t)(k_in * tokens / 2), kAlignWs);
    // a handed-in amax replaces that operand's amax pass
    nvfp4_status_t st = do_quantize(dy, dtype, tokens, n_out, lddy, NVFP4_COL16, rule, dy_amax, c_dy, s_dy,
                                    alpha_dy, part_dy, stream, rht_signs);
    if (st != NVFP4_OK)
        return st;
    st = do_quantize(x, dtype, tokens, k_in, ldx, NVFP4_COL16, rule, x_amax, c_x, s_x, alpha_x, part_x, stream,
                     rht_signs);
    if (st != NVFP4_OK)
        return st;
    GemmOperand A{c_dy, s_dy, alpha_dy, NVFP4_SCALE_1D};
    GemmOperand B{c_x, s_x, alpha_x, NVFP4_SCALE_1D};
    return launch_status(launch_gemm(A, B, n_out, k_in, tokens, dw, dw_dtype, lddw, nullptr, stream));
}

nvfp4_status_t nvfp4_transpose_tile16(const uint8_t *codes, const uint8_t *scales, const float *alpha,
                                     int64_t rows, int64_t cols, uint8_t *codes_t, uint8_t *scales_t,
                                     float *alpha_t, hipStream_t stream)
{
    if (!dims_ok(rows, cols) || !lanes_fit(rows, cols) || rows % 16 != 0 || cols % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!alpha || !alpha_t)
        return NVFP4_ERR_NULL;
    if (rows > 0 && cols > 0 && (!codes || !scales || !codes_t || !scales_t))
        return NVFP4_ERR_NULL;
    if ((codes && !aligned16(codes)) || (codes_t && !aligned16(codes_t)) || (scales && !aligned16(scales)) ||
        (scales_t && !aligned16(scales_t)) || ((uintptr_t)alpha & 3u) || ((uintptr_t)alpha_t & 3u))
        return NVFP4_ERR_ALIGN;
    return launch_status(launch_transpose_tile16(codes, scales, alpha, rows, cols, codes_t, scales_t, alpha_t,
                                                 stream));
}

nvfp4_status_t nvfp4_quantize_col16_rht(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                       int rule, int rht_signs, const float *amax, uint8_t *codes, uint8_t *scales,
                                       float *alpha, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!signs_ok(rht_signs) || rht_signs < 0)
        return NVFP4_ERR_DTYPE;
    nvfp4_status_t st = check_quant_args(x, x_dtype, rows, cols, ldx, NVFP4_COL16, rule, codes, scales, alpha);
    if (st != NVFP4_OK)
        return st;
    if (!amax) {
        if (!workspace || workspace_bytes < nvfp4_quantize_workspace_size(rows, cols))
            return NVFP4_ERR_WORKSPACE;
        if (!aligned16(workspace))
            return NVFP4_ERR_ALIGN;
    }
    return do_quantize(x, x_dtype, rows, cols, ldx, NVFP4_COL16, rule, amax, codes, scales, alpha,
                       (float *)workspace, stream, rht_signs);
}

size_t nvfp4_kv_chunked_workspace_size(int64_t tensors, int64_t heads, int64_t tokens, int64_t head_dim,
                                       int64_t tokens_per_chunk)
{
    (void)heads; (void)head_dim;
    if (tensors <= 0 || tokens <= 0 || tokens_per_chunk <= 0)
        return kAlignWs;
    const int64_t nch = (tokens + tokens_per_chunk - 1) / tokens_per_chunk;
    return round_up((size_t)tensors * (size_t)nch * kMaxAmaxSrc * sizeof(float), kAlignWs);
}

namespace {
// The checks shared by the chunked KV quantize and dequantize.
nvfp4_status_t check_kv_chunked(int64_t tensors, int64_t heads, int64_t tokens, int64_t head_dim,
                                int64_t tokens_per_chunk)
{
    if (tensors < 0 || tensors > 65535 || heads < 1 || heads > kMaxAmaxSrc || tokens < 0 || head_dim < 16 ||
        head_dim % 16 != 0 || tokens_per_chunk < 1 || tokens >= kMaxDim || head_dim >= kMaxDim ||
        !lanes_fit(tensors * heads * tokens, head_dim))
        return NVFP4_ERR_SHAPE;
    const int64_t nch = (tokens + tokens_per_chunk - 1) / tokens_per_chunk;
    const int64_t bpr = head_dim / 16;
    // grid limits of the launches: units (tensor, chunk) and quantize workgroups per segment
    if (tensors * nch > 65535 ||
        (tokens_per_chunk < tokens ? tokens_per_chunk : tokens) * bpr / kQuantThreads >= 0x7fffffff)
        return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}
}  // namespace

nvfp4_status_t nvfp4_kv_quantize_chunked(const void *kv, int kv_dtype, int64_t tensors, int64_t heads,
                                         int64_t tokens, int64_t head_dim, int64_t tokens_per_chunk, int rule,
                                         const float *chunk_amax, uint8_t *codes, uint8_t *scales, float *alphas,
                                         void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!dtype_ok(kv_dtype) || !rule_ok(rule))
        return NVFP4_ERR_DTYPE;
    nvfp4_status_t st = check_kv_chunked(tensors, heads, tokens, head_dim, tokens_per_chunk);
    if (st != NVFP4_OK)
        return st;
    if (tokens == 0 || tensors == 0)
        return NVFP4_OK;                                  // no chunk, nothing to write
    if (!kv || !codes || !scales || !alphas)
        return NVFP4_ERR_NULL;
    if (!aligned16(kv) || !aligned16(codes) || !aligned16(scales) || ((uintptr_t)alphas & 3u) ||
        ((uintptr_t)chunk_amax & 3u))
        return NVFP4_ERR_ALIGN;
    if (!chunk_amax) {
        if (!workspace || workspace_bytes < nvfp4_kv_chunked_workspace_size(tensors, heads, tokens, head_dim,
                                                                            tokens_per_chunk))
            return NVFP4_ERR_WORKSPACE;
        if (!aligned16(workspace))
            return NVFP4_ERR_ALIGN;
    }
    return launch_status(launch_kv_quantize_chunked(kv, kv_dtype, tensors, heads, tokens, head_dim,
                                                    tokens_per_chunk, rule, chunk_amax, codes, scales, alphas,
                                                    (float *)workspace, stream));
}

nvfp4_status_t nvfp4_kv_dequantize_chunked(const uint8_t *codes, const uint8_t *scales, const float *alphas,
                                           int64_t tensors, int64_t heads, int64_t tokens, int64_t head_dim,
                                           int64_t tokens_per_chunk, void *y, int y_dtype, hipStream_t stream)
{
    if (!dtype_ok(y_dtype))
        return NVFP4_ERR_DTYPE;
    nvfp4_status_t st = check_kv_chunked(tensors, heads, tokens, head_dim, tokens_per_chunk);
    if (st != NVFP4_OK)
        return st;
    if (tokens == 0 || tensors == 0)
        return NVFP4_OK;
    if (!codes || !scales || !alphas || !y)
        return NVFP4_ERR_NULL;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(y) || ((uintptr_t)alphas & 3u))
        return NVFP4_ERR_ALIGN;
    return launch_status(launch_kv_dequantize_chunked(codes, scales, alphas, tensors, heads, tokens, head_dim,
                                                      tokens_per_chunk, y, y_dtype, stream));
}

size_t nvfp4_kv_smooth_workspace_size(int64_t vectors, int64_t head_dim)
{
    (void)vectors; (void)head_dim;
    return kAmaxBytes;
}

nvfp4_status_t nvfp4_kv_quantize_smoothed(const void *k, int k_dtype, int64_t vectors, int64_t head_dim, int rule,
                                          uint8_t *codes, uint8_t *scales, float *alpha, float *means,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!dtype_ok(k_dtype) || !rule_ok(rule))
        return NVFP4_ERR_DTYPE;
    if (!dims_ok(vectors, head_dim) || !lanes_fit(vectors, head_dim) || head_dim < 16 || head_dim > 1024 ||
        (head_dim & (head_dim - 1)) != 0)
        return NVFP4_ERR_SHAPE;
    if (!alpha || (vectors > 0 && (!k || !codes || !scales || !means)))
        return NVFP4_ERR_NULL;
    if ((k && !aligned16(k)) || (codes && !aligned16(codes)) || (scales && !aligned16(scales)) ||
        (means && ((uintptr_t)means & 3u)) || ((uintptr_t)alpha & 3u))
        return NVFP4_ERR_ALIGN;
    if (!workspace || workspace_bytes < nvfp4_kv_smooth_workspace_size(vectors, head_dim))
        return NVFP4_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return NVFP4_ERR_ALIGN;
    return launch_status(launch_kv_smooth_quantize(k, k_dtype, vectors, head_dim, rule, codes, scales, alpha, means,
                                                   (float *)workspace, stream));
}

nvfp4_status_t nvfp4_kv_dequantize_window(const nvfp4_kv_segment_t *segments, int n_segments, int64_t head_dim,
                                          void *out, int out_dtype, int64_t ldo, hipStream_t stream)
{
    if (!dtype_ok(out_dtype))
        return NVFP4_ERR_DTYPE;
    if (n_segments < 0 || n_segments > NVFP4_MAX_KV_SEGMENTS || head_dim < 16 || head_dim % 16 != 0 ||
        head_dim >= kMaxDim || ldo < head_dim)
        return NVFP4_ERR_SHAPE;
    if (n_segments > 0 && !segments)
        return NVFP4_ERR_NULL;
    static_assert(NVFP4_MAX_KV_SEGMENTS == kMaxKvSegments, "segment table size");
    KvWindowArgs a{};
    a.n = n_segments;
    a.bpr = (int)(head_dim / 16);
    int64_t rows = 0, wgs = 0;
    for (int i = 0; i < n_segments; i++) {
        const nvfp4_kv_segment_t &g = segments[i];
        if (g.first < 0 || g.count < 0 || g.first >= kMaxDim || g.count >= kMaxDim)
            return NVFP4_ERR_SHAPE;
        if (g.count > 0 && (!g.codes || !g.scales || !g.alpha))
            return NVFP4_ERR_NULL;
        if ((g.codes && !aligned16(g.codes)) || (g.scales && !aligned16(g.scales)) || ((uintptr_t)g.alpha & 3u) ||
            ((uintptr_t)g.means & 3u))
            return NVFP4_ERR_ALIGN;
        if (g.count * a.bpr >= kMaxDim)
            return NVFP4_ERR_SHAPE;
        a.seg[i] = KvSegmentDev{g.codes, g.scales, g.alpha, g.means, g.first, g.count, rows, wgs};
        rows += g.count;
        wgs += (g.count * a.bpr + kQuantThreads - 1) / kQuantThreads;
    }
    a.wgs = wgs;
    if (rows >= kMaxDim || rows * a.bpr >= kMaxDim)
        return NVFP4_ERR_SHAPE;
    a.rows = rows;
    if (rows > 0 && !out)
        return NVFP4_ERR_NULL;
    if (out && (!aligned16(out) || (ldo * (out_dtype == NVFP4_BF16 ? 2 : 4)) % 16 != 0))
        return NVFP4_ERR_ALIGN;
    return launch_status(launch_kv_window(a, out, out_dtype, ldo, stream));
}

}  // extern "C"
