// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"

namespace nvfp4 {

constexpr int kQuantThreads = 256;      // threads per quantize workgroup
constexpr int kRowBlocks = 1;           // 16-element blocks per lane in the ROW16 kernel
// Inputs of at least this many bytes are read with non-temporal loads by the
// amax and ROW16 quantize passes; smaller ones with ordinary loads, so that
// the quantize pass finds part of what the amax pass read in the last-level
// cache (256 MB).  Thresholds of 64, 128 and 256 MiB measured on 16, 76,
// 113.5 and 201 MB inputs: 128 MiB was best or level on each.
constexpr int64_t kStreamLoadBytes = (int64_t)128 << 20;
constexpr int kAmaxThreads = 1024;      // threads per amax workgroup
constexpr int kAmaxUnroll = 8;          // 16-byte loads in flight per thread of the per-chunk amax pass
constexpr int kMaxAmaxPartials = 256;   // amax pass: at most this many workgroups
constexpr size_t kAmaxBytes = kMaxAmaxPartials * sizeof(float);
constexpr int kMaxAmaxSrc = 1024;       // ROW16 quantize: at most this many amax partials (others: 256)

// number of amax workgroups (= partial maxima) for a rows x cols tensor
int amax_partials(int64_t rows, int64_t cols);

// dtype: 0 fp32, 1 bf16.  block: 0 ROW16, 1 TILE16, 2 COL16.
hipError_t launch_amax(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, float *partials,
                       int n_partials, hipStream_t s);

// amax partials of the COL16 blocks after the random Hadamard transform
hipError_t launch_amax_col16_rht(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, uint32_t signs,
                                 float *partials, int n_partials, hipStream_t s);

// amax_src: n_amax partial maxima (n_amax > 1) or one amax (n_amax == 1).
// rht_signs >= 0 (COL16 only): transform every block first (signs in bits 0-15).
hipError_t launch_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int block, int rule,
                           const float *amax_src, int n_amax, uint8_t *codes, uint8_t *scales, float *alpha,
                           hipStream_t s, int rht_signs = -1);

hipError_t launch_dequantize(const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t rows,
                             int64_t cols, int block, void *y, int ydtype, int64_t ldy, hipStream_t s);

// Key smoothing + quantization of a [vectors][head_dim] key tensor (two passes:
// means and amax, then quantize); head_dim a power of two in [16, 1024].
hipError_t launch_kv_smooth_quantize(const void *x, int dtype, int64_t vectors, int64_t head_dim, int rule,
                                     uint8_t *codes, uint8_t *scales, float *alpha, float *means, float *partials,
                                     hipStream_t s);

// KV caches [tensors][heads][tokens][d] with one alpha per tensor and chunk of
// tpc tokens: per-unit amax partials (unless chunk_amax [tensors][n_chunks]
// is given), then the ROW16 quantizer with each unit's alpha; alphas
// [tensors][n_chunks].  partials: tensors * n_chunks * kMaxAmaxSrc floats of
// scratch.  heads <= kMaxAmaxSrc.
int kv_chunk_pseg(int64_t heads, int64_t units);
hipError_t launch_kv_quantize_chunked(const void *x, int dtype, int64_t tensors, int64_t heads, int64_t tokens,
                                      int64_t d, int64_t tpc, int rule, const float *chunk_amax, uint8_t *codes,
                                      uint8_t *scales, float *alphas, float *partials, hipStream_t s);
hipError_t launch_kv_dequantize_chunked(const uint8_t *codes, const uint8_t *scales, const float *alphas,
                                        int64_t tensors, int64_t heads, int64_t tokens, int64_t d, int64_t tpc,
                                        void *y, int ydtype, hipStream_t s);

// Window reconstruction from cached chunks (segment table passed by value).
constexpr int kMaxKvSegments = 32;
struct KvSegmentDev {
    const uint8_t *codes;
    const uint8_t *scales;
    const float *alpha;
    const float *means;     // NULL: no mean to add back
    int64_t first;          // first row (vector) of the chunk taken
    int64_t count;          // rows taken
    int64_t out_row;        // first output row of this segment
    int64_t wg0;            // first workgroup serving this segment
};
struct KvWindowArgs {
    KvSegmentDev seg[kMaxKvSegments];
    int n;
    int bpr;                // 16-element blocks per row (head_dim / 16)
    int64_t rows;           // output rows in total
    int64_t wgs;            // workgroups in total
};
hipError_t launch_kv_window(const KvWindowArgs &a, void *y, int ydtype, int64_t ldy, hipStream_t s);

struct GemmOperand {
    const uint8_t *codes;
    const uint8_t *scales;
    const float *alpha;
    int scale2d;
};

// W^T of a 16x16-tile tensor W [rows][cols]: codes [cols][rows/2], scales
// [cols/16][rows/16], alpha copied.  rows, cols multiples of 16.
hipError_t launch_transpose_tile16(const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t rows,
                                   int64_t cols, uint8_t *codes_t, uint8_t *scales_t, float *alpha_t, hipStream_t s);

// Optional BF16 LoRA branch added in the GEMM: C += scale * U B^T with U [m][r]
// and B [n][r] bf16 (r a multiple of 16, at most 128).
struct LoraBranch {
    const uint16_t *u;
    const uint16_t *b;
    int r;
    float scale;
};

// c_amax (optional): receives max |C| of the stored values
hipError_t launch_gemm(const GemmOperand &a, const GemmOperand &b, int64_t m, int64_t n, int64_t k, void *c,
                       int cdtype, int64_t ldc, float *c_amax, hipStream_t s, const LoraBranch *lora = nullptr);

// U [m][r] = bf16(x A^T): x [m][k] bf16 (ld ldx), A [r][k] bf16; r % 32 == 0,
// r <= 128.  partials: lora_slices(m, k) * m * r floats of scratch.
int lora_slices(int64_t m, int64_t k);
constexpr int kLoraMaxSlicesAbi = 8;
hipError_t launch_lora_down(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, const uint16_t *a, int r,
                            uint16_t *u, float *partials, hipStream_t s);
// The same in two launches: the K-slice partial products, which also write
// one max |x| per workgroup to amax_part (lora_amax_partials(m, k) of them;
// none when k == 0), then their sum into U.
int lora_amax_partials(int64_t m, int64_t k);
hipError_t launch_lora_partial(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, const uint16_t *a, int r,
                               float *partials, float *amax_part, hipStream_t s);
hipError_t launch_lora_reduce(int64_t m, int64_t k, int r, const float *partials, uint16_t *u, hipStream_t s);

}  // namespace nvfp4
