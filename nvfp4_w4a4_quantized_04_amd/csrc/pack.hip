// Packed-layout utilities: the transpose of a 16x16-tile NVFP4 tensor.
//
// A weight quantized with one E4M3 scale per 16x16 tile ("LongLive-2.0: An
// NVFP4 Parallel Infrastructure for Long Video Generation", architecture
// walkthrough page, NVFP4 Training section, "NVFP4 training recipe": 2D block
// scaling for weights) holds the same tiles in either orientation.  DGRAD
// contracts the weight over its output dimension ("The three GEMMs of
// backpropagation"), so it needs W^T with that dimension contiguous: the same
// codes and scales, transposed.  No value is re-quantized.
#include "internal.h"

namespace nvfp4 {

// One lane per 16x16 tile: its 16 code rows (8 bytes each, element 2j in the
// low nibble) form a 16x16 matrix of nibbles in 16 64-bit words (nibble j of
// word i = element (i, j)); four exchange stages of halving block size
// transpose it in registers.
__global__ __launch_bounds__(256) void k_transpose_tile16(const uint8_t *__restrict__ codes,
                                                          const uint8_t *__restrict__ scales,
                                                          const float *__restrict__ alpha, int64_t rows,
                                                          int64_t cols, uint8_t *__restrict__ codes_t,
                                                          uint8_t *__restrict__ scales_t, float *__restrict__ alpha_t)
{
    const int64_t tiles_c = cols / 16, tiles_r = rows / 16;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t == 0)
        *alpha_t = *alpha;
    if (t >= tiles_r * tiles_c)
        return;
    const int64_t tr = t / tiles_c, tc = t - tr * tiles_c;
    uint64_t w[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint2 v = *reinterpret_cast<const uint2 *>(codes + (tr * 16 + i) * (cols / 2) + tc * 8);
        w[i] = (uint64_t)v.x | ((uint64_t)v.y << 32);
    }
    // stage b: rows i and i+b (i & b == 0) exchange the nibble columns j with
    // j & b set (row i) against those with j & b clear (row i+b)
    constexpr uint64_t kMask[4] = {0x00000000FFFFFFFFull, 0x0000FFFF0000FFFFull, 0x00FF00FF00FF00FFull,
                                   0x0F0F0F0F0F0F0F0Full};
#pragma unroll
    for (int st = 0; st < 4; st++) {
        const int b = 8 >> st;
        const int sh = 4 * b;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            if (i & b)
                continue;
            const uint64_t d = ((w[i] >> sh) ^ w[i + b]) & kMask[st];
            w[i + b] ^= d;
            w[i] ^= d << sh;
        }
    }
#pragma unroll
    for (int j = 0; j < 16; j++)
        *reinterpret_cast<uint2 *>(codes_t + (tc * 16 + j) * (rows / 2) + tr * 8) =
            make_uint2((uint32_t)w[j], (uint32_t)(w[j] >> 32));
    scales_t[tc * tiles_r + tr] = scales[tr * tiles_c + tc];
}

hipError_t launch_transpose_tile16(const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t rows,
                                   int64_t cols, uint8_t *codes_t, uint8_t *scales_t, float *alpha_t, hipStream_t s)
{
    const int64_t tiles = (rows / 16) * (cols / 16);
    const int64_t grid = tiles > 0 ? (tiles + 255) / 256 : 1;
    k_transpose_tile16<<<(unsigned)grid, 256, 0, s>>>(codes, scales, alpha, rows, cols, codes_t, scales_t, alpha_t);
    return hipGetLastError();
}

}  // namespace nvfp4
