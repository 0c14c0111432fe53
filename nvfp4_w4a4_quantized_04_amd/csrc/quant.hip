// NVFP4 quantize / dequantize / amax kernels for gfx950.
//
// Operation ("LongLive-2.0: An NVFP4 Parallel Infrastructure for Long Video
// Generation", architecture walkthrough page, NVFP4 Training section,
// "Hierarchical scaling" and "Quantization rule for a tensor block"; NVFP4
// Inference section, "Scale-search mechanism" and "Chunkwise quantization
// procedure" for the KV cache):
//   pass 1  amax of the tensor -> per-workgroup partial maxima
//   pass 2  every workgroup reduces the partials (identical alpha everywhere),
//           then each lane quantizes whole 16-element blocks held in its own
//           registers: no cross-lane traffic on the hot path.
#include "internal.h"

#include <type_traits>

namespace nvfp4 {

// alpha from the amax partial maxima (n_amax > 1) or from one amax
// (n_amax == 1), in two phases.  Vector loads complete in order, so a partial
// loaded after a kernel's data loads would wait for all of them: alpha_issue
// starts the partial load first, the kernel then issues its data loads, and
// alpha_finish reduces while the data is in flight.  Every thread of the
// block (kQuantThreads) must call both; all get the same alpha.
static_assert(kMaxAmaxPartials <= kQuantThreads, "one partial per thread");

// The loads are unconditional (n_amax >= 1): a thread past the partials
// re-reads the last one, which cannot change the max; with one amax every
// thread reads it.  NPT: partials per thread (up to NPT * kQuantThreads).
template <int NPT = 1>
__device__ __forceinline__ float alpha_issue(const float *__restrict__ amax_src, int n_amax)
{
    float a = amax_src[(int)threadIdx.x < n_amax ? (int)threadIdx.x : n_amax - 1];
#pragma unroll
    for (int j = 1; j < NPT; j++) {
        const int i = (int)threadIdx.x + j * kQuantThreads;
        a = fmaxf(a, amax_src[i < n_amax ? i : n_amax - 1]);
    }
    return a;
}

__device__ __forceinline__ float alpha_finish(float part, const float *__restrict__ amax_src, int n_amax)
{
    (void)amax_src;
    __shared__ float red[kQuantThreads / 64];
    float a;
    if (n_amax == 1) {
        a = part;
    } else {
        a = wave_max(part);
        if ((threadIdx.x & 63) == 0)
            red[threadIdx.x >> 6] = a;
        __syncthreads();
        a = red[0];
#pragma unroll
        for (int w = 1; w < kQuantThreads / 64; w++)
            a = fmaxf(a, red[w]);
    }
    return global_scale(a);
}

// ---------------------------------------------------------------- amax

template <typename T>
__device__ __forceinline__ float absmax16B(uint4 v, float a)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
        if (sizeof(T) == 2)
            a = fmaxf(a, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
        else
            a = fmaxf(a, fabsf(__uint_as_float(w[j])));
    }
    return a;
}

// Partial maxima: workgroup w takes the groups w, w + grid, w + 2 grid, ... of
// TH * U consecutive 16-byte vectors, every thread keeping U loads in flight
// (the last group's loads are predicated, not serialized); vec: the tensor is
// contiguous and 16-byte aligned, else rows are read element by element.
// NT: non-temporal vector loads (large inputs).
template <typename T, int TH, int U, bool NT>
__global__ __launch_bounds__(TH) void k_amax(const T *__restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                                             bool vec, float *__restrict__ partials)
{
    __shared__ float red[TH / 64];
    float a = 0.0f;
    if (vec) {
        constexpr int V = 16 / sizeof(T);
        const int64_t n = rows * cols;
        const int64_t nv = n / V;
        const uint4 *xv = reinterpret_cast<const uint4 *>(x);
        const int64_t step = (int64_t)gridDim.x * TH * U;
        for (int64_t g = (int64_t)blockIdx.x * TH * U; g < nv; g += step) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t i = g + u * TH + threadIdx.x;
                v[u] = i < nv ? (NT ? load_stream(xv + i) : xv[i]) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; u++)
                a = absmax16B<T>(v[u], a);
        }
        // elements past the last whole vector
        const int64_t stride = (int64_t)gridDim.x * TH;
        for (int64_t t = nv * V + (int64_t)blockIdx.x * TH + threadIdx.x; t < n; t += stride)
            a = fmaxf(a, fabsf(load1(x + t)));
    } else {
        // strided rows: rows spread over workgroups, threads along the row
        for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
            for (int64_t c = threadIdx.x; c < cols; c += TH)
                a = fmaxf(a, fabsf(load1(x + r * ldx + c)));
    }
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = red[0];
#pragma unroll
        for (int w = 1; w < TH / 64; w++)
            b = fmaxf(b, red[w]);
        partials[blockIdx.x] = b;
    }
}

// The 16 values of one block from its raw 16-byte vectors (2 for bf16, 4 for fp32).
template <typename T>
__device__ __forceinline__ void unpack16(const uint4 (&raw)[sizeof(T)], float (&v)[16])
{
    if constexpr (sizeof(T) == 2) {
        const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            v[4 * q] = __uint_as_float(raw[q].x);
            v[4 * q + 1] = __uint_as_float(raw[q].y);
            v[4 * q + 2] = __uint_as_float(raw[q].z);
            v[4 * q + 3] = __uint_as_float(raw[q].w);
        }
    }
}

// An empty tensor: only alpha (from the given amax or partials; 1 when 0).
__global__ __launch_bounds__(kQuantThreads) void k_alpha_only(const float *__restrict__ amax_src, int n_amax,
                                                              float *__restrict__ alpha_out)
{
    const float apart = alpha_issue(amax_src, n_amax);
    const float alpha = alpha_finish(apart, amax_src, n_amax);
    if (threadIdx.x == 0)
        *alpha_out = alpha;
}

// ------------------------------------------------------ ROW16 (1D, along cols)

// Each lane quantizes kRowBlocks whole 16-element blocks held in its own
// registers (blocks b, b+256, ... of the workgroup's range, so every load and
// store instruction of a wave is contiguous).  Blocks are numbered row-major:
// block b's codes are bytes [8b, 8b+8), its scale is byte b (cols % 16 == 0).
template <typename T, bool RULE4, int NPT, bool NT>
__global__ __launch_bounds__(kQuantThreads) void k_quant_row16(const T *__restrict__ x, int64_t rows, int64_t bpr,
                                                               int64_t ldx, const float *__restrict__ amax_src,
                                                               int n_amax, uint8_t *__restrict__ codes,
                                                               uint8_t *__restrict__ scales,
                                                               float *__restrict__ alpha_out)
{
    __shared__ float ktab[128];
    const int64_t nb = rows * bpr;
    const bool flat = ldx == bpr * 16;
    const int64_t b0 = (int64_t)blockIdx.x * (kQuantThreads * kRowBlocks) + threadIdx.x;
    // partial load, then the data loads; alpha and the kappa table are set up
    // while the data is in flight.  The data loads are unconditional (a lane
    // past the end re-reads the last block and stores nothing) and the raw
    // words are only unpacked after the table is built: a load under a
    // branch, or a use of its value, would be waited for right there.
    constexpr int kVec = (int)sizeof(T);                  // 16-byte vectors per block
    const float apart = alpha_issue<NPT>(amax_src, n_amax);
    uint4 raw[kRowBlocks][kVec];
#pragma unroll
    for (int j = 0; j < kRowBlocks; j++) {
        const int64_t b = b0 + j * kQuantThreads < nb ? b0 + j * kQuantThreads : nb - 1;   // nb >= 1
        int64_t off;
        if (flat) {
            off = b * 16;
        } else {
            const int64_t r = b / bpr;
            off = r * ldx + (b - r * bpr) * 16;
        }
        const uint4 *src = reinterpret_cast<const uint4 *>(x + off);
#pragma unroll
        for (int u = 0; u < kVec; u++)
            raw[j][u] = NT ? load_stream(src + u) : src[u];
    }
    const float alpha = alpha_finish(apart, amax_src, n_amax);
    build_kappa_table(ktab, alpha);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *alpha_out = alpha;
#pragma unroll
    for (int j = 0; j < kRowBlocks; j++) {
        const int64_t b = b0 + j * kQuantThreads;
        if (b < nb) {
            float v[16];
            unpack16<T>(raw[j], v);
            uint32_t c0, c1, sb;
            quant_block16<RULE4>(v, alpha, ktab, c0, c1, sb);
            store_block_stream(codes + b * 8, scales + b, c0, c1, sb);
        }
    }
}

// ------------------------------------------------ COL16 (1D, along rows)

// Blocks of 16 consecutive rows of one column; output is the ROW16 packing of
// x^T: codes [cols][rows/2], scales [cols][rows/16].  A workgroup owns
// kColCols columns (two per lane) and walks groups of kColGroupRB row-blocks:
// each wave loads the 16 rows of one row-block for its lane's two columns
// straight into registers (the block is then lane-local), quantizes them, and
// parks codes and scales in LDS; once a group is done the workgroup writes
// each column's codes (8 bytes per row-block) and scales as contiguous runs.
constexpr int kColCols = 128;                       // columns per workgroup
constexpr int kColGroupRB = 16;                     // row-blocks per group (4 waves x 4 steps)
constexpr int kColCodePitch = kColGroupRB * 8 + 16; // LDS bytes per column of parked codes

template <typename T, bool RULE4, bool RHT, bool PAIR>
__global__ __launch_bounds__(kQuantThreads) void k_quant_col16(const T *__restrict__ x, int64_t rows, int64_t cols,
                                                               int64_t ldx, const float *__restrict__ amax_src,
                                                               int n_amax, uint8_t *__restrict__ codes,
                                                               uint8_t *__restrict__ scales,
                                                               float *__restrict__ alpha_out, uint32_t signs)
{
    constexpr int kWaves = kQuantThreads / 64;
    constexpr int kSteps = kColGroupRB / kWaves;
    __shared__ float ktab[128];
    __shared__ __attribute__((aligned(16))) uint8_t cpark[kColCols * kColCodePitch];
    __shared__ __attribute__((aligned(16))) uint8_t spark[kColCols * kColGroupRB];

    const float apart = alpha_issue(amax_src, n_amax);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t nrb = rows / 16;
    const int64_t col0 = (int64_t)blockIdx.x * kColCols;
    const int64_t c = col0 + 2 * lane;                  // this lane's first column
    const bool c0ok = c < cols, c1ok = c + 1 < cols;
    // PAIR (chosen by the launcher: even column count, ldx and x aligned to a
    // pair): both columns in one 2-element vector load, with no branch at all,
    // so that the loads stay in flight across the alpha set-up
    const int64_t cp = c0ok ? c : cols - 2;             // lanes past the last column re-read the last pair

    // the 16 rows x 2 columns of row-block rb, as 16 packed pairs; a row-block
    // past the end re-reads the last one (nrb >= 1; its results are not stored)
    typedef typename std::conditional<sizeof(T) == 2, uint32_t, uint2>::type Pair;
    auto load_block = [&](int64_t rb, Pair (&v)[16]) {
        rb = rb < nrb ? rb : nrb - 1;
        if constexpr (PAIR) {
            const T *p = x + rb * 16 * ldx + cp;
#pragma unroll
            for (int i = 0; i < 16; i++)
                v[i] = *reinterpret_cast<const Pair *>(p + i * ldx);
        } else {
            const T *p = x + rb * 16 * ldx + c;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                T e[2] = {T(0), T(0)};
                if (c0ok)
                    e[0] = p[i * ldx];
                if (c1ok)
                    e[1] = p[i * ldx + 1];
                v[i] = __builtin_bit_cast(Pair, e);
            }
        }
    };

    // the first group's first row-block is in flight while alpha and the
    // kappa table are set up
    Pair v[2][16];
    const int64_t gfirst = (int64_t)blockIdx.y * kColGroupRB;
    load_block(gfirst + wave, v[0]);                    // gfirst < nrb: grid.y <= the group count
    const float alpha = alpha_finish(apart, amax_src, n_amax);
    build_kappa_table(ktab, alpha);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        *alpha_out = alpha;

    static_assert(kSteps % 2 == 0, "the next group's first row-block goes to v[0]");
    const int64_t gstride = (int64_t)gridDim.y * kColGroupRB;
    for (int64_t g0 = gfirst; g0 < nrb; g0 += gstride) {
        const int ng = nrb - g0 < kColGroupRB ? (int)(nrb - g0) : kColGroupRB;
        int64_t rb = g0 + wave;
#pragma unroll
        for (int st = 0; st < kSteps; st++) {
            const int slot = st * kWaves + wave;            // row-block index inside the group
            // every step prefetches the next one; the last step prefetches the
            // next group's first row-block, or re-reads its own (a cache hit)
            if (st + 1 < kSteps) {
                load_block(rb + kWaves, v[(st + 1) & 1]);
            } else {
                const int64_t nx = g0 + gstride + wave;
                load_block(nx < nrb ? nx : rb, v[0]);
            }
            if (slot < ng) {
#pragma unroll
                for (int k = 0; k < 2; k++) {
                    float f[16];
#pragma unroll
                    for (int i = 0; i < 16; i++) {
                        if constexpr (sizeof(T) == 2)
                            f[i] = k == 0 ? bf16_lo(v[st & 1][i]) : bf16_hi(v[st & 1][i]);
                        else
                            f[i] = __uint_as_float(k == 0 ? v[st & 1][i].x : v[st & 1][i].y);
                    }
                    if (RHT)
                        rht16(f, signs);
                    uint32_t q0, q1, sb;
                    quant_block16<RULE4>(f, alpha, ktab, q0, q1, sb);
                    const int cc = 2 * lane + k;
                    *reinterpret_cast<uint2 *>(&cpark[cc * kColCodePitch + slot * 8]) = make_uint2(q0, q1);
                    spark[cc * kColGroupRB + slot] = (uint8_t)sb;
                }
            }
            rb += kWaves;
        }
        __syncthreads();
        // each column's run: ng*8 code bytes, ng scale bytes
        const int ncol = cols - col0 < kColCols ? (int)(cols - col0) : kColCols;
        const int64_t cstride = rows / 2;
        for (int q = tid; q < ncol * kColGroupRB; q += kQuantThreads) {
            const int cc = q / kColGroupRB, part = q - cc * kColGroupRB;
            if (part < ng) {
                *reinterpret_cast<uint2 *>(codes + (col0 + cc) * cstride + g0 * 8 + part * 8) =
                    *reinterpret_cast<const uint2 *>(&cpark[cc * kColCodePitch + part * 8]);
                scales[(col0 + cc) * nrb + g0 + part] = spark[cc * kColGroupRB + part];
            }
        }
        __syncthreads();    // the parking area is refilled by the next group
    }
}

// amax of the transformed COL16 blocks: each lane takes a pair of columns and
// one row-block per task (16 rows, consecutive lanes on consecutive pairs).
template <typename T>
__global__ __launch_bounds__(kAmaxThreads) void k_amax_col16_rht(const T *__restrict__ x, int64_t rows, int64_t cols,
                                                                 int64_t ldx, uint32_t signs,
                                                                 float *__restrict__ partials)
{
    __shared__ float red[kAmaxThreads / 64];
    typedef typename std::conditional<sizeof(T) == 2, uint32_t, uint2>::type Pair;
    const int64_t pairs = (cols + 1) / 2, nrb = rows / 16;
    const int64_t tasks = pairs * nrb;
    const bool vec = cols % 2 == 0 && ldx % 2 == 0 && reinterpret_cast<uintptr_t>(x) % (2 * sizeof(T)) == 0;
    float a = 0.0f;
    for (int64_t t = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x; t < tasks;
         t += (int64_t)gridDim.x * kAmaxThreads) {
        const int64_t rb = t / pairs, cp = t - rb * pairs;
        const int64_t c = 2 * cp;
        const T *p = x + rb * 16 * ldx + c;
        Pair v[16];
        if (vec) {
#pragma unroll
            for (int i = 0; i < 16; i++)
                v[i] = *reinterpret_cast<const Pair *>(p + i * ldx);
        } else {
#pragma unroll
            for (int i = 0; i < 16; i++) {
                T e[2] = {p[i * ldx], T(0)};
                if (c + 1 < cols)
                    e[1] = p[i * ldx + 1];
                v[i] = __builtin_bit_cast(Pair, e);
            }
        }
#pragma unroll
        for (int k = 0; k < 2; k++) {
            float f[16];
#pragma unroll
            for (int i = 0; i < 16; i++) {
                if constexpr (sizeof(T) == 2)
                    f[i] = k == 0 ? bf16_lo(v[i]) : bf16_hi(v[i]);
                else
                    f[i] = __uint_as_float(k == 0 ? v[i].x : v[i].y);
            }
            rht16(f, signs);
#pragma unroll
            for (int i = 0; i < 16; i++)
                a = fmaxf(a, fabsf(f[i]));
        }
    }
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = red[0];
#pragma unroll
        for (int w = 1; w < kAmaxThreads / 64; w++)
            b = fmaxf(b, red[w]);
        partials[blockIdx.x] = b;
    }
}

// ---------------------------------------------------- TILE16 (16x16, weights)

// Groups of 16 lanes own one tile; lane j of a group holds tile row j.  The
// block error is the sum, in row order, of the per-row fma chains.
template <typename T, bool RULE4>
__global__ __launch_bounds__(kQuantThreads) void k_quant_tile16(const T *__restrict__ x, int64_t rows, int64_t cols,
                                                                int64_t ldx, const float *__restrict__ amax_src,
                                                                int n_amax, uint8_t *__restrict__ codes,
                                                                uint8_t *__restrict__ scales,
                                                                float *__restrict__ alpha_out)
{
    __shared__ float ktab[128];
    const float alpha = alpha_finish(alpha_issue(amax_src, n_amax), amax_src, n_amax);
    build_kappa_table(ktab, alpha);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        *alpha_out = alpha;
    const int lane16 = threadIdx.x & 15;
    const int64_t tb = (int64_t)blockIdx.x * (kQuantThreads / 16) + (threadIdx.x >> 4);   // tile column
    const int64_t tpr = cols / 16;
    // whole 16-lane groups leave together, so the shuffles below stay inside
    // fully active groups
    if (tb >= tpr)
        return;
    for (int64_t rb = blockIdx.y; rb < rows / 16; rb += gridDim.y) {     // tile row
        const int64_t r = rb * 16 + lane16;
        float v[16];
        load16(x + r * ldx + tb * 16, v);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++)
            m = fmaxf(m, fabsf(v[i]));
#pragma unroll
        for (int o = 8; o > 0; o >>= 1)
            m = fmaxf(m, __shfl_xor(m, o, 16));
        const uint32_t sb = block_scale_bytes(m, alpha, ktab);
        const float s6 = e4m3_get<0>(sb);
        uint32_t c0, c1;
        float er = 0.0f;
        encode16(v, s6, ktab[sb & 0xffu], alpha, c0, c1, er);
        float e6 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++)
            e6 = e6 + __shfl(er, i, 16);
        uint32_t sbyte = sb & 0xffu;
        if (RULE4) {
            const float s4 = e4m3_get<1>(sb);
            uint32_t d0, d1;
            float er4 = 0.0f;
            encode16(v, s4, ktab[(sb >> 8) & 0xffu], alpha, d0, d1, er4);
            float e4 = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; i++)
                e4 = e4 + __shfl(er4, i, 16);
            if (e4 < e6) {
                c0 = d0;
                c1 = d1;
                sbyte = (sb >> 8) & 0xffu;
            }
        }
        *reinterpret_cast<uint2 *>(codes + r * (cols / 2) + tb * 8) = make_uint2(c0, c1);
        if (lane16 == 0)
            scales[rb * tpr + tb] = (uint8_t)sbyte;
    }
}

// ------------------------------------------------------------ dequantize

template <typename O>
__device__ __forceinline__ void store1(O *p, float v);
template <>
__device__ __forceinline__ void store1<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store1<uint16_t>(uint16_t *p, float v)
{
    __bf16 h = (__bf16)v;                  // round to nearest even
    *p = __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ void decode16(uint32_t c0, uint32_t c1, float s, float alpha, float (&y)[16])
{
    float2v t;
    uint32_t w[2] = {c0, c1};
#pragma unroll
    for (int h = 0; h < 2; h++) {
        t = e2m1_get2<0>(w[h]); y[8 * h + 0] = t[0]; y[8 * h + 1] = t[1];
        t = e2m1_get2<1>(w[h]); y[8 * h + 2] = t[0]; y[8 * h + 3] = t[1];
        t = e2m1_get2<2>(w[h]); y[8 * h + 4] = t[0]; y[8 * h + 5] = t[1];
        t = e2m1_get2<3>(w[h]); y[8 * h + 6] = t[0]; y[8 * h + 7] = t[1];
    }
#pragma unroll
    for (int i = 0; i < 16; i++)
        y[i] = (y[i] * s) * alpha;
}

// ROW16 / TILE16: one lane per 16-element row segment.
// The 16 outputs of a lane as 16-byte pieces: 2 (bf16, round to nearest even)
// or 4 (fp32).
template <typename O>
__device__ __forceinline__ void pack16(const float (&v)[16], uint4 (&pc)[sizeof(O)])
{
    if constexpr (sizeof(O) == 4) {
#pragma unroll
        for (int i = 0; i < 4; i++)
            pc[i] = make_uint4(__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]), __float_as_uint(v[4 * i + 2]),
                               __float_as_uint(v[4 * i + 3]));
    } else {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            __bf16 lo = (__bf16)v[2 * i], hi = (__bf16)v[2 * i + 1];
            w[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        pc[0] = make_uint4(w[0], w[1], w[2], w[3]);
        pc[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
}

// Workgroup-wide store of one 16-element output row per lane, the rows of
// consecutive lanes consecutive in memory from `out` on: the pieces go
// through LDS so that every store instruction of a wave writes one contiguous
// 1 KiB run, non-temporal (a lane's own 32 or 64 bytes at a 32- or 64-byte
// stride store measurably slower, and so do the same runs as ordinary
// stores).  n_valid: how many of the workgroup's rows exist (a prefix).
// Every thread of the workgroup must call it (it synchronizes).
template <typename O>
__device__ __forceinline__ void store16_staged(O *out, const float (&v)[16], int n_valid, uint4 *stage)
{
    constexpr int P = (int)sizeof(O);                   // 16-byte pieces per row
    uint4 pc[P];
    pack16<O>(v, pc);
#pragma unroll
    for (int j = 0; j < P; j++)
        stage[threadIdx.x * P + j] = pc[j];
    __syncthreads();
    const int w0 = (int)(threadIdx.x & ~63u) * P;       // first piece of this wave's rows
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < P; j++) {
        const int piece = w0 + j * 64 + lane;
        if (piece < n_valid * P)
            store16_stream(reinterpret_cast<uint4 *>(out) + piece, stage[piece]);
    }
}

template <typename O, bool TILE>
__global__ __launch_bounds__(kQuantThreads) void k_dequant_rows(const uint8_t *__restrict__ codes,
                                                                const uint8_t *__restrict__ scales,
                                                                const float *__restrict__ alpha_p, int64_t rows,
                                                                int64_t bpr, O *__restrict__ y, int64_t ldy)
{
    __shared__ uint4 stage[kQuantThreads * sizeof(O)];
    const int64_t nb = rows * bpr;
    const int64_t b0 = (int64_t)blockIdx.x * kQuantThreads;
    const int64_t b = b0 + threadIdx.x;
    const bool flat = !TILE && ldy == bpr * 16;
    if (!flat && b >= nb)
        return;
    const int64_t bc = b < nb ? b : nb - 1;             // past the end: re-read the last block, store nothing
    const float alpha = *alpha_p;
    // 32-bit division while the block index fits (every tensor here does)
    const int64_t r = bc < 0x7fffffff ? (int64_t)((uint32_t)bc / (uint32_t)bpr) : bc / bpr;
    const int64_t cb = bc - r * bpr;
    const uint2 c = *reinterpret_cast<const uint2 *>(codes + bc * 8);
    const int64_t soff = TILE ? (r / 16) * bpr + cb : bc;
    const float s = e4m3_get<0>(scales[soff]);
    float v[16];
    decode16(c.x, c.y, s, alpha, v);
    if (flat) {                                         // workgroup-uniform
        const int64_t left = nb - b0;
        store16_staged<O>(y + b0 * 16, v, left < kQuantThreads ? (int)left : kQuantThreads, stage);
    } else {
        uint4 pc[sizeof(O)];
        pack16<O>(v, pc);
        uint4 *out = reinterpret_cast<uint4 *>(y + r * ldy + cb * 16);
#pragma unroll
        for (int j = 0; j < (int)sizeof(O); j++)
            out[j] = pc[j];
    }
}

// COL16: lanes take consecutive columns of the original [rows][cols] tensor.
template <typename O>
__global__ __launch_bounds__(kQuantThreads) void k_dequant_col16(const uint8_t *__restrict__ codes,
                                                                 const uint8_t *__restrict__ scales,
                                                                 const float *__restrict__ alpha_p, int64_t rows,
                                                                 int64_t cols, O *__restrict__ y, int64_t ldy)
{
    const int64_t idx = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    const int64_t nrb = rows / 16;
    if (idx >= cols * nrb)
        return;
    const float alpha = *alpha_p;
    const int64_t rb = idx / cols;
    const int64_t c = idx - rb * cols;
    const uint2 cw = *reinterpret_cast<const uint2 *>(codes + c * (rows / 2) + rb * 8);
    const float s = e4m3_get<0>(scales[c * nrb + rb]);
    float v[16];
    decode16(cw.x, cw.y, s, alpha, v);
#pragma unroll
    for (int i = 0; i < 16; i++)
        store1<O>(y + (rb * 16 + i) * ldy + c, v[i]);
}

// ------------------------------------------------ KV cache: key smoothing

// Key smoothing ("Key smoothing", NVFP4 Inference section of the architecture
// walkthrough page): each key vector of d = head_dim elements loses its mean
// over d.  fp32 order (shared with the quantize pass below): each 16-element
// block's partial sum in index order, the d/16 partials added in block order,
// mean = sum / d, key[u] - mean.  G = d/16 lanes hold one vector (one block
// each); the partials travel by shuffles, so every lane of the group forms the
// same sum in the same order.
template <typename T>
__global__ __launch_bounds__(kAmaxThreads) void k_kv_smooth_amax(const T *__restrict__ x, int64_t vectors, int g_log2,
                                                                 float *__restrict__ means,
                                                                 float *__restrict__ partials)
{
    __shared__ float red[kAmaxThreads / 64];
    const int G = 1 << g_log2;
    const int64_t d = (int64_t)G * 16;
    const int lane = threadIdx.x & 63;
    const int j = lane & (G - 1), base = lane - j;
    float a = 0.0f;
    const int64_t per_iter = ((int64_t)gridDim.x * kAmaxThreads) >> g_log2;
    for (int64_t v = (((int64_t)blockIdx.x * kAmaxThreads + threadIdx.x) >> g_log2); v < vectors; v += per_iter) {
        float f[16];
        load16(x + v * d + j * 16, f);
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++)
            p = p + f[i];
        float sum = 0.0f;
        for (int b = 0; b < G; b++)
            sum = sum + __shfl(p, base + b, 64);
        const float mean = sum / (float)d;
        if (j == 0)
            means[v] = mean;
#pragma unroll
        for (int i = 0; i < 16; i++)
            a = fmaxf(a, fabsf(f[i] - mean));
    }
    a = wave_max(a);
    if (lane == 0)
        red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = red[0];
#pragma unroll
        for (int w = 1; w < kAmaxThreads / 64; w++)
            b = fmaxf(b, red[w]);
        partials[blockIdx.x] = b;
    }
}

// Quantize the smoothed keys: one lane per 16-element block, the vector's mean
// (written by the pass above) subtracted first.
template <typename T, bool RULE4>
__global__ __launch_bounds__(kQuantThreads) void k_kv_quant_smoothed(const T *__restrict__ x, int64_t vectors, int g_log2,
                                                                     const float *__restrict__ means,
                                                                     const float *__restrict__ amax_src, int n_amax,
                                                                     uint8_t *__restrict__ codes,
                                                                     uint8_t *__restrict__ scales,
                                                                     float *__restrict__ alpha_out)
{
    __shared__ float ktab[128];
    const int64_t nb = vectors << g_log2;
    const int64_t b = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    const float apart = alpha_issue(amax_src, n_amax);
    // data and mean loads without a branch (a lane past the end re-reads the
    // last block and stores nothing; nb >= 1), unpacked only after alpha and
    // the kappa table, as in k_quant_row16
    const int64_t bc = b < nb ? b : nb - 1;
    uint4 raw[sizeof(T)];
    const uint4 *src = reinterpret_cast<const uint4 *>(x + bc * 16);
#pragma unroll
    for (int u = 0; u < (int)sizeof(T); u++)
        raw[u] = src[u];
    const float mean = means[bc >> g_log2];
    const float alpha = alpha_finish(apart, amax_src, n_amax);
    build_kappa_table(ktab, alpha);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *alpha_out = alpha;
    if (b >= nb)
        return;
    float f[16];
    unpack16<T>(raw, f);
#pragma unroll
    for (int i = 0; i < 16; i++)
        f[i] = f[i] - mean;
    uint32_t c0, c1, sb;
    quant_block16<RULE4>(f, alpha, ktab, c0, c1, sb);
    store_block_stream(codes + b * 8, scales + b, c0, c1, sb);
}

// ------------------------------------------------ KV cache: window dequantize

// One launch reconstructs the attention window from several cached chunks
// ("Parallel CUDA dequantization kernel" paragraph: chunks of the active window
// dequantized together into the window buffer): segment i contributes rows
// [first, first + count) of its chunk, in segment order.  One lane per 16
// elements; the vector's mean is added back for smoothed keys.
// Store 16 fp32 values as fp32 or bf16 (round to nearest even), one lane's
// own 32 or 64 bytes.
template <typename O>
__device__ __forceinline__ void store16(O *out, const float (&v)[16])
{
    uint4 pc[sizeof(O)];
    pack16<O>(v, pc);
#pragma unroll
    for (int j = 0; j < (int)sizeof(O); j++)
        reinterpret_cast<uint4 *>(out)[j] = pc[j];
}

// Each workgroup serves one segment (the host gives segment i the workgroups
// [wg0_i, wg0_{i+1})), so the segment's pointers are uniform; one lane per
// 16-element block of the segment's rows.
template <typename O>
__global__ __launch_bounds__(kQuantThreads) void k_kv_window(KvWindowArgs a, O *__restrict__ y, int64_t ldy)
{
    __shared__ uint4 stage[kQuantThreads * sizeof(O)];
    const int wg = blockIdx.x;
    int si = 0;
    while (si + 1 < a.n && wg >= a.seg[si + 1].wg0)
        si++;
    const KvSegmentDev &sg = a.seg[si];
    const uint32_t bpr = (uint32_t)a.bpr;
    // count * bpr < 2^31 (checked by the caller): 32-bit index arithmetic
    const uint32_t n = (uint32_t)sg.count * bpr;
    const uint32_t local0 = (uint32_t)(wg - sg.wg0) * kQuantThreads;
    const uint32_t local = local0 + threadIdx.x;
    // dense output rows: the segment's rows are one contiguous run of the
    // window buffer, stored through LDS (workgroup-uniform)
    const bool flat = ldy == a.bpr * 16;
    if (!flat && local >= n)
        return;
    const uint32_t lc = local < n ? local : n - 1;   // past the end: re-read the last block, store nothing
    const uint32_t r = lc / bpr;
    const int cb = (int)(lc - r * bpr);
    const int64_t v = sg.first + r;
    const int64_t blk = v * bpr + cb;
    // the key mean is loaded with the codes and the scale (a segment without
    // means reads alpha instead and ignores it): loaded under the branch, it
    // would only be issued once the decode had waited for the others
    const float *mp = sg.means ? sg.means + v : sg.alpha;
    const uint2 c = *reinterpret_cast<const uint2 *>(sg.codes + blk * 8);
    const uint32_t sb = sg.scales[blk];
    const float m = *mp;
    __builtin_amdgcn_sched_barrier(0);         // all three loads issued before the decode
    float val[16];
    decode16(c.x, c.y, e4m3_get<0>(sb), *sg.alpha, val);
    if (sg.means) {
#pragma unroll
        for (int i = 0; i < 16; i++)
            val[i] = val[i] + m;
    }
    if (flat) {
        const uint32_t left = n - local0;
        store16_staged<O>(y + sg.out_row * ldy + (int64_t)local0 * 16, val,
                          left < (uint32_t)kQuantThreads ? (int)left : kQuantThreads, stage);
    } else {
        store16(y + (sg.out_row + r) * ldy + cb * 16, val);
    }
}

// ------------------------------------- KV cache: one global scale per chunk

// KV caches of heads x tokens key (or value) vectors, [tensors][heads][tokens][d]
// (e.g. K and V of a layer as two tensors), with one global scale per tensor
// and chunk of tokens_per_chunk tokens ("Chunkwise quantization procedure": a
// per-chunk, per-layer FP32 global scale).  Chunk c of tensor u holds tokens
// [c*tpc, min((c+1)*tpc, tokens)) of every head of u, i.e. `heads` contiguous
// row segments of the [tensors*heads*tokens][d] view.  Unit z = u * nch + c
// (grid z) indexes the scales, the amax partials and chunk_amax.
struct KvChunks {
    int64_t tokens, tpc;      // tokens, tokens per chunk
    int64_t d;                // head_dim
    int64_t heads;
    int nch;                  // chunks per tensor
    int pseg;                 // amax workgroups per (unit, head) segment
    uint64_t nch_magic;       // ceil(2^32 / nch): z / nch == (z * nch_magic) >> 32 for every z < 2^16
};

inline uint64_t kv_nch_magic(int64_t nch) { return ((1ull << 32) + (uint64_t)nch - 1) / (uint64_t)nch; }

// The head-h segment of unit z (z < 2^16): its first row and its row count.
// The unit's tensor and chunk come from a multiply and shift (checked against
// division for every z < 2^16 and every chunk count below 2^16) instead of an
// integer division, which would hold up the workgroup's first loads.
__device__ __forceinline__ void unit_segment(const KvChunks &k, int z, int h, int64_t &row0, int64_t &len)
{
    const int u = (int)(((uint64_t)(uint32_t)z * k.nch_magic) >> 32);
    const int c = z - u * k.nch;
    const int64_t t0 = (int64_t)c * k.tpc;
    len = k.tokens - t0 < k.tpc ? k.tokens - t0 : k.tpc;
    row0 = ((int64_t)u * k.heads + h) * k.tokens + t0;
}

// Partial maxima: workgroup (p, h, z) reduces part p of the head-h segment of
// unit z into partials[z * heads * pseg + h * pseg + p]: one contiguous range
// of the segment per workgroup, eight streaming 16-byte loads in flight per
// thread.
template <typename T>
__global__ __launch_bounds__(kAmaxThreads) void k_amax_kv_chunked(const T *__restrict__ x, KvChunks k,
                                                                  float *__restrict__ partials)
{
    __shared__ float red[kAmaxThreads / 64];
    constexpr int V = 16 / sizeof(T);
    const int p = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
    int64_t row0, len;
    unit_segment(k, z, h, row0, len);
    const int64_t nv = len * k.d / V;                                   // d % 16 == 0: whole vectors
    const uint4 *xv = reinterpret_cast<const uint4 *>(x + row0 * k.d);
    const int64_t per_wg = ((nv + k.pseg - 1) / k.pseg + kAmaxThreads - 1) / kAmaxThreads * kAmaxThreads;
    const int64_t beg = (int64_t)p * per_wg;
    const int64_t end = beg + per_wg < nv ? beg + per_wg : nv;
    constexpr int64_t kIter = (int64_t)kAmaxThreads * kAmaxUnroll;
    float a = 0.0f;
    for (int64_t base = beg; base < end; base += kIter) {
        uint4 v[kAmaxUnroll];
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; u++) {
            const int64_t i = base + u * kAmaxThreads + threadIdx.x;
            v[u] = i < end ? load_stream(xv + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; u++)
            a = absmax16B<T>(v[u], a);
    }
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = red[0];
#pragma unroll
        for (int w = 1; w < kAmaxThreads / 64; w++)
            b = fmaxf(b, red[w]);
        partials[((int64_t)z * gridDim.y + h) * k.pseg + p] = b;
    }
}

// Quantize: workgroup (bx, h, z) takes 256 consecutive 16-element blocks of
// the head-h segment of unit z, one per lane, with unit z's alpha (from its
// n_amax partials at amax_src + z * amax_stride); otherwise as k_quant_row16.
template <typename T, bool RULE4, int NPT>
__global__ __launch_bounds__(kQuantThreads) void k_quant_kv_chunked(const T *__restrict__ x, KvChunks k,
                                                                    const float *__restrict__ amax_src,
                                                                    int64_t amax_stride, int n_amax,
                                                                    uint8_t *__restrict__ codes,
                                                                    uint8_t *__restrict__ scales,
                                                                    float *__restrict__ alphas)
{
    __shared__ float ktab[128];
    const int h = blockIdx.y, z = blockIdx.z;
    const int64_t bpr = k.d / 16;
    int64_t row0, len;
    unit_segment(k, z, h, row0, len);
    const int64_t nb = len * bpr;                             // blocks of this segment
    const int64_t b0 = (int64_t)blockIdx.x * kQuantThreads;
    if (b0 >= nb)
        return;                                               // the whole workgroup: past a short last chunk
    const float *src = amax_src + (int64_t)z * amax_stride;
    const float apart = alpha_issue<NPT>(src, n_amax);
    const int64_t seg0 = row0 * bpr;                          // first block of the segment
    const int64_t bl = b0 + threadIdx.x;
    const int64_t b = seg0 + (bl < nb ? bl : nb - 1);         // past the end: re-read the last block
    constexpr int kVec = (int)sizeof(T);
    uint4 raw[kVec];
    const uint4 *p = reinterpret_cast<const uint4 *>(x + b * 16);
#pragma unroll
    for (int u = 0; u < kVec; u++)
        raw[u] = load_stream(p + u);
    const float alpha = alpha_finish(apart, src, n_amax);
    build_kappa_table(ktab, alpha);
    if (blockIdx.x == 0 && h == 0 && threadIdx.x == 0)
        alphas[z] = alpha;
    if (bl < nb) {
        float v[16];
        unpack16<T>(raw, v);
        uint32_t c0, c1, sb;
        quant_block16<RULE4>(v, alpha, ktab, c0, c1, sb);
        store_block_stream(codes + b * 8, scales + b, c0, c1, sb);
    }
}

// Dequantize a chunked KV tensor: one lane per 16-element block, alpha of the
// block's chunk.
template <typename O>
__global__ __launch_bounds__(kQuantThreads) void k_dequant_kv_chunked(const uint8_t *__restrict__ codes,
                                                                      const uint8_t *__restrict__ scales,
                                                                      const float *__restrict__ alphas, KvChunks k,
                                                                      int64_t nblocks, O *__restrict__ y)
{
    __shared__ uint4 stage[kQuantThreads * sizeof(O)];
    const int64_t b0 = (int64_t)blockIdx.x * kQuantThreads;
    const int64_t b = b0 + threadIdx.x;
    const int64_t bc = b < nblocks ? b : nblocks - 1;        // past the end: re-read the last block, store nothing
    const int64_t bpr = k.d / 16;
    const int64_t row = bc / bpr;
    const int64_t ht = row / k.tokens;                        // tensor * heads + head
    const int64_t t = row - ht * k.tokens;
    const uint2 cw = *reinterpret_cast<const uint2 *>(codes + bc * 8);
    const float s = e4m3_get<0>(scales[bc]);
    const float alpha = alphas[(ht / k.heads) * k.nch + t / k.tpc];
    float v[16];
    decode16(cw.x, cw.y, s, alpha, v);
    const int64_t left = nblocks - b0;
    store16_staged<O>(y + b0 * 16, v, left < kQuantThreads ? (int)left : kQuantThreads, stage);
}

// ------------------------------------------------------------ launchers

int amax_partials(int64_t rows, int64_t cols)
{
    // enough workgroups to cover every CU even for small tensors: about one
    // 16-byte vector per thread per workgroup, at most kMaxAmaxPartials (more
    // partials cost the quantizer more than they gain the amax pass)
    const int64_t n = rows * cols;
    const int64_t per_wg = (int64_t)kAmaxThreads * 8;
    int64_t p = (n + per_wg - 1) / per_wg;
    if (p < 1) p = 1;
    if (p > kMaxAmaxPartials) p = kMaxAmaxPartials;
    return (int)p;
}

hipError_t launch_amax(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, float *partials,
                       int n_partials, hipStream_t s)
{
    // the flat vector path needs whole 16-byte vectors: entry points that take
    // element-aligned inputs (COL16, WGRAD) fall back to the row loop
    const bool vec = ldx == cols && (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
    const bool nt = rows * cols * (dtype == 1 ? 2 : 4) >= kStreamLoadBytes;
    auto go = [&](auto kernel, auto xt) {
        kernel<<<n_partials, kAmaxThreads, 0, s>>>(xt, rows, cols, ldx, vec, partials);
    };
    if (dtype == 1)
        nt ? go(k_amax<uint16_t, kAmaxThreads, 4, true>, (const uint16_t *)x)
           : go(k_amax<uint16_t, kAmaxThreads, 4, false>, (const uint16_t *)x);
    else
        nt ? go(k_amax<float, kAmaxThreads, 4, true>, (const float *)x)
           : go(k_amax<float, kAmaxThreads, 4, false>, (const float *)x);
    return hipGetLastError();
}

template <typename T, bool R4>
static void launch_quant_t(const T *x, int64_t rows, int64_t cols, int64_t ldx, int block, const float *amax_src,
                           int n_amax, uint8_t *codes, uint8_t *scales, float *alpha, hipStream_t s, int rht_signs)
{
    if (block == 0) {
        const int64_t bpr = cols / 16;
        const int64_t nb = rows * bpr;
        const int64_t per_wg = (int64_t)kQuantThreads * kRowBlocks;
        const unsigned grid = (unsigned)((nb + per_wg - 1) / per_wg);
        const bool nt = rows * cols * (int64_t)sizeof(T) >= kStreamLoadBytes;
        auto go = [&](auto kernel) {
            kernel<<<grid, kQuantThreads, 0, s>>>(x, rows, bpr, ldx, amax_src, n_amax, codes, scales, alpha);
        };
        constexpr int kNpt4 = kMaxAmaxSrc / kQuantThreads;
        if (n_amax > kQuantThreads)             // up to kMaxAmaxSrc partials (four per thread)
            nt ? go(k_quant_row16<T, R4, kNpt4, true>) : go(k_quant_row16<T, R4, kNpt4, false>);
        else
            nt ? go(k_quant_row16<T, R4, 1, true>) : go(k_quant_row16<T, R4, 1, false>);
    } else if (block == 1) {
        const int64_t tpr = cols / 16;
        const int64_t ty = rows / 16 < 65535 ? rows / 16 : 65535;
        dim3 grid((unsigned)((tpr + kQuantThreads / 16 - 1) / (kQuantThreads / 16)), (unsigned)ty);
        k_quant_tile16<T, R4><<<grid, kQuantThreads, 0, s>>>(x, rows, cols, ldx, amax_src, n_amax, codes, scales, alpha);
    } else {
        const int64_t nrb = rows / 16;
        // about seven resident workgroups per CU; groups spread evenly over grid.y
        const int64_t gx = (cols + kColCols - 1) / kColCols;
        const int64_t ngroups = (nrb + kColGroupRB - 1) / kColGroupRB;
        const int64_t want = (1792 + gx - 1) / gx;
        const int64_t per = (ngroups + want - 1) / want;
        int64_t gy = (ngroups + per - 1) / per;
        if (gy > 65535) gy = 65535;
        if (gy < 1) gy = 1;
        dim3 grid((unsigned)gx, (unsigned)gy);
        const bool pair = cols % 2 == 0 && ldx % 2 == 0 && reinterpret_cast<uintptr_t>(x) % (2 * sizeof(T)) == 0;
        const uint32_t signs = rht_signs >= 0 ? (uint32_t)rht_signs : 0u;
        auto go = [&](auto kernel) {
            kernel<<<grid, kQuantThreads, 0, s>>>(x, rows, cols, ldx, amax_src, n_amax, codes, scales, alpha, signs);
        };
        if (rht_signs >= 0)
            pair ? go(k_quant_col16<T, R4, true, true>) : go(k_quant_col16<T, R4, true, false>);
        else
            pair ? go(k_quant_col16<T, R4, false, true>) : go(k_quant_col16<T, R4, false, false>);
    }
}

hipError_t launch_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int block, int rule,
                           const float *amax_src, int n_amax, uint8_t *codes, uint8_t *scales, float *alpha,
                           hipStream_t s, int rht_signs)
{
    // the kernels read at most kMaxAmaxSrc partials (ROW16) or kQuantThreads (the others)
    if (n_amax < 1 || n_amax > (block == 0 ? kMaxAmaxSrc : kQuantThreads))
        return hipErrorInvalidValue;
    if (rows == 0 || cols == 0) {
        // nothing to encode; alpha still follows the rule (amax 0 -> 1)
        k_alpha_only<<<1, kQuantThreads, 0, s>>>(amax_src, n_amax, alpha);
        return hipGetLastError();
    }
    if (dtype == 1) {
        if (rule) launch_quant_t<uint16_t, true>((const uint16_t *)x, rows, cols, ldx, block, amax_src, n_amax, codes, scales, alpha, s, rht_signs);
        else      launch_quant_t<uint16_t, false>((const uint16_t *)x, rows, cols, ldx, block, amax_src, n_amax, codes, scales, alpha, s, rht_signs);
    } else {
        if (rule) launch_quant_t<float, true>((const float *)x, rows, cols, ldx, block, amax_src, n_amax, codes, scales, alpha, s, rht_signs);
        else      launch_quant_t<float, false>((const float *)x, rows, cols, ldx, block, amax_src, n_amax, codes, scales, alpha, s, rht_signs);
    }
    return hipGetLastError();
}

hipError_t launch_amax_col16_rht(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, uint32_t signs,
                                 float *partials, int n_partials, hipStream_t s)
{
    if (dtype == 1)
        k_amax_col16_rht<uint16_t><<<n_partials, kAmaxThreads, 0, s>>>((const uint16_t *)x, rows, cols, ldx, signs,
                                                                       partials);
    else
        k_amax_col16_rht<float><<<n_partials, kAmaxThreads, 0, s>>>((const float *)x, rows, cols, ldx, signs,
                                                                    partials);
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t rows,
                             int64_t cols, int block, void *y, int ydtype, int64_t ldy, hipStream_t s)
{
    if (rows == 0 || cols == 0)
        return hipSuccess;
    if (block == 2) {
        const int64_t n = cols * (rows / 16);
        const unsigned grid = (unsigned)((n + kQuantThreads - 1) / kQuantThreads);
        if (ydtype == 1)
            k_dequant_col16<uint16_t><<<grid, kQuantThreads, 0, s>>>(codes, scales, alpha, rows, cols, (uint16_t *)y, ldy);
        else
            k_dequant_col16<float><<<grid, kQuantThreads, 0, s>>>(codes, scales, alpha, rows, cols, (float *)y, ldy);
    } else {
        const int64_t bpr = cols / 16;
        const unsigned grid = (unsigned)((rows * bpr + kQuantThreads - 1) / kQuantThreads);
        if (block == 1) {
            if (ydtype == 1)
                k_dequant_rows<uint16_t, true><<<grid, kQuantThreads, 0, s>>>(codes, scales, alpha, rows, bpr, (uint16_t *)y, ldy);
            else
                k_dequant_rows<float, true><<<grid, kQuantThreads, 0, s>>>(codes, scales, alpha, rows, bpr, (float *)y, ldy);
        } else {
            if (ydtype == 1)
                k_dequant_rows<uint16_t, false><<<grid, kQuantThreads, 0, s>>>(codes, scales, alpha, rows, bpr, (uint16_t *)y, ldy);
            else
                k_dequant_rows<float, false><<<grid, kQuantThreads, 0, s>>>(codes, scales, alpha, rows, bpr, (float *)y, ldy);
        }
    }
    return hipGetLastError();
}

hipError_t launch_kv_smooth_quantize(const void *x, int dtype, int64_t vectors, int64_t head_dim, int rule,
                                     uint8_t *codes, uint8_t *scales, float *alpha, float *means, float *partials,
                                     hipStream_t s)
{
    int g_log2 = 0;
    while ((16 << g_log2) < head_dim)
        g_log2++;
    const int n = amax_partials(vectors, head_dim);
    if (dtype == 1)
        k_kv_smooth_amax<uint16_t><<<n, kAmaxThreads, 0, s>>>((const uint16_t *)x, vectors, g_log2, means, partials);
    else
        k_kv_smooth_amax<float><<<n, kAmaxThreads, 0, s>>>((const float *)x, vectors, g_log2, means, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t nb = vectors << g_log2;
    if (nb == 0) {
        k_alpha_only<<<1, kQuantThreads, 0, s>>>(partials, n, alpha);
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)((nb + kQuantThreads - 1) / kQuantThreads);
    if (dtype == 1) {
        if (rule) k_kv_quant_smoothed<uint16_t, true><<<grid, kQuantThreads, 0, s>>>((const uint16_t *)x, vectors, g_log2, means, partials, n, codes, scales, alpha);
        else      k_kv_quant_smoothed<uint16_t, false><<<grid, kQuantThreads, 0, s>>>((const uint16_t *)x, vectors, g_log2, means, partials, n, codes, scales, alpha);
    } else {
        if (rule) k_kv_quant_smoothed<float, true><<<grid, kQuantThreads, 0, s>>>((const float *)x, vectors, g_log2, means, partials, n, codes, scales, alpha);
        else      k_kv_quant_smoothed<float, false><<<grid, kQuantThreads, 0, s>>>((const float *)x, vectors, g_log2, means, partials, n, codes, scales, alpha);
    }
    return hipGetLastError();
}

int kv_chunk_pseg(int64_t heads, int64_t units)
{
    // about 512 amax workgroups in all, at most kMaxAmaxSrc partials per unit
    int64_t p = (512 + heads * units - 1) / (heads * units);
    const int64_t cap = kMaxAmaxSrc / heads;
    if (p > cap) p = cap;
    if (p < 1) p = 1;
    return (int)p;
}

hipError_t launch_kv_quantize_chunked(const void *x, int dtype, int64_t tensors, int64_t heads, int64_t tokens,
                                      int64_t d, int64_t tpc, int rule, const float *chunk_amax, uint8_t *codes,
                                      uint8_t *scales, float *alphas, float *partials, hipStream_t s)
{
    const int64_t nch = (tokens + tpc - 1) / tpc;
    if (nch == 0 || tensors == 0)
        return hipSuccess;
    const int64_t units = tensors * nch;
    KvChunks k{tokens, tpc, d, heads, (int)nch, kv_chunk_pseg(heads, units), kv_nch_magic(nch)};
    const float *src = chunk_amax;
    int64_t stride = 1;
    int n_amax = 1;
    if (!chunk_amax) {
        dim3 ga((unsigned)k.pseg, (unsigned)heads, (unsigned)units);
        if (dtype == 1)
            k_amax_kv_chunked<uint16_t><<<ga, kAmaxThreads, 0, s>>>((const uint16_t *)x, k, partials);
        else
            k_amax_kv_chunked<float><<<ga, kAmaxThreads, 0, s>>>((const float *)x, k, partials);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        src = partials;
        n_amax = (int)(heads * k.pseg);
        stride = n_amax;
    }
    const int64_t bpr = d / 16;
    const int64_t longest = tpc < tokens ? tpc : tokens;           // tokens of the longest chunk
    dim3 gq((unsigned)((longest * bpr + kQuantThreads - 1) / kQuantThreads), (unsigned)heads, (unsigned)units);
    // partials per thread: one up to kQuantThreads of them, else up to four
    auto go = [&](auto kernel, auto xt) {
        kernel<<<gq, kQuantThreads, 0, s>>>(xt, k, src, stride, n_amax, codes, scales, alphas);
    };
    constexpr int NPT = kMaxAmaxSrc / kQuantThreads;
    const bool one = n_amax <= kQuantThreads;
    const uint16_t *xh = (const uint16_t *)x;
    const float *xf = (const float *)x;
    if (dtype == 1) {
        if (rule) one ? go(k_quant_kv_chunked<uint16_t, true, 1>, xh) : go(k_quant_kv_chunked<uint16_t, true, NPT>, xh);
        else      one ? go(k_quant_kv_chunked<uint16_t, false, 1>, xh) : go(k_quant_kv_chunked<uint16_t, false, NPT>, xh);
    } else {
        if (rule) one ? go(k_quant_kv_chunked<float, true, 1>, xf) : go(k_quant_kv_chunked<float, true, NPT>, xf);
        else      one ? go(k_quant_kv_chunked<float, false, 1>, xf) : go(k_quant_kv_chunked<float, false, NPT>, xf);
    }
    return hipGetLastError();
}

hipError_t launch_kv_dequantize_chunked(const uint8_t *codes, const uint8_t *scales, const float *alphas,
                                        int64_t tensors, int64_t heads, int64_t tokens, int64_t d, int64_t tpc,
                                        void *y, int ydtype, hipStream_t s)
{
    const int64_t nblocks = tensors * heads * tokens * (d / 16);
    if (nblocks == 0)
        return hipSuccess;
    const int64_t nch = (tokens + tpc - 1) / tpc;
    KvChunks k{tokens, tpc, d, heads, (int)nch, 1, kv_nch_magic(nch)};
    const unsigned grid = (unsigned)((nblocks + kQuantThreads - 1) / kQuantThreads);
    if (ydtype == 1)
        k_dequant_kv_chunked<uint16_t><<<grid, kQuantThreads, 0, s>>>(codes, scales, alphas, k, nblocks, (uint16_t *)y);
    else
        k_dequant_kv_chunked<float><<<grid, kQuantThreads, 0, s>>>(codes, scales, alphas, k, nblocks, (float *)y);
    return hipGetLastError();
}

hipError_t launch_kv_window(const KvWindowArgs &a, void *y, int ydtype, int64_t ldy, hipStream_t s)
{
    if (a.wgs == 0)
        return hipSuccess;
    if (ydtype == 1)
        k_kv_window<uint16_t><<<(unsigned)a.wgs, kQuantThreads, 0, s>>>(a, (uint16_t *)y, ldy);
    else
        k_kv_window<float><<<(unsigned)a.wgs, kQuantThreads, 0, s>>>(a, (float *)y, ldy);
    return hipGetLastError();
}


}  // namespace nvfp4
