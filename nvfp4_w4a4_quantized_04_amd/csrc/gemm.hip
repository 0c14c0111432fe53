// NVFP4 x NVFP4 GEMM for gfx950:  C = alpha_A alpha_B sum_k Ahat[m,k] Bhat[n,k].
//
// The pages' contraction ("LongLive-2.0: An NVFP4 Parallel Infrastructure for
// Long Video Generation", architecture walkthrough page, NVFP4 Training
// section, "The three GEMMs of backpropagation" and "Quantization-
// dequantization flow") runs on Blackwell FP4 tensor cores with E4M3 block
// scales.  gfx950's scaled FP4 MFMA only takes power-of-two (E8M0) scales per
// 32 elements, so it cannot carry an E4M3 scale per 16 elements exactly.
// Instead, every dequantized operand value q*s has at most 6 significant
// bits and lies in [2^-10, 2688], so it is EXACT in fp16.  The kernel
// therefore
//   1. stages the packed operands (0.5 B codes + 1/16 B scales per element)
//      from HBM into LDS, double buffered;
//   2. each wave decodes its MFMA fragments with v_cvt_scalef32_pk_f16_fp4
//      (exact) and one v_pk_mul_f16 by the block scale (exact);
//   3. accumulates with v_mfma_f32_32x32x16_f16 in fp32;
//   4. multiplies by alpha_A * alpha_B in the epilogue and stores fp32/bf16.
//
// Tiling: 256 threads = 4 waves in a 2x2 grid, each wave TM x TN MFMA tiles
// of 32x32, so a workgroup tile is (64 TM) x (64 TN) with BK = 64 (four
// 16-element scale blocks).  K order inside a BK step: lanes 0-31 of a
// fragment hold k in [0, 32) and lanes 32-63 k in [32, 64) of the step, 8 per
// MFMA; A and B use the same assignment, so the sum is over every k once.
#include "internal.h"

namespace nvfp4 {

constexpr int kBK = 64;             // K elements per main-loop step
constexpr int kRowBytes = kBK / 2;  // code bytes per row per step
constexpr int kLdsStride = 48;      // padded LDS row stride (bank-conflict free 16 B reads)

struct GemmArgs {
    const uint8_t *a_codes, *a_scales;
    const uint8_t *b_codes, *b_scales;
    const float *a_alpha, *b_alpha;
    void *c;
    int64_t ldc;
    int M, N, K;
    int a2d, b2d;
    int tiles_n;
    int c_bf16;
};

template <int ROWS>
struct StageRegs {
    uint4 codes[(2 * ROWS + 255) / 256];
    uint32_t scales[(ROWS + 255) / 256];
};

// Global -> registers for one operand tile of ROWS rows at K-step kt.
template <int ROWS>
__device__ __forceinline__ void load_stage(StageRegs<ROWS> &r, const uint8_t *__restrict__ codes,
                                           const uint8_t *__restrict__ scales, int s2d, int row0, int nrows,
                                           int K, int kt, bool kfull)
{
    const int tid = threadIdx.x;
    const int64_t rb = K / 2;       // code bytes per row
    const int64_t sb = K / 16;      // scale bytes per scale row
#pragma unroll
    for (int i = 0; i < (2 * ROWS + 255) / 256; i++) {
        const int q = tid + 256 * i;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (q < 2 * ROWS) {
            const int row = q >> 1, ch = q & 1;
            const int gr = row0 + row;
            if (gr < nrows) {
                const int64_t off = (int64_t)gr * rb + (int64_t)kt * kRowBytes + ch * 16;
                if (kfull) {
                    v = *reinterpret_cast<const uint4 *>(codes + off);
                } else {
                    const int64_t left = rb - ((int64_t)kt * kRowBytes + ch * 16);
                    if (left >= 8) {
                        uint2 lo = *reinterpret_cast<const uint2 *>(codes + off);
                        v.x = lo.x; v.y = lo.y;
                    }
                    if (left >= 16) {
                        uint2 hi = *reinterpret_cast<const uint2 *>(codes + off + 8);
                        v.z = hi.x; v.w = hi.y;
                    }
                }
            }
        }
        r.codes[i] = v;
    }
#pragma unroll
    for (int i = 0; i < (ROWS + 255) / 256; i++) {
        const int row = tid + 256 * i;
        uint32_t w = 0;
        if (row < ROWS) {
            const int gr = row0 + row;
            if (gr < nrows) {
                const int64_t srow = s2d ? gr / 16 : gr;
                const int64_t off = srow * sb + (int64_t)kt * 4;
                if (kfull) {
                    w = *reinterpret_cast<const uint32_t *>(scales + off);
                } else {
                    const int64_t left = sb - (int64_t)kt * 4;
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        if (j < left)
                            w |= (uint32_t)scales[off + j] << (8 * j);
                }
            }
        }
        r.scales[i] = w;
    }
}

template <int ROWS>
__device__ __forceinline__ void store_stage(const StageRegs<ROWS> &r, uint8_t *lds_codes, uint32_t *lds_scales)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < (2 * ROWS + 255) / 256; i++) {
        const int q = tid + 256 * i;
        if (q < 2 * ROWS)
            *reinterpret_cast<uint4 *>(lds_codes + (q >> 1) * kLdsStride + (q & 1) * 16) = r.codes[i];
    }
#pragma unroll
    for (int i = 0; i < (ROWS + 255) / 256; i++) {
        const int row = tid + 256 * i;
        if (row < ROWS)
            lds_scales[row] = r.scales[i];
    }
}

// 8 fp16 operand values (exact q*s) from one code dword and a block scale.
__device__ __forceinline__ half8v dequant8(uint32_t w, _Float16 s)
{
    const half2v ss = {s, s};
    half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    half8v o = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    return o;
}

template <int TM, int TN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_nvfp4(GemmArgs g)
{
    constexpr int BM = 64 * TM, BN = 64 * TN;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * kLdsStride];
    __shared__ uint32_t lds_as[2][BM];
    __shared__ uint32_t lds_bs[2][BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    const int tm = blockIdx.x / g.tiles_n;
    const int tn = blockIdx.x - tm * g.tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (g.K + kBK - 1) / kBK;
    const bool kfull = (g.K % kBK) == 0;

    float16v acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
            acc[i][j] = float16v{};

    StageRegs<BM> ra;
    StageRegs<BN> rb;
    if (nk > 0) {
        load_stage<BM>(ra, g.a_codes, g.a_scales, g.a2d, m0, g.M, g.K, 0, kfull);
        load_stage<BN>(rb, g.b_codes, g.b_scales, g.b2d, n0, g.N, g.K, 0, kfull);
        store_stage<BM>(ra, lds_a[0], lds_as[0]);
        store_stage<BN>(rb, lds_b[0], lds_bs[0]);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            load_stage<BM>(ra, g.a_codes, g.a_scales, g.a2d, m0, g.M, g.K, kt + 1, kfull);
            load_stage<BN>(rb, g.b_codes, g.b_scales, g.b2d, n0, g.N, g.K, kt + 1, kfull);
        }
        // fragments of this step: 16 code bytes (32 k values) + 2 scales per tile
        uint4 ca[TM], cb[TN];
        half2v sa[TM], sbv[TN];
#pragma unroll
        for (int i = 0; i < TM; i++) {
            const int row = wm * 32 * TM + i * 32 + l32;
            ca[i] = *reinterpret_cast<const uint4 *>(&lds_a[cur][row * kLdsStride + half * 16]);
            const uint32_t sw = lds_as[cur][row] >> (16 * half);
            sa[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int row = wn * 32 * TN + j * 32 + l32;
            cb[j] = *reinterpret_cast<const uint4 *>(&lds_b[cur][row * kLdsStride + half * 16]);
            const uint32_t sw = lds_bs[cur][row] >> (16 * half);
            sbv[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
        }
#pragma unroll
        for (int s = 0; s < 4; s++) {
            half8v af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const uint32_t w = s == 0 ? ca[i].x : s == 1 ? ca[i].y : s == 2 ? ca[i].z : ca[i].w;
                af[i] = dequant8(w, sa[i][s >> 1]);
            }
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const uint32_t w = s == 0 ? cb[j].x : s == 1 ? cb[j].y : s == 2 ? cb[j].z : cb[j].w;
                bf[j] = dequant8(w, sbv[j][s >> 1]);
            }
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            store_stage<BM>(ra, lds_a[cur ^ 1], lds_as[cur ^ 1]);
            store_stage<BN>(rb, lds_b[cur ^ 1], lds_bs[cur ^ 1]);
        }
        __syncthreads();
    }

    // epilogue: 32x32 accumulator layout -- register r of lane l holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32
    const float scale = *g.a_alpha * *g.b_alpha;
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int col = n0 + wn * 32 * TN + j * 32 + l32;
            if (col >= g.N)
                continue;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int row = m0 + wm * 32 * TM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (row < g.M) {
                    const float v = acc[i][j][r] * scale;
                    if (g.c_bf16) {
                        __bf16 h = (__bf16)v;
                        reinterpret_cast<uint16_t *>(g.c)[(int64_t)row * g.ldc + col] =
                            __builtin_bit_cast(uint16_t, h);
                    } else {
                        reinterpret_cast<float *>(g.c)[(int64_t)row * g.ldc + col] = v;
                    }
                }
            }
        }
}

template <int TM, int TN>
static hipError_t launch_tm_tn(GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (g.M + 64 * TM - 1) / (64 * TM);
    g.tiles_n = (g.N + 64 * TN - 1) / (64 * TN);
    const int64_t grid = (int64_t)tiles_m * g.tiles_n;
    k_gemm_nvfp4<TM, TN><<<(unsigned)grid, 256, 0, s>>>(g);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmOperand &a, const GemmOperand &b, int64_t m, int64_t n, int64_t k, void *c,
                       int cdtype, int64_t ldc, hipStream_t s)
{
    if (m == 0 || n == 0)
        return hipSuccess;
    GemmArgs g;
    g.a_codes = a.codes; g.a_scales = a.scales; g.a_alpha = a.alpha; g.a2d = a.scale2d;
    g.b_codes = b.codes; g.b_scales = b.scales; g.b_alpha = b.alpha; g.b2d = b.scale2d;
    g.c = c; g.ldc = ldc; g.c_bf16 = cdtype == 1;
    g.M = (int)m; g.N = (int)n; g.K = (int)k;
    g.tiles_n = 0;
    // tile choice: the largest tile that still gives about one full round of
    // workgroups over the 256 compute units
    const int64_t t44 = ((m + 255) / 256) * ((n + 255) / 256);
    const int64_t t24 = ((m + 127) / 128) * ((n + 255) / 256);
    if (t44 >= 256)
        return launch_tm_tn<4, 4>(g, s);
    if (t24 >= 256)
        return launch_tm_tn<2, 4>(g, s);
    return launch_tm_tn<2, 2>(g, s);
}

}  // namespace nvfp4
