// Device-side building blocks of the NVFP4 kernels for gfx950 (CDNA4).
//
// Format ("LongLive-2.0: An NVFP4 Parallel Infrastructure for Long Video
// Generation", architecture walkthrough page, section "NVFP4 Training"):
// E2M1 element codes, one E4M3 scale per 16-element block, one fp32 scale per
// tensor, Xhat = X_FP4 * alpha_FP8 * alpha_FP32.
//
// Hardware conversions used (their rounding was checked against exact
// references on the device):
//   v_cvt_scalef32_pk_fp4_f32  fp32 pair -> E2M1 pair; with scale 1.0 it is
//                              round-to-nearest-even, saturating at 6, and it
//                              keeps the sign of zero (the scale operand only
//                              contributes its exponent, so it is left at 1).
//   v_cvt_scalef32_pk_f32_fp4  E2M1 pair -> fp32 pair, exact.
//   v_cvt_scalef32_pk_f16_fp4  E2M1 pair -> fp16 pair, exact.
//   v_cvt_pk_fp8_f32           fp32 pair -> E4M3FN pair, nearest-even with
//                              subnormals; returns NaN above 464, so inputs are
//                              clamped to 448 first (the saturating rule).
//   v_cvt_f32_fp8 / v_cvt_scalef32_pk_f16_fp8  E4M3 -> fp32 / fp16, exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

// M_FP8 * M_FP4: the global scale maps the tensor max to 448 * 6.
constexpr float kGlobalRange = 2688.0f;
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// alpha_FP32 from the tensor's absolute maximum.
__device__ __forceinline__ float global_scale(float amax)
{
    return amax == 0.0f ? 1.0f : amax / kGlobalRange;
}

// Two E2M1 codes (a -> low nibble, b -> high nibble) into byte SEL of old.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_put2(uint32_t old, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Values of the two codes in byte SEL of w.
template <int SEL>
__device__ __forceinline__ float2v e2m1_get2(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// E4M3 bytes of two non-negative values: byte 0 <- a, byte 1 <- b.
__device__ __forceinline__ uint32_t e4m3_put2(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(a, kE4M3Max), fminf(b, kE4M3Max), 0, false) &
           0xffffu;
}

template <int SEL>
__device__ __forceinline__ float e4m3_get(uint32_t w)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// One candidate encoding of a 16-element block row with block scale s and
// kappa = 1 / (s * alpha) (0 when s == 0): codes of x * kappa, and the fma
// chain of squared residuals d = x - q*s*alpha (exact product, one rounding),
// continued from e.
__device__ __forceinline__ void encode16(const float (&x)[16], float s, float kappa, float alpha, uint32_t &c0,
                                         uint32_t &c1, float &e)
{
    uint32_t w0 = 0, w1 = 0;
    w0 = e2m1_put2<0>(w0, x[0] * kappa, x[1] * kappa);
    w0 = e2m1_put2<1>(w0, x[2] * kappa, x[3] * kappa);
    w0 = e2m1_put2<2>(w0, x[4] * kappa, x[5] * kappa);
    w0 = e2m1_put2<3>(w0, x[6] * kappa, x[7] * kappa);
    w1 = e2m1_put2<0>(w1, x[8] * kappa, x[9] * kappa);
    w1 = e2m1_put2<1>(w1, x[10] * kappa, x[11] * kappa);
    w1 = e2m1_put2<2>(w1, x[12] * kappa, x[13] * kappa);
    w1 = e2m1_put2<3>(w1, x[14] * kappa, x[15] * kappa);
    // residual d = x - (q*s)*alpha with q*s formed exactly in fp16 (<= 6
    // significant bits, within fp16's normal range) and a mixed-precision fma
    // (exact operand conversion, one rounding): equal to fmaf(-(q*s), alpha, x)
    const _Float16 sh = (_Float16)s;                 // E4M3 values are exact in fp16
    const half2v ss = {sh, sh};
    half2v qs[8];
    qs[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0) * ss;
    qs[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1) * ss;
    qs[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2) * ss;
    qs[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3) * ss;
    qs[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 0) * ss;
    qs[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 1) * ss;
    qs[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 2) * ss;
    qs[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 3) * ss;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float d = __builtin_fmaf(-(float)qs[i >> 1][i & 1], alpha, x[i]);
        e = __builtin_fmaf(d, d, e);
    }
    c0 = w0;
    c1 = w1;
}

// RN(a / b) from y = RN(1 / b) without a division: q0 = RN(a * y), then one
// fma correction q = RN(q0 + RN(a - q0 * b) * y) with the residual exact
// (Markstein's correction step).  Checked against IEEE division on the CPU
// for all 2^46 pairs of fp32 significands in [1, 2) and, for b = 6, every
// fp32 a whose quotient is normal.  Exact while the residual does not
// underflow: callers use it only where quotients below 2^-9 end up in E4M3
// conversions that map them to zero either way.
__device__ __forceinline__ float div_rcp(float a, float b, float y)
{
    const float q0 = a * y;
    return __builtin_fmaf(__builtin_fmaf(-q0, b, a), y, q0);
}

// Slot 127 of the kappa table (E4M3 byte 127 is NaN and never a scale: scales
// are clamped to 448) holds RN(1 / (alpha * sc)), sc = alpha_rescale(alpha).
constexpr int kRcpAlphaSlot = 127;

// Power of two that keeps the residual of div_rcp(m * sc, alpha * sc, ...)
// clear of underflow for every block max m with m / alpha >= 2^-9 (smaller
// quotients give E4M3 zero either way): 1 for alpha >= 2^-90, else 2^100.
// Scaling both operands by a power of two is exact and leaves the quotient
// unchanged.
__device__ __forceinline__ float alpha_rescale(float alpha)
{
    return alpha >= 0x1p-90f ? 1.0f : 0x1p100f;
}

// kappa = RN(1 / RN(s * alpha)) for every E4M3 scale byte b in [0, 127), 0 for
// s == 0; built once per workgroup so blocks look it up instead of dividing.
// Every thread of the workgroup must call it (it synchronizes).
__device__ __forceinline__ void build_kappa_table(float *tab, float alpha)
{
    for (int b = threadIdx.x; b < 128; b += blockDim.x) {
        float k = 0.0f;
        if (b == kRcpAlphaSlot) {
            k = 1.0f / (alpha * alpha_rescale(alpha));     // IEEE division (correctly rounded)
        } else if (b != 0) {
            const float d = __builtin_amdgcn_cvt_f32_fp8(b, 0) * alpha;
            k = 1.0f / d;
        }
        tab[b] = k;
    }
    __syncthreads();
}

// The two candidate scale bytes of a block with max |x| = m: byte 0 E4M3(mu /
// 6), byte 1 E4M3(mu / 4), mu = m / alpha, with the bytes IEEE division would
// give.  Non-finite quotients (alpha 0, infinite m) come out NaN where the
// division gives infinity; the 448 clamp maps both to the same byte.
__device__ __forceinline__ uint32_t block_scale_bytes(float m, float alpha, const float *ktab)
{
    const float sc = alpha_rescale(alpha);
    const float mu = div_rcp(m * sc, alpha * sc, ktab[kRcpAlphaSlot]);
    const float t6 = div_rcp(mu, 6.0f, 1.0f / 6.0f);
    const float t4 = mu * 0.25f;                 // == RN(mu / 4)
    return e4m3_put2(t6, t4);                    // byte0: s6, byte1: s4
}

// Quantize one 1D block of 16 values (RULE4: four-over-six): codes (8 bytes)
// and the E4M3 scale byte.  ktab: the workgroup's kappa table.
template <bool RULE4>
__device__ __forceinline__ void quant_block16(const float (&x)[16], float alpha, const float *ktab, uint32_t &c0,
                                              uint32_t &c1, uint32_t &sbyte)
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++)
        m = fmaxf(m, fabsf(x[i]));
    const uint32_t sb = block_scale_bytes(m, alpha, ktab);
    const uint32_t b6 = sb & 0xffu, b4 = (sb >> 8) & 0xffu;
    const float s6 = e4m3_get<0>(sb);
    float e6 = 0.0f;
    encode16(x, s6, ktab[b6], alpha, c0, c1, e6);
    sbyte = b6;
    if (RULE4) {
        const float s4 = e4m3_get<1>(sb);
        uint32_t d0, d1;
        float e4 = 0.0f;
        encode16(x, s4, ktab[b4], alpha, d0, d1, e4);
        if (e4 < e6) {
            c0 = d0;
            c1 = d1;
            sbyte = b4;
        }
    }
}

// 16-byte load marked non-temporal: the data is streamed through once, so the
// caches need not keep it (measured faster on the tensor-sized passes).  One
// vector load, so that it stays one 16-byte instruction.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4 *p)
{
    const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Stores marked non-temporal, for outputs the writing kernel does not read
// back (measured faster for the quantizers' packed codes and scales and for
// the GEMM's C tile).
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

// one block's 8 code bytes (8-byte aligned) and its scale byte
__device__ __forceinline__ void store_block_stream(uint8_t *codes8, uint8_t *scale, uint32_t c0, uint32_t c1,
                                                   uint32_t sb)
{
    __builtin_nontemporal_store(u32x2v{c0, c1}, reinterpret_cast<u32x2v *>(codes8));
    __builtin_nontemporal_store((uint8_t)sb, scale);
}

// 16 bytes (16-byte aligned)
__device__ __forceinline__ void store16_stream(void *p, uint4 v)
{
    __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v *>(p));
}

// 16 consecutive elements of row-major input (16-byte aligned).
__device__ __forceinline__ void load16(const uint16_t *p, float (&x)[16])
{
    uint4 a = *reinterpret_cast<const uint4 *>(p);
    uint4 b = *reinterpret_cast<const uint4 *>(p + 8);
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        x[2 * i] = bf16_lo(w[i]);
        x[2 * i + 1] = bf16_hi(w[i]);
    }
}

__device__ __forceinline__ void load16(const float *p, float (&x)[16])
{
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float4 v = *reinterpret_cast<const float4 *>(p + 4 * i);
        x[4 * i] = v.x;
        x[4 * i + 1] = v.y;
        x[4 * i + 2] = v.z;
        x[4 * i + 3] = v.w;
    }
}

__device__ __forceinline__ float load1(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float load1(const float *p) { return *p; }

// Random Hadamard transform of one 16-element block along the reduction axis
// (NVFP4 Training section, "Random Hadamard Transform (RHT) for gradient
// stabilization"): x <- (1/4) H16 D x, D = diag(-1 where bit i of signs is
// set).  fp32 order: sign flips, butterfly stages h = 1, 2, 4, 8 with
// (a, b) -> (a + b, a - b), then the exact scaling by 1/4.
__device__ __forceinline__ void rht16(float (&x)[16], uint32_t signs)
{
#pragma unroll
    for (int i = 0; i < 16; i++)
        x[i] = ((signs >> i) & 1u) ? -x[i] : x[i];
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            if (i & h)
                continue;
            const float a = x[i], b = x[i + h];
            x[i] = a + b;
            x[i + h] = a - b;
        }
    }
#pragma unroll
    for (int i = 0; i < 16; i++)
        x[i] = x[i] * 0.25f;
}

// Wave-wide max (64 lanes).
// v from another lane by a DPP control; lanes of rows outside ROW_MASK get 0
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_or_zero(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Max over the wave of NON-NEGATIVE values (0 is the identity), the same in
// every lane: butterflies inside each row of 16 lanes (quad permutes, half-row
// and row mirrors), then the row broadcasts carry rows 0-2 into row 3, and
// lane 63 is read back as a uniform value.
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_or_zero<0xB1>(v));          // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_or_zero<0x4E>(v));          // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_or_zero<0x141>(v));         // row_half_mirror
    v = fmaxf(v, dpp_or_zero<0x140>(v));         // row_mirror: every lane holds its row's max
    v = fmaxf(v, dpp_or_zero<0x142, 0xa>(v));    // row_bcast15 into rows 1 and 3
    v = fmaxf(v, dpp_or_zero<0x143, 0xc>(v));    // row_bcast31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

}  // namespace nvfp4
