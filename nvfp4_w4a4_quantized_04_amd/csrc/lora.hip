// Down projection of the BF16 low-rank (LoRA) branch of a W4A4 linear layer:
// U = bf16(x A^T), later added as lora_scale * U B^T by the NVFP4 GEMM
// ("LongLive-2.0: An NVFP4 Parallel Infrastructure for Long Video
// Generation", architecture walkthrough page: "LoRA parameterization", rank
// 128 adapters in BF16, and the NVFP4 Inference section, where the adapters
// stay a separate BF16 branch on the quantized backbone).
#include "internal.h"

namespace nvfp4 {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

// ------------------------------------------------ LoRA down projection

// U [M][r] = RN_bf16(x [M][K] A^T), A [r][K], bf16 operands, fp32 sums.
// Stage 1: workgroup (m tile of 32 rows, K slice) stages 64-k steps of x and A
// in LDS with 16-byte coalesced loads (the next step's loads in flight) and
// accumulates a 32 x r partial with 32x32x16 bf16 MFMA, one 32-column block
// per wave.  Stage 2 adds the K-slice partials in slice order and rounds once.
constexpr int kLoraRowB = 64 * 2 + 16;   // LDS bytes per staged row (64 k + pad)


// amax_part (optional): max |x| over the x chunks this workgroup staged
// (rows m0..m0+31 of its K slice; clamped rows repeat row M-1), one float
// per workgroup at blockIdx.y * gridDim.x + blockIdx.x.
__global__ __launch_bounds__(256) void k_lora_partial(const uint16_t *__restrict__ x, int64_t ldx, int M, int K,
                                                      const uint16_t *__restrict__ a, int r, int kslice,
                                                      float *__restrict__ part, float *__restrict__ amax_part)
{
    __shared__ float red[4];
    float xmax = 0.0f;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(32 + 128) * kLoraRowB];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5;
    const int m0 = blockIdx.x * 32;
    const int kb = blockIdx.y * kslice, ke = kb + kslice < K ? kb + kslice : K;
    const int nrows = 32 + r;                      // staged rows: 32 of x, r of A
    const int chunks = nrows * 8;                  // 16-byte chunks per 64-k step
    float16v acc = float16v{};
    const bool active = wave * 32 < r;
    // Every load is issued unconditionally (a load under a branch is waited
    // for before the next one goes out): a chunk index past the end re-reads
    // the last chunk, a k past the slice reads column 0 of the same row, and
    // the bits of `ok` say which chunks lie inside the slice (the rest are
    // staged as zero).
    auto fetch = [&](int k0, uint4 (&v)[5]) -> unsigned {
        unsigned ok = 0;
#pragma unroll
        for (int u = 0; u < 5; u++) {
            const int q = tid + u * 256 < chunks ? tid + u * 256 : chunks - 1;
            const int row = q >> 3, c = q & 7;
            const int k = k0 + c * 8;
            ok |= (unsigned)(k < ke) << u;                // of the clamped chunk: a repeat stores the same value
            const uint16_t *src = row < 32 ? x + (int64_t)(m0 + row < M ? m0 + row : M - 1) * ldx
                                           : a + (int64_t)(row - 32) * K;
            v[u] = *reinterpret_cast<const uint4 *>(src + (k < ke ? k : 0));
        }
        return ok;
    };
    auto stash = [&](uint8_t *buf, const uint4 (&v)[5], unsigned ok) {
#pragma unroll
        for (int u = 0; u < 5; u++) {
            const int q = tid + u * 256 < chunks ? tid + u * 256 : chunks - 1;
            uint4 w = v[u];
            if (!((ok >> u) & 1))
                w = make_uint4(0, 0, 0, 0);
            if (q < 32 * 8) {                      // a chunk of x (rows 0-31)
                const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int j = 0; j < 4; j++)
                    xmax = fmaxf(xmax, fmaxf(fabsf(__uint_as_float(e[j] << 16)),
                                             fabsf(__uint_as_float(e[j] & 0xffff0000u))));
            }
            // past the end: the last chunk again (same value, same place)
            *reinterpret_cast<uint4 *>(buf + (q >> 3) * kLoraRowB + (q & 7) * 16) = w;
        }
    };
    uint4 v[5];
    unsigned ok = 0;
    int buf = 0;
    if (kb < ke) {
        ok = fetch(kb, v);
        stash(lds[0], v, ok);
    }
    __syncthreads();
    for (int k0 = kb; k0 < ke; k0 += 64) {
        const bool more = k0 + 64 < ke;
        if (more)
            ok = fetch(k0 + 64, v);                // in flight under this step's MFMAs
        if (active) {
            const uint8_t *st = lds[buf];
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const bf16x8v fa = *reinterpret_cast<const bf16x8v *>(st + (32 + wave * 32 + l32) * kLoraRowB + s * 32 + half * 16);
                const bf16x8v fx = *reinterpret_cast<const bf16x8v *>(st + l32 * kLoraRowB + s * 32 + half * 16);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fx, acc, 0, 0, 0);
            }
        }
        if (more)
            stash(lds[buf ^ 1], v, ok);
        __syncthreads();
        buf ^= 1;
    }
    if (amax_part) {
        xmax = wave_max(xmax);
        if (lane == 0)
            red[wave] = xmax;
        __syncthreads();
        if (tid == 0)
            amax_part[blockIdx.y * gridDim.x + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
    // lane l, register q: row m0 + l%32, column 32*wave + 8*(q/4) + 4*(l/32) + q%4
    if (active) {
        float *dst = part + ((int64_t)blockIdx.y * M + m0 + l32) * r + wave * 32 + 4 * half;
        if (m0 + l32 < M) {
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++)
                *reinterpret_cast<float4 *>(dst + 8 * q4) =
                    make_float4(acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]);
        }
    }
}

__global__ __launch_bounds__(256) void k_lora_reduce(const float *__restrict__ part, int slices, int64_t n,
                                                     uint16_t *__restrict__ u)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    float v = slices > 0 ? part[i] : 0.0f;
    for (int s = 1; s < slices; s++)
        v = v + part[s * n + i];
    const __bf16 h = (__bf16)v;
    u[i] = __builtin_bit_cast(uint16_t, h);
}

int lora_slices(int64_t m, int64_t k)
{
    const int64_t mt = (m + 31) / 32;
    int64_t sl = (768 + mt - 1) / mt;               // about three workgroups per CU
    const int64_t steps = (k + 63) / 64;
    if (sl > steps) sl = steps;
    if (sl > kLoraMaxSlicesAbi) sl = kLoraMaxSlicesAbi;
    return (int)(sl < 1 ? 1 : sl);
}

int lora_amax_partials(int64_t m, int64_t k)
{
    return k > 0 && m > 0 ? (int)((m + 31) / 32) * lora_slices(m, k) : 0;
}

hipError_t launch_lora_partial(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, const uint16_t *a, int r,
                               float *partials, float *amax_part, hipStream_t s)
{
    if (m == 0 || k == 0)
        return hipSuccess;
    const int sl = lora_slices(m, k);
    const int64_t steps = (k + 63) / 64;
    const int kslice = (int)((steps + sl - 1) / sl * 64);
    dim3 grid((unsigned)((m + 31) / 32), (unsigned)sl);
    k_lora_partial<<<grid, 256, 0, s>>>(x, ldx, (int)m, (int)k, a, r, kslice, partials, amax_part);
    return hipGetLastError();
}

hipError_t launch_lora_reduce(int64_t m, int64_t k, int r, const float *partials, uint16_t *u, hipStream_t s)
{
    if (m == 0)
        return hipSuccess;
    const int64_t n = m * r;
    // k == 0: no partial was written and U is zero
    k_lora_reduce<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(partials, k > 0 ? lora_slices(m, k) : 0, n, u);
    return hipGetLastError();
}

hipError_t launch_lora_down(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, const uint16_t *a, int r,
                            uint16_t *u, float *partials, hipStream_t s)
{
    const hipError_t e = launch_lora_partial(x, ldx, m, k, a, r, partials, nullptr, s);
    if (e != hipSuccess)
        return e;
    return launch_lora_reduce(m, k, r, partials, u, s);
}

}  // namespace nvfp4
