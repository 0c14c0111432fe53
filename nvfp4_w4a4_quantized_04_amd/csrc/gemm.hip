// NVFP4 x NVFP4 GEMM for gfx950:  C = alpha_A alpha_B sum_k Ahat[m,k] Bhat[n,k].
//
// The pages' contraction ("LongLive-2.0: An NVFP4 Parallel Infrastructure for
// Long Video Generation", architecture walkthrough page, NVFP4 Training
// section, "The three GEMMs of backpropagation" and "Quantization-
// dequantization flow") runs on Blackwell FP4 tensor cores with E4M3 block
// scales.  gfx950's scaled FP4 MFMA only takes power-of-two (E8M0) scales per
// 32 elements, so it cannot carry an E4M3 scale per 16 elements exactly.
// Every dequantized operand value q*s, however, has at most 6 significant
// bits and lies in [2^-10, 2688]: it is EXACT in fp16, and fp16 MFMA runs at
// the dense bf16 rate.  So the packed operands are decoded on chip and
// contracted with v_mfma_f32_32x32x16_f16 (fp32 accumulation).
//
// Workgroup = 8 waves, two per SIMD, specialised:
//   producers (waves 4-7) fetch packed stages (0.5 B codes + 1/16 B scale per
//     element) from HBM PD steps ahead into registers, decode them with
//     v_cvt_scalef32_pk_f16_fp4 + v_pk_mul_f16 by the E4M3 block scale (both
//     exact; the convert's own scale operand contributes only its exponent,
//     so it cannot apply an E4M3 scale) and write fp16 tiles into LDS (double
//     buffered, rows padded to 144 B so 16 consecutive rows hit distinct
//     banks);
//   consumers (waves 0-3, 2x2 grid) hold the fp32 accumulators, read MFMA
//     fragments from LDS one 16-k substep ahead and issue the MFMAs.
// The decode VALU work of one wave then overlaps the MFMA work of the other
// wave on the same SIMD.  One barrier per 64-k step hands a stage over.
// Epilogue (bf16 C): the consumers write the scaled, rounded tile into the
// idle stage buffers and all eight waves store it as whole 16-byte row
// chunks; storing the 32x32 fragments directly leaves every store
// instruction 16 bytes in each of 32 rows, which is slower when every
// workgroup of a round writes its tile at once.
// Workgroup tile (64 TM) x (64 TN), BK = 64; consumer wave tile (32 TM) x (32 TN).
#include "internal.h"

#include <cmath>
#include <type_traits>

namespace nvfp4 {

constexpr int kBK = 64;                  // K elements per main-loop step
constexpr int kRowBytes = kBK / 2;       // packed code bytes per row per step
constexpr int kLdsRow = kBK * 2 + 16;    // fp16 LDS row: 128 B + 16 B pad
constexpr int kPrefetch = 4;             // packed stages a producer holds in registers

struct GemmArgs {
    const uint8_t *a_codes, *a_scales;
    const uint8_t *b_codes, *b_scales;
    const float *a_alpha, *b_alpha;
    void *c;
    int64_t ldc;
    int M, N, K;
    int a2d, b2d;
    int tiles_m, tiles_n;
    int band;       // tile rows per band of the tile order (see the kernel)
    int c_bf16;
    int vec_ok;     // C pointer and ldc allow 4-element vector stores
    int stage_ok;   // bf16 C, 16-byte aligned rows, N % 8 == 0: epilogue staged through LDS
    float *c_amax;  // optional: max |C| of the stored values (atomic max, zeroed before the launch)
    // optional BF16 LoRA branch: C += lora_scale * U B^T, U [M][r], B [N][r]
    const uint16_t *lora_u;
    const uint16_t *lora_b;
    int lora_r;
    float lora_scale;
};

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

// LDS row of a LoRA operand tile: r bf16 values + 16 bytes of padding.
__host__ __device__ constexpr int lora_row_bytes(int r) { return 2 * r + 16; }

template <int B, int E, typename F>
__host__ __device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// A producer thread's share of one operand tile: "chunks" of 32 k values
// (16 code bytes + 2 scale bytes) of one row; 2 chunks per row and step.
// W64: write each decoded 16-byte piece to LDS as two 8-byte stores.  Measured
// on the 128-row tiles (FFN shapes 2.5% faster) but slower on the 192/256-row
// tiles, so the choice is per tile shape.
template <int ROWS, bool KFULL, int NSLOT, bool W64 = false>
struct Producer {
    static constexpr int kTotal = 2 * ROWS;
    static constexpr int kPer = (kTotal + 255) / 256;
    static_assert(kTotal % 64 == 0, "repeated chunks fill whole producer waves");
    uint32_t code_off[kPer];    // byte offset of the chunk in the code array at step 0
    uint32_t scale_off[kPer];
    uint32_t lds_off[kPer];
    int ch_off[kPer];           // 0 or 16: the chunk's byte offset inside a step
    bool live[kPer];            // false: the slot only repeats the last chunk
    uint4 codes[NSLOT][kPer];
    uint32_t scales[NSLOT][kPer];
    int rb;                     // code bytes per row (K/2)

    __device__ __forceinline__ void init(int ptid, int s2d, int row0, int nrows, int K)
    {
        rb = K / 2;
        const int sb = K / 16;
#pragma unroll
        for (int i = 0; i < kPer; i++) {
            int q = ptid + 256 * i;
            live[i] = q < kTotal;
            q = q < kTotal ? q : kTotal - 1;        // extra threads load the last chunk again (never stored)
            const int row = q >> 1, ch = q & 1;
            int gr = row0 + row;
            gr = gr < nrows ? gr : nrows - 1;       // rows past the end re-read the last row; never stored
            const int srow = s2d ? gr / 16 : gr;
            code_off[i] = (uint32_t)gr * (uint32_t)rb + ch * 16;
            scale_off[i] = (uint32_t)srow * (uint32_t)sb + ch * 2;
            lds_off[i] = row * kLdsRow + ch * 64;
            ch_off[i] = ch * 16;
        }
    }

    template <int SLOT>
    __device__ __forceinline__ void load(const uint8_t *__restrict__ cbase, const uint8_t *__restrict__ sbase,
                                         int kt)
    {
#pragma unroll
        for (int i = 0; i < kPer; i++) {
            const uint32_t off = code_off[i] + (uint32_t)kt * kRowBytes;
            const uint32_t soff = scale_off[i] + (uint32_t)kt * 4;
            if (KFULL) {
                codes[SLOT][i] = *reinterpret_cast<const uint4 *>(cbase + off);
                scales[SLOT][i] = *reinterpret_cast<const uint16_t *>(sbase + soff);
            } else {
                // K % 64 != 0: codes past K read as zero (their scale is then irrelevant)
                uint4 v = make_uint4(0, 0, 0, 0);
                uint32_t s = 0;
                const int pos = kt * kRowBytes + ch_off[i];
                if (pos + 8 <= rb) {
                    const uint2 lo = *reinterpret_cast<const uint2 *>(cbase + off);
                    v.x = lo.x; v.y = lo.y;
                    s = sbase[soff];
                }
                if (pos + 16 <= rb) {
                    const uint2 hi = *reinterpret_cast<const uint2 *>(cbase + off + 8);
                    v.z = hi.x; v.w = hi.y;
                    s |= (uint32_t)sbase[soff + 1] << 8;
                }
                codes[SLOT][i] = v;
                scales[SLOT][i] = s;
            }
        }
    }

    // decode the chunks of register slot SLOT and write them as fp16 to LDS.
    // A repeated chunk is neither decoded nor written: LDS writes are the
    // costly half of the tile traffic (16-byte writes move about 76 B per
    // clock per CU, reads about 185), and for 192-row operands the repeats
    // are an eighth of them.  Repeats fill whole waves (kTotal is a multiple
    // of 64), so the skip is a uniform branch; the loads stay unconditional.
    template <int SLOT>
    __device__ __forceinline__ void store(uint8_t *lds) const
    {
#pragma unroll
        for (int i = 0; i < kPer; i++) {
            if (kTotal % 256 != 0 && i == kPer - 1 && !live[i])
                continue;
            const half2v s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scales[SLOT][i], 1.0f, false);
            const half2v lo = {s2[0], s2[0]};
            const half2v hi = {s2[1], s2[1]};
            const uint32_t w[4] = {codes[SLOT][i].x, codes[SLOT][i].y, codes[SLOT][i].z, codes[SLOT][i].w};
            uint4 *dst = reinterpret_cast<uint4 *>(lds + lds_off[i]);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const half2v sc = j < 2 ? lo : hi;       // code dwords 0-1: first 16-block, 2-3: second
                const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[j], 1.0f, 0) * sc;
                const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[j], 1.0f, 1) * sc;
                const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[j], 1.0f, 2) * sc;
                const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[j], 1.0f, 3) * sc;
                if (W64) {
                    uint2 *d2 = reinterpret_cast<uint2 *>(dst + j);
                    d2[0] = make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
                    __builtin_amdgcn_sched_barrier(0);
                    d2[1] = make_uint2(__builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
                } else {
                    dst[j] = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                        __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
                }
            }
        }
    }
};

// MFMA fragments of substep s: the wave's first A and B fragment offsets in
// the stage buffer plus constant strides (32 LDS rows per fragment), so the
// offsets live in two registers and the rest are instruction immediates.
template <int TM, int TN>
__device__ __forceinline__ void read_frags(const uint8_t *stage, int a_frag, int b_frag, int s, half8v (&af)[TM],
                                           half8v (&bf)[TN])
{
#pragma unroll
    for (int i = 0; i < TM; i++)
        af[i] = *reinterpret_cast<const half8v *>(stage + a_frag + i * 32 * kLdsRow + s * 32);
#pragma unroll
    for (int j = 0; j < TN; j++)
        bf[j] = *reinterpret_cast<const half8v *>(stage + b_frag + j * 32 * kLdsRow + s * 32);
}

// Row pitch of the bf16 C tile staged in LDS for the epilogue (16 bytes of
// padding per row).
__host__ __device__ constexpr int c_pitch(int bn) { return bn * 2 + 16; }

// All 512 threads copy the staged bf16 tile [BM][BN] to C, 16 bytes per
// non-temporal store, consecutive threads along a row.
template <int BM, int BN>
__device__ __forceinline__ void store_staged_c(const GemmArgs &g, const uint8_t *lds, int m0, int n0, int tid)
{
    constexpr int kChunks = BN / 8;                     // 16-byte chunks per row
    static_assert((BM * kChunks) % 512 == 0, "whole chunks per thread");
#pragma unroll
    for (int u = 0; u < BM * kChunks / 512; u++) {
        const int idx = tid + 512 * u;
        const int r = idx / kChunks, c = idx - r * kChunks;
        const int row = m0 + r, col = n0 + c * 8;
        if (row < g.M && col < g.N) {
            const uint4 v = *reinterpret_cast<const uint4 *>(lds + r * c_pitch(BN) + c * 16);
            store16_stream(reinterpret_cast<uint16_t *>(g.c) + (int64_t)row * g.ldc + col, v);
        }
    }
}

// EPI bit 0: stage a bf16 C tile through LDS (else store C straight from the
// accumulators); bit 1: add the LoRA branch first.  Separate instances keep
// each epilogue's registers out of the others.
template <int TM, int TN, bool KFULL, int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_nvfp4(GemmArgs g)
{
    constexpr bool LORA = (EPI & 2) != 0;
    constexpr bool STAGED = (EPI & 1) != 0;
    constexpr int BM = 64 * TM, BN = 64 * TN;
    constexpr int kStage = (BM + BN) * kLdsRow;
    constexpr int PD = kPrefetch;
    static_assert(BM * c_pitch(BN) <= 2 * kStage, "the staged C tile fits in the stage buffers");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;

    // Workgroups are dispatched round-robin over the 8 XCDs, each with its own
    // L2.  Renumber so consecutive logical ids run on one XCD.  Logical ids
    // walk bands of g.band tile rows, column after column (tm fastest inside a
    // band): the tiles an XCD runs at once then form a compact block of about
    // band x (32 / band) tiles, whose distinct A and B panels are what its L2
    // fetches per K step.
    const int nwg = g.tiles_m * g.tiles_n;
    const int per_xcd = (nwg + 7) / 8;
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int full = nwg - (per_xcd - 1) * 8;              // XCDs that host per_xcd workgroups
    const int lid = xcd < full ? xcd * per_xcd + idx : full * per_xcd + (xcd - full) * (per_xcd - 1) + idx;
    const int band = lid / (g.band * g.tiles_n);
    const int in_band = lid - band * g.band * g.tiles_n;
    const int band_rows = min(g.band, g.tiles_m - band * g.band);   // the last band may be shorter
    const int tn = in_band / band_rows;
    const int tm = band * g.band + (in_band - tn * band_rows);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (g.K + kBK - 1) / kBK;

    if (wave >= 4) {
        // ------------------------------------------------------ producers
        // Stage j lives in register slot j % PD.  Step kt decodes stage kt+1
        // into LDS buffer (kt+1)&1, then refills its slot with stage kt+1+PD.
        Producer<BM, KFULL, PD, TM == 2> pa;
        Producer<BN, KFULL, PD, TM == 2> pb;
        const int ptid = tid - 256;
        pa.init(ptid, g.a2d, m0, g.M, g.K);
        pb.init(ptid, g.b2d, n0, g.N, g.K);
        if (nk > 0) {
            static_for<0, PD>([&](auto c) {
                constexpr int S = decltype(c)::value;
                const int ks = S < nk ? S : nk - 1;         // clamped: a repeated fetch is harmless
                pa.template load<S>(g.a_codes, g.a_scales, ks);
                pb.template load<S>(g.b_codes, g.b_scales, ks);
            });
            pa.template store<0>(lds);
            pb.template store<0>(lds + BM * kLdsRow);
            const int kp = PD < nk ? PD : nk - 1;
            pa.template load<0>(g.a_codes, g.a_scales, kp);
            pb.template load<0>(g.b_codes, g.b_scales, kp);
        }
        __syncthreads();
        auto pstep = [&](int kt, auto slot_tag) {
            constexpr int NS = decltype(slot_tag)::value;
            uint8_t *nxt = lds + ((kt + 1) & 1) * kStage;
            pa.template store<NS>(nxt);
            pb.template store<NS>(nxt + BM * kLdsRow);
            const int kf = kt + 1 + PD < nk ? kt + 1 + PD : nk - 1;
            pa.template load<NS>(g.a_codes, g.a_scales, kf);
            pb.template load<NS>(g.b_codes, g.b_scales, kf);
            __syncthreads();
        };
        int kt = 0;
        for (; kt + PD < nk; kt += PD)
            static_for<0, PD>([&](auto c) {
                constexpr int S = decltype(c)::value;
                pstep(kt + S, std::integral_constant<int, (S + 1) % PD>{});
            });
        static_for<0, PD>([&](auto c) {
            constexpr int S = decltype(c)::value;
            if (kt + S + 1 < nk)
                pstep(kt + S, std::integral_constant<int, (S + 1) % PD>{});
            else if (kt + S < nk)
                __syncthreads();              // matches the consumers' last step
        });
        if (LORA) {
            // every fragment read of the main loop completed before the last
            // barrier: stage the U rows of this tile and the B rows into LDS
            const int pr = lora_row_bytes(g.lora_r);
            const int vpr = g.lora_r / 8;                   // 16-byte vectors per row
            const int total = (BM + BN) * vpr;
            constexpr int kBatch = 8;                       // loads in flight per thread
            for (int q0 = ptid; q0 < total; q0 += 256 * kBatch) {
                uint4 v[kBatch];
                // every load unconditional (an index past the end re-reads the
                // last chunk): a load under a branch would be waited for
                // before the next one is issued
#pragma unroll
                for (int u = 0; u < kBatch; u++) {
                    const int q = q0 + u * 256 < total ? q0 + u * 256 : total - 1;
                    const int row = q / vpr, cv = q - row * vpr;
                    const uint16_t *src;
                    if (row < BM) {
                        const int gr = m0 + row < g.M ? m0 + row : g.M - 1;
                        src = g.lora_u + (int64_t)gr * g.lora_r;
                    } else {
                        const int gr = n0 + row - BM < g.N ? n0 + row - BM : g.N - 1;
                        src = g.lora_b + (int64_t)gr * g.lora_r;
                    }
                    v[u] = *reinterpret_cast<const uint4 *>(src + cv * 8);
                }
#pragma unroll
                for (int u = 0; u < kBatch; u++) {
                    // past the end: the last chunk again (same value, same place)
                    const int q = q0 + u * 256 < total ? q0 + u * 256 : total - 1;
                    const int row = q / vpr, cv = q - row * vpr;
                    *reinterpret_cast<uint4 *>(lds + row * pr + cv * 16) = v[u];
                }
            }
            __syncthreads();
        }
        if (STAGED) {
            if (LORA)
                __syncthreads();                          // the consumers' reads of U and B are done
            __syncthreads();                              // the consumers staged C in LDS
            store_staged_c<BM, BN>(g, lds, m0, n0, tid);
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    const int lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    float16v acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
            acc[i][j] = float16v{};

    // fragment of MFMA tile i: LDS row (tile row + lane%32), k half (lane/32);
    // tile i adds i * 32 rows to the first one
    const int a_frag = (wm * 32 * TM + l32) * kLdsRow + half * 16;
    const int b_frag = (BM + wn * 32 * TN + l32) * kLdsRow + half * 16;

    __syncthreads();
    half8v af[2][TM], bf[2][TN];
    if (nk > 0)
        read_frags<TM, TN>(lds, a_frag, b_frag, 0, af[0], bf[0]);
    for (int kt = 0; kt < nk; kt++) {
        const uint8_t *cur = lds + (kt & 1) * kStage;
        const uint8_t *nxt = lds + ((kt + 1) & 1) * kStage;
        const bool more = kt + 1 < nk;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int p = s & 1;
            if (s < 3)
                read_frags<TM, TN>(cur, a_frag, b_frag, s + 1, af[p ^ 1], bf[p ^ 1]);
            if (s == 3) {
                // every fragment of stage kt is in registers: hand the buffer
                // back, wait for stage kt+1, fetch its first fragments under
                // this substep's MFMAs
                __syncthreads();
                if (more)
                    read_frags<TM, TN>(nxt, a_frag, b_frag, 0, af[0], bf[0]);
            }
            // weight fragment first: each lane's accumulator quad is then 4
            // consecutive output columns (vector stores in the epilogue)
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[p][j], af[p][i], acc[i][j], 0, 0, 0);
            if (s < 3) {
                // spread the next substep's LDS reads between the MFMAs
#pragma unroll
                for (int h = 0; h < TM + TN; h++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - TM - TN, 0);
            }
        }
    }

    // The lane's coordinates after the loop, recovered from the fragment
    // offsets, which are live through the main loop anyway (keeping the wave
    // and lane indices themselves alive across the loop costs registers the
    // loop does not have): arow = wm*32*TM + l32, brow = BM + wn*32*TN + l32,
    // ehalf = lane / 32.
    // The empty asm makes the offsets opaque, so the compiler derives the
    // coordinates from them here instead of keeping the index arithmetic of
    // the loop set-up alive through the loop.
    int af0 = a_frag, bf0 = b_frag;
    asm volatile("" : "+v"(af0), "+v"(bf0));
    const int arow = af0 / kLdsRow;
    const int ehalf = (af0 - arow * kLdsRow) >> 4;
    const int brow = bf0 / kLdsRow;
    float scale = *g.a_alpha * *g.b_alpha;
    if (LORA) {
        // C = scale_q * acc + lora_scale * U B^T, accumulated as
        // lora_scale * (acc * (scale_q / lora_scale) + U B^T) with bf16 MFMA
        const float f = scale / g.lora_scale;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++)
                acc[i][j] = acc[i][j] * f;
        scale = g.lora_scale;
        __syncthreads();                                  // the producers staged U and B
        const int pr = lora_row_bytes(g.lora_r);
        const uint8_t *ua_base = lds + arow * pr + ehalf * 16;
        const uint8_t *ub_base = lds + brow * pr + ehalf * 16;
        for (int kk = 0; kk < g.lora_r; kk += 16) {
            // hold the fragments of the shorter side in registers (fewer live
            // registers next to the accumulators), stream the other side
            if constexpr (TM <= TN) {
                bf16x8v ua[TM];
#pragma unroll
                for (int i = 0; i < TM; i++)
                    ua[i] = *reinterpret_cast<const bf16x8v *>(ua_base + i * 32 * pr + kk * 2);
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const bf16x8v ub = *reinterpret_cast<const bf16x8v *>(ub_base + j * 32 * pr + kk * 2);
#pragma unroll
                    for (int i = 0; i < TM; i++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ub, ua[i], acc[i][j], 0, 0, 0);
                }
            } else {
                bf16x8v ub[TN];
#pragma unroll
                for (int j = 0; j < TN; j++)
                    ub[j] = *reinterpret_cast<const bf16x8v *>(ub_base + j * 32 * pr + kk * 2);
#pragma unroll
                for (int i = 0; i < TM; i++) {
                    const bf16x8v ua = *reinterpret_cast<const bf16x8v *>(ua_base + i * 32 * pr + kk * 2);
#pragma unroll
                    for (int j = 0; j < TN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ub[j], ua, acc[i][j], 0, 0, 0);
                }
            }
        }
    }

    // epilogue: register r of lane l holds C[row = l%32][col = 8*(r/4) +
    // 4*(l/32) + r%4] of each 32x32 tile
    float amax = 0.0f;                  // max |C| over this lane's stored outputs
    if (STAGED) {
        if (LORA)
            __syncthreads();          // every wave has read its U and B fragments: LDS is free
        // bf16 tile into the (now idle) stage buffers, then all eight waves
        // write whole rows with 16-byte stores
        const int bcol0 = brow - BM - (arow & 31);                 // wn*32*TN
#pragma unroll
        for (int i = 0; i < TM; i++) {
            const int lrow = arow + i * 32;
            const bool rok = m0 + lrow < g.M;
#pragma unroll
            for (int j = 0; j < TN; j++) {
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int lcol = bcol0 + j * 32 + 8 * q + 4 * ehalf;
                    const float v0 = acc[i][j][4 * q + 0] * scale, v1 = acc[i][j][4 * q + 1] * scale;
                    const float v2 = acc[i][j][4 * q + 2] * scale, v3 = acc[i][j][4 * q + 3] * scale;
                    if (rok && n0 + lcol < g.N)         // N % 8 == 0: the quad is in or out as a whole
                        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3))));
                    const __bf16 h0 = (__bf16)v0, h1 = (__bf16)v1, h2 = (__bf16)v2, h3 = (__bf16)v3;
                    const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                    const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, h2) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
                    *reinterpret_cast<uint2 *>(lds + lrow * c_pitch(BN) + lcol * 2) = make_uint2(w0, w1);
                }
            }
        }
        __syncthreads();
        // wave = 2*wm + wn, lane = 32*half + l32
        const int ctid = ((arow / (32 * TM)) * 2 + bcol0 / (32 * TN)) * 64 + ehalf * 32 + (arow & 31);
        store_staged_c<BM, BN>(g, lds, m0, n0, ctid);
    } else {
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const int row = m0 + arow + i * 32;
        if (row >= g.M)
            continue;
#pragma unroll
        for (int j = 0; j < TN; j++) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int col = n0 + (brow - BM - (arow & 31)) + j * 32 + 8 * q + 4 * ehalf;
                const float v0 = acc[i][j][4 * q + 0] * scale, v1 = acc[i][j][4 * q + 1] * scale;
                const float v2 = acc[i][j][4 * q + 2] * scale, v3 = acc[i][j][4 * q + 3] * scale;
                const int64_t off = (int64_t)row * g.ldc + col;
                if (col + 3 < g.N)
                    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3))));
                if (col + 3 < g.N && g.vec_ok) {
                    if (g.c_bf16) {
                        const __bf16 h0 = (__bf16)v0, h1 = (__bf16)v1, h2 = (__bf16)v2, h3 = (__bf16)v3;
                        const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                                            ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                        const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, h2) |
                                            ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
                        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(g.c) + off) = make_uint2(w0, w1);
                    } else {
                        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(g.c) + off) =
                            make_float4(v0, v1, v2, v3);
                    }
                } else {
                    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        if (col + e < g.N) {
                            amax = fmaxf(amax, fabsf(v[e]));
                            if (g.c_bf16) {
                                const __bf16 h = (__bf16)v[e];
                                reinterpret_cast<uint16_t *>(g.c)[off + e] = __builtin_bit_cast(uint16_t, h);
                            } else {
                                reinterpret_cast<float *>(g.c)[off + e] = v[e];
                            }
                        }
                    }
                }
            }
        }
    }
    }
    if (g.c_amax) {
        // rounding to bf16 is monotone: the max of the stored values is the
        // rounded max
        if (g.c_bf16)
            amax = (float)(__bf16)amax;
        amax = wave_max(amax);
        // lane index recomputed (mbcnt) rather than kept live across the main loop
        if (__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) == 0)
            atomicMax(reinterpret_cast<unsigned int *>(g.c_amax), __float_as_uint(amax));
    }
}

template <int TM, int TN>
static hipError_t launch_tm_tn(GemmArgs &g, hipStream_t s)
{
    g.tiles_m = (g.M + 64 * TM - 1) / (64 * TM);
    g.tiles_n = (g.N + 64 * TN - 1) / (64 * TN);
    // Band height: the 32 tiles an XCD (32 CUs) runs at once fetch the fewest
    // panel rows per K step as a block of h x (32 / h) tiles with
    // h * BM ~ (32 / h) * BN.
    const int h = (int)std::lround(std::sqrt(32.0 * TN / TM));
    g.band = h < 1 ? 1 : (h > g.tiles_m ? g.tiles_m : h);
    const int64_t grid = (int64_t)g.tiles_m * g.tiles_n;
    if (grid * 512 > (int64_t)0xFFFFFFFF)
        return hipErrorInvalidConfiguration;   // a dispatch counts its work-items in 32 bits
    const bool kfull = g.K % kBK == 0;
    const int epi = (g.lora_u ? 2 : 0) | (g.stage_ok ? 1 : 0);
    static_for<0, 4>([&](auto e) {
        constexpr int E = decltype(e)::value;
        if (epi == E) {
            if (kfull)
                k_gemm_nvfp4<TM, TN, true, E><<<(unsigned)grid, 512, 0, s>>>(g);
            else
                k_gemm_nvfp4<TM, TN, false, E><<<(unsigned)grid, 512, 0, s>>>(g);
        }
    });
    return hipGetLastError();
}

// Estimated time of a tile shape: rounds of workgroups over the 256 CUs times
// the per-tile work, inflated for smaller tiles (more LDS traffic and decode
// per MFMA).
static double tile_cost(int64_t m, int64_t n, int tm, int tn)
{
    const int64_t tiles = ((m + 64 * tm - 1) / (64 * tm)) * ((n + 64 * tn - 1) / (64 * tn));
    const int64_t rounds = (tiles + 255) / 256;
    const double work = (double)(64 * tm) * (64 * tn);
    const double overhead = 1.0 + 0.5 * (1.0 / tm + 1.0 / tn);
    return (double)rounds * work * overhead;
}

__global__ void k_zero_float(float *p) { *p = 0.0f; }

hipError_t launch_gemm(const GemmOperand &a, const GemmOperand &b, int64_t m, int64_t n, int64_t k, void *c,
                       int cdtype, int64_t ldc, float *c_amax, hipStream_t s, const LoraBranch *lora)
{
    if (c_amax) {
        // non-negative floats order like their bit patterns: the epilogue
        // combines workgroups with an unsigned atomic max on a zeroed word
        k_zero_float<<<1, 1, 0, s>>>(c_amax);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (m == 0 || n == 0)
        return hipSuccess;
    GemmArgs g;
    g.c_amax = c_amax;
    g.lora_u = lora ? lora->u : nullptr;
    g.lora_b = lora ? lora->b : nullptr;
    g.lora_r = lora ? lora->r : 0;
    g.lora_scale = lora ? lora->scale : 1.0f;
    g.a_codes = a.codes; g.a_scales = a.scales; g.a_alpha = a.alpha; g.a2d = a.scale2d;
    g.b_codes = b.codes; g.b_scales = b.scales; g.b_alpha = b.alpha; g.b2d = b.scale2d;
    g.c = c; g.ldc = ldc; g.c_bf16 = cdtype == 1;
    g.M = (int)m; g.N = (int)n; g.K = (int)k;
    g.tiles_m = g.tiles_n = 0;
    const uintptr_t esz = cdtype == 1 ? 2 : 4;
    g.vec_ok = ((uintptr_t)c % (4 * esz) == 0) && (ldc % 4 == 0);
    g.stage_ok = cdtype == 1 && (uintptr_t)c % 16 == 0 && ldc % 8 == 0 && n % 8 == 0;
    // candidate tiles (TM, TN); 256x256 needs more registers than a 2-wave/SIMD launch has
    const int cand[4][2] = {{3, 4}, {4, 3}, {2, 4}, {2, 2}};
    int pick = 0;
    double best = tile_cost(m, n, cand[0][0], cand[0][1]);
    for (int i = 1; i < 4; i++) {
        const double cst = tile_cost(m, n, cand[i][0], cand[i][1]);
        if (cst < best) {
            best = cst;
            pick = i;
        }
    }
    switch (pick) {
    case 0: return launch_tm_tn<3, 4>(g, s);
    case 1: return launch_tm_tn<4, 3>(g, s);
    case 2: return launch_tm_tn<2, 4>(g, s);
    default: return launch_tm_tn<2, 2>(g, s);
    }
}

}  // namespace nvfp4
