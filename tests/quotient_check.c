/* The block quantizer's division-free quotients against IEEE division.
 *
 * The GPU quantizer forms mu = m / alpha and mu / 6 (the "Four Over Six"
 * candidate scales of a block with max |x| = m) as
 *     q = fma(fma(-q0, b, a), y, q0),  q0 = a * y,  y = RN(1 / b)
 * with a and b first scaled by sc = 1 (alpha >= 2^-90) or 2^100.  This
 * restates that arithmetic in C (fmaf is the IEEE fused multiply-add) and
 * checks it against the correctly rounded division:
 *   1. every pair (b, a) of significands in [1, 2), a a bf16 significand;
 *   2. a / 6 for every 61st float a >= 2^-123 (normal quotients);
 *   3. the E4M3 scale bytes (nearest-even, clamped at 448) for random alpha
 *      over the whole float range (subnormal and zero alpha included) and
 *      random block maxima including 0, infinity and NaN.
 * Exit status 0 and "quotient check ok" when every case agrees. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float fbits(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t ubits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float div_rcp(float a, float b, float y) { const float q0 = a * y; return fmaf(fmaf(-q0, b, a), y, q0); }

static double e4v[127];
static int e4m3_byte(float t)                      /* t >= 0 or NaN; NaN and t >= 448 give 448 */
{
    t = fminf(t, 448.0f);
    if (t >= 448.0f) return 126;
    int lo = 0, hi = 126;
    while (hi - lo > 1) { const int mid = (lo + hi) / 2; if (e4v[mid] <= t) lo = mid; else hi = mid; }
    const double dl = t - e4v[lo], dh = e4v[hi] - t;
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1) ? hi : lo;
}

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) { rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17; return rs; }

int main(void)
{
    for (int c = 0; c < 127; c++) {
        const int e = c >> 3, m = c & 7;
        e4v[c] = e == 0 ? m / 8.0 * ldexp(1.0, -6) : (1 + m / 8.0) * ldexp(1.0, e - 7);
    }
    unsigned long long bad1 = 0, bad2 = 0, bad3 = 0, n3 = 0;
    for (uint32_t B = 0; B < (1u << 23); B++) {
        const float b = fbits(0x3f800000u | B), y = 1.0f / b;
        for (uint32_t A = 0; A < 128; A++) {
            const float a = fbits(0x3f800000u | (A << 16));
            bad1 += ubits(div_rcp(a, b, y)) != ubits(a / b);
        }
    }
    const float r6 = 1.0f / 6.0f;
    for (uint32_t u = ubits(0x1p-123f); u < 0x7f800000u; u += 61) {
        const float a = fbits(u);
        bad2 += ubits(div_rcp(a, 6.0f, r6)) != ubits(a / 6.0f);
    }
    for (int t = 0; t < 2000; t++) {
        const float amax = t == 0 ? 0x1p-149f : fbits((uint32_t)(rnd() % 0x7f800000u));
        const float alpha = amax / 2688.0f;                    /* 0 for the smallest maxima */
        const float sc = alpha >= 0x1p-90f ? 1.0f : 0x1p100f;
        const float y = 1.0f / (alpha * sc);
        for (int k = 0; k < 20000; k++) {
            const uint64_t q = rnd();
            float m;
            if (k == 0) m = 0.0f;
            else if (k == 1) m = INFINITY;
            else if (k == 2) m = NAN;
            else if (q & 1) m = fbits(ubits(amax) - (uint32_t)((q >> 1) % (1u << 28)));
            else m = amax * ((float)((q >> 8) & 0xffffff) / 16777216.0f);
            if (m < 0.0f) continue;
            const float ref = m / alpha;
            const float mu = div_rcp(m * sc, alpha * sc, y);
            n3++;
            bad3 += e4m3_byte(div_rcp(mu, 6.0f, r6)) != e4m3_byte(ref / 6.0f) ||
                    e4m3_byte(mu * 0.25f) != e4m3_byte(ref * 0.25f);
        }
    }
    printf("significand pairs: %llu wrong; a/6: %llu wrong; scale bytes: %llu wrong of %llu\n", bad1, bad2, bad3, n3);
    if (bad1 || bad2 || bad3) return 1;
    printf("quotient check ok\n");
    return 0;
}
