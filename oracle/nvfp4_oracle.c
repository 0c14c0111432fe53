/*
 * NVFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-checkable CPU implementation of the NVFP4 format
 * and of the W4A4 contraction.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the library never does.  It shares
 * no code, header, table or constant with the HIP path.
 *
 * What it follows ("LongLive-2.0: An NVFP4 Parallel Infrastructure for Long
 * Video Generation", long-form architecture walkthrough page, section
 * "NVFP4 Training: End-to-End 4-Bit Precision for Video DiTs" and section
 * "NVFP4 Inference", plus the paper-notes page, section 3.4):
 *   - element format E2M1, values {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}
 *     ("NVFP4 numeric format");
 *   - hierarchical scaling  Xhat = X_FP4 * alpha_FP8 * alpha_FP32, one E4M3
 *     scale per 16-element block and one FP32 scale per tensor
 *     ("Hierarchical scaling" equation);
 *   - block scale alpha_FP8 = cast_E4M3(max|U_B| / M_FP4), U = X / alpha_FP32,
 *     M_FP4 = 6, M_FP8 = 448 ("Quantization rule for a tensor block");
 *   - four-over-six: try the block max mapped to 6 and to 4, keep the scale
 *     with the smaller squared reconstruction error ("Scale-search mechanism"
 *     equations, NVFP4 Inference section);
 *   - weights in 16x16 tiles, activations/gradients in 16-element vectors
 *     along the reduction dimension ("NVFP4 training recipe").
 *
 * Readings where the pages leave a step open (each is one of the numbered
 * readings listed in the design notes):
 *   R1  alpha_FP32 = RN32(amax / (M_FP8 * M_FP4)) = RN32(amax / 2688); a zero
 *       tensor gets alpha = 1.
 *   R3  fp32 evaluation order: mu = RN32(m / alpha); t_c = RN32(mu / c);
 *       s_c = E4M3(t_c); d_c = RN32(s_c * alpha); kappa_c = RN32(1 / d_c)
 *       (0 when s_c == 0); v = RN32(x * kappa_c); code = E2M1(v).
 *   R4  candidate error in the X domain: the residual d = x - q*s*alpha of
 *       each element with the exact product and a single rounding
 *       (d = fmaf(-(q*s), alpha, x); q*s is exact), then per block row an
 *       fmaf chain e = fma(d, d, e) over the row's 16 elements in index
 *       order, rows summed in order; choose 4 iff e4 < e6.
 *   R5  E4M3 rounding: nearest finite E4FN value, ties to even, subnormals
 *       kept, saturating at 448 (never NaN).
 *   R6  E2M1 rounding: nearest, ties to even, saturating at 6, the sign bit
 *       of x is kept (so -0.0 and small negatives give code 0x8).
 *   R8  element 2j in the low nibble of byte j; scales row-major.
 *
 * Every rounding step is one IEEE binary32 operation (round to nearest even);
 * the file must be built with -ffp-contract=off and without fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define NVO_ROW16 0
#define NVO_TILE16 1
#define NVO_COL16 2
#define NVO_STATIC6 0
#define NVO_4OVER6 1

/* ---------------------------------------------------------------- formats */

/* E2M1 magnitudes, indexed by the 3 low bits of a code. */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double nvo_e2m1_value(int code)
{
    double m = kE2M1[code & 7];
    return (code & 8) ? -m : m;
}

/* Nearest E2M1 magnitude by exhaustive search; ties go to the even code.
 * Values beyond 6 saturate to 6 (stated explicitly: for huge inputs the
 * double-precision distances would all round to the same number). */
int nvo_e2m1_encode(float v)
{
    int sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (a >= 6.0)                       /* at or beyond the largest value */
        return sign | 7;
    int best = 0;
    double bd = a;                      /* distance to code 0 */
    for (int c = 1; c < 8; c++) {
        double d = fabs(a - kE2M1[c]);
        if (d < bd || (d == bd && (c % 2) == 0)) {
            bd = d;
            best = c;
        }
    }
    return sign | best;
}

/* E4M3FN value of byte b in [0,126] (sign bit ignored): 4 exponent bits with
 * bias 7, 3 mantissa bits, exponent field 0 is subnormal (m * 2^-9). */
double nvo_e4m3_value(int b)
{
    int e = (b >> 3) & 15, m = b & 7;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (b & 0x80) ? -v : v;
}

/* Nearest finite non-negative E4M3 value to t >= 0 by exhaustive search over
 * bytes 0..126; ties to the even byte; anything above 448 is nearest to 448. */
int nvo_e4m3_encode(float t)
{
    double a = (double)t;
    if (a >= 448.0)
        return 126;
    int best = 0;
    double bd = fabs(a);
    for (int b = 1; b <= 126; b++) {
        double d = fabs(a - nvo_e4m3_value(b));
        if (d < bd || (d == bd && (b % 2) == 0)) {
            bd = d;
            best = b;
        }
    }
    return best;
}

/* Reading R1: decode global scale from the tensor's absolute maximum. */
float nvo_global_scale(float amax)
{
    if (amax == 0.0f)
        return 1.0f;
    return amax / 2688.0f;              /* 2688 = M_FP8 * M_FP4 = 448 * 6 */
}

/* ------------------------------------------------------- block geometry */

/* A block is described by where its elements live in x and where its codes
 * go.  Element i (canonical order) sits in block-row i / 16, column i % 16.
 *   ROW16 : 1 row,  x[r][cb*16 + j]                 scales [rows][cols/16]
 *   TILE16: 16 rows, x[rb*16 + i][cb*16 + j]         scales [rows/16][cols/16]
 *   COL16 : 1 row,  x[rb*16 + i][c]  (along rows)    scales [cols][rows/16]
 * Codes: ROW16/TILE16 [rows][cols/2]; COL16 [cols][rows/2] (the contraction
 * dimension, rows, is contiguous).  Element 2j -> low nibble of byte j. */
typedef struct {
    int64_t x_off[256];     /* element offsets into x */
    int64_t c_byte[256];    /* byte offsets into codes */
    int c_hi[256];          /* 1: high nibble */
    int n;                  /* elements in block: 16 or 256 */
    int64_t s_off;          /* offset into scales */
} block_geo;

static int64_t nblocks_of(int block, int64_t rows, int64_t cols)
{
    if (block == NVO_ROW16) return rows * (cols / 16);
    if (block == NVO_TILE16) return (rows / 16) * (cols / 16);
    return cols * (rows / 16);
}

static void geometry(int block, int64_t rows, int64_t cols, int64_t ld, int64_t b, block_geo *g)
{
    if (block == NVO_ROW16) {
        int64_t bpr = cols / 16, r = b / bpr, cb = b % bpr;
        g->n = 16;
        for (int j = 0; j < 16; j++) {
            int64_t c = cb * 16 + j;
            g->x_off[j] = r * ld + c;
            g->c_byte[j] = r * (cols / 2) + c / 2;
            g->c_hi[j] = (int)(c & 1);
        }
        g->s_off = r * bpr + cb;
    } else if (block == NVO_TILE16) {
        int64_t bpr = cols / 16, rb = b / bpr, cb = b % bpr;
        g->n = 256;
        for (int i = 0; i < 16; i++)
            for (int j = 0; j < 16; j++) {
                int64_t r = rb * 16 + i, c = cb * 16 + j;
                g->x_off[i * 16 + j] = r * ld + c;
                g->c_byte[i * 16 + j] = r * (cols / 2) + c / 2;
                g->c_hi[i * 16 + j] = (int)(c & 1);
            }
        g->s_off = rb * bpr + cb;
    } else {
        int64_t bpc = rows / 16, c = b / bpc, rb = b % bpc;
        g->n = 16;
        for (int i = 0; i < 16; i++) {
            int64_t r = rb * 16 + i;
            g->x_off[i] = r * ld + c;
            g->c_byte[i] = c * (rows / 2) + r / 2;
            g->c_hi[i] = (int)(r & 1);
        }
        g->s_off = c * bpc + rb;
    }
}

/* ------------------------------------------------------- one block */

typedef struct {
    int scale_byte;
    int codes[256];
    float err;
    float t;                /* unrounded scale argument RN32(mu / c) */
} candidate;

/* Encode a block with block max mapped to c (6 or 4). */
static void encode_candidate(const float *xs, int n, float mu, float alpha, float c, candidate *out)
{
    float t = mu / c;
    int sb = nvo_e4m3_encode(t);
    float s = (float)nvo_e4m3_value(sb);        /* exact */
    float kappa = 0.0f;
    if (s != 0.0f) {
        float d = s * alpha;
        kappa = 1.0f / d;
    }
    float e = 0.0f;
    for (int r = 0; r < n / 16; r++) {
        float er = 0.0f;
        for (int j = 0; j < 16; j++) {
            float x = xs[r * 16 + j];
            float v = x * kappa;
            int code = nvo_e2m1_encode(v);
            float q = (float)nvo_e2m1_value(code);
            float qs = q * s;                   /* exact: <= 6 significant bits */
            float d = fmaf(-qs, alpha, x);      /* x - q*s*alpha, exact product, one rounding */
            er = fmaf(d, d, er);
            out->codes[r * 16 + j] = code;
        }
        e = e + er;
    }
    out->scale_byte = sb;
    out->err = e;
    out->t = t;
}

/* Quantize one block; returns 1 when the 4-candidate was chosen. */
static int quantize_block(const float *xs, int n, float alpha, int rule, candidate *chosen, int *sat4)
{
    float m = 0.0f;
    for (int i = 0; i < n; i++) {
        float a = fabsf(xs[i]);
        if (a > m) m = a;
    }
    float mu = m / alpha;
    encode_candidate(xs, n, mu, alpha, 6.0f, chosen);
    *sat4 = 0;
    if (rule != NVO_4OVER6)
        return 0;
    candidate c4;
    encode_candidate(xs, n, mu, alpha, 4.0f, &c4);
    *sat4 = c4.t > 448.0f;
    if (c4.err < chosen->err) {
        *chosen = c4;
        return 1;
    }
    return 0;
}

/* --------------------------------------------------------- tensor level */

int nvo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

float nvo_amax(const float *x, int64_t rows, int64_t cols, int64_t ld)
{
    float a = 0.0f;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            float v = fabsf(x[r * ld + c]);
            if (v > a) a = v;
        }
    return a;
}

/* Quantize x [rows][cols] (row stride ld, fp32 values; bf16 inputs are
 * widened exactly before the call).  amax_in: NULL to use max|x|.
 * stats (may be NULL): [0] blocks choosing 4, [1] blocks whose 4-candidate
 * scale argument exceeded 448 (saturated E4M3). */
void nvo_quantize(const float *x, int64_t rows, int64_t cols, int64_t ld, int block, int rule,
                  const float *amax_in, uint8_t *codes, uint8_t *scales, float *alpha_out,
                  int64_t *stats)
{
    float amax = amax_in ? *amax_in : nvo_amax(x, rows, cols, ld);
    float alpha = nvo_global_scale(amax);
    int64_t nb = nblocks_of(block, rows, cols);
    int64_t n4 = 0, ns = 0;
    size_t ncode_bytes = (size_t)(rows * cols / 2);
    memset(codes, 0, ncode_bytes);
    /* Blocks never share a code byte (block widths are even), so blocks can
     * be processed in any order. */
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : n4, ns)
    for (int64_t b = 0; b < nb; b++) {
        block_geo g;
        float xs[256];
        candidate ch;
        int sat4 = 0;
        geometry(block, rows, cols, ld, b, &g);
        for (int i = 0; i < g.n; i++)
            xs[i] = x[g.x_off[i]];
        n4 += quantize_block(xs, g.n, alpha, rule, &ch, &sat4);
        ns += sat4;
        scales[g.s_off] = (uint8_t)ch.scale_byte;
        for (int i = 0; i < g.n; i++) {
            uint8_t nib = (uint8_t)(ch.codes[i] & 15);
            codes[g.c_byte[i]] |= g.c_hi[i] ? (uint8_t)(nib << 4) : nib;
        }
    }
    *alpha_out = alpha;
    if (stats) {
        stats[0] = n4;
        stats[1] = ns;
    }
}

/* ------------------------------------------------ random Hadamard transform */

/* The random Hadamard transform applied to the WGRAD operands before
 * quantization (architecture walkthrough page, NVFP4 Training section,
 * "Random Hadamard Transform (RHT) for gradient stabilization"): both
 * operands are multiplied by one fixed orthogonal matrix along the reduction
 * (token) axis, so dW = (R dY)^T (R X) = dY^T X before quantization.
 *
 * Reading (the pages give neither size nor construction): R = (1/4) H16 D on
 * every 16-element block of a column along the tokens, the blocks of the COL16
 * quantization; H16 the Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i&j)),
 * D = diag(d_i) with d_i = -1 where bit i of `signs` is set.  fp32 evaluation
 * order: flip the signs, then the butterfly stages h = 1, 2, 4, 8, each
 * replacing (v[i], v[i+h]) for i & h == 0 by (v[i] + v[i+h], v[i] - v[i+h])
 * (one rounding each), then multiply by 0.25. */
void nvo_rht16(float *v, unsigned signs)
{
    for (int i = 0; i < 16; i++)
        if ((signs >> i) & 1u)
            v[i] = -v[i];
    for (int h = 1; h < 16; h <<= 1)
        for (int i = 0; i < 16; i++)
            if (!(i & h)) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    for (int i = 0; i < 16; i++)
        v[i] = v[i] * 0.25f;
}

/* COL16 quantization of R x: x [rows][cols] (ld), rows % 16 == 0.  The
 * transformed tensor is formed first, then quantized exactly as nvo_quantize
 * does (its amax is that of R x). */
void nvo_quantize_col16_rht(const float *x, int64_t rows, int64_t cols, int64_t ld, int rule, unsigned signs,
                            const float *amax_in, uint8_t *codes, uint8_t *scales, float *alpha_out,
                            int64_t *stats)
{
    float *t = (float *)malloc((size_t)(rows * cols > 0 ? rows * cols : 1) * sizeof(float));
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        float v[16];
        for (int64_t rb = 0; rb < rows / 16; rb++) {
            for (int i = 0; i < 16; i++)
                v[i] = x[(rb * 16 + i) * ld + c];
            nvo_rht16(v, signs);
            for (int i = 0; i < 16; i++)
                t[(rb * 16 + i) * cols + c] = v[i];
        }
    }
    nvo_quantize(t, rows, cols, cols, NVO_COL16, rule, amax_in, codes, scales, alpha_out, stats);
    free(t);
}

/* ------------------------------------------------------------ K smoothing */

/* Key smoothing before KV quantization (architecture walkthrough page, NVFP4
 * Inference section, "Key smoothing"): every key vector loses its mean over
 * the head dimension, K'[u] = K[u] - (1/d) sum_u K[u].
 *
 * Reading of the fp32 order: partial sums of each 16-element block in index
 * order, the d/16 partials added in block order, mean = RN32(sum / d),
 * K'[u] = RN32(K[u] - mean).  The means are returned so the consumer can add
 * them back (the pages do not say what happens to them; without the add-back
 * a key's dot products with a query change by mean * sum(q)). */
void nvo_kv_smooth(const float *x, int64_t vectors, int64_t d, float *out, float *means)
{
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < vectors; v++) {
        const float *k = x + v * d;
        float s = 0.0f;
        for (int64_t b = 0; b < d / 16; b++) {
            float p = 0.0f;
            for (int i = 0; i < 16; i++)
                p = p + k[b * 16 + i];
            s = s + p;
        }
        const float m = s / (float)d;
        means[v] = m;
        for (int64_t u = 0; u < d; u++)
            out[v * d + u] = k[u] - m;
    }
}

/* Dequantize to fp32 y [rows][cols] (original orientation, row stride ldy):
 * xhat = RN32(RN32(q * s) * alpha). */
void nvo_dequantize(const uint8_t *codes, const uint8_t *scales, float alpha, int64_t rows,
                    int64_t cols, int block, float *y, int64_t ldy)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            int64_t byte, soff;
            int hi;
            if (block == NVO_ROW16) {
                byte = r * (cols / 2) + c / 2; hi = (int)(c & 1); soff = r * (cols / 16) + c / 16;
            } else if (block == NVO_TILE16) {
                byte = r * (cols / 2) + c / 2; hi = (int)(c & 1); soff = (r / 16) * (cols / 16) + c / 16;
            } else {
                byte = c * (rows / 2) + r / 2; hi = (int)(r & 1); soff = c * (rows / 16) + r / 16;
            }
            int code = hi ? (codes[byte] >> 4) : (codes[byte] & 15);
            float q = (float)nvo_e2m1_value(code);
            float s = (float)nvo_e4m3_value(scales[soff]);
            float qs = q * s;
            y[r * ldy + c] = qs * alpha;
        }
}

/* ------------------------------------------------------------ GEMM (fp64) */

/* A GEMM operand is a packed matrix of `rows` rows and K columns (K is the
 * contraction dimension, contiguous): codes [rows][K/2]; scales 1D
 * [rows][K/16] (scale2d = 0) or 2D [rows/16][K/16] (scale2d = 1).  Returns
 * q * s (exact in double) for element (r, k). */
static double operand_value(const uint8_t *codes, const uint8_t *scales, int scale2d, int64_t K,
                            int64_t r, int64_t k)
{
    uint8_t byte = codes[r * (K / 2) + k / 2];
    int code = (k & 1) ? (byte >> 4) : (byte & 15);
    int64_t soff = scale2d ? (r / 16) * (K / 16) + k / 16 : r * (K / 16) + k / 16;
    return nvo_e2m1_value(code) * nvo_e4m3_value(scales[soff]);
}

static void dequant_operand_f64(const uint8_t *codes, const uint8_t *scales, int scale2d,
                                int64_t rows, int64_t K, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < K; k++)
            out[r * K + k] = operand_value(codes, scales, scale2d, K, r, k);
}

/* C[m][n] = alpha_a * alpha_b * sum_k Ahat[m][k] * Bhat[n][k], in fp64 with a
 * sequential k loop, then times alpha_a, then times alpha_b. */
int nvo_gemm_f64(const uint8_t *ca, const uint8_t *sa, float alpha_a, int a2d,
                 const uint8_t *cb, const uint8_t *sb, float alpha_b, int b2d,
                 int64_t M, int64_t N, int64_t K, double *C)
{
    double *A = (double *)malloc((size_t)(M * K) * sizeof(double));
    double *B = (double *)malloc((size_t)(N * K) * sizeof(double));
    if (!A || !B) {
        free(A);
        free(B);
        return -1;
    }
    dequant_operand_f64(ca, sa, a2d, M, K, A);
    dequant_operand_f64(cb, sb, b2d, N, K, B);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++)
                acc += A[m * K + k] * B[n * K + k];
            C[m * N + n] = acc * (double)alpha_a * (double)alpha_b;
        }
    free(A);
    free(B);
    return 0;
}

/* Same contraction for a list of (m, n) output positions only. */
void nvo_gemm_f64_sampled(const uint8_t *ca, const uint8_t *sa, float alpha_a, int a2d,
                          const uint8_t *cb, const uint8_t *sb, float alpha_b, int b2d,
                          int64_t K, const int64_t *ms, const int64_t *ns, int64_t count,
                          double *out)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < count; i++) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++)
            acc += operand_value(ca, sa, a2d, K, ms[i], k) * operand_value(cb, sb, b2d, K, ns[i], k);
        out[i] = acc * (double)alpha_a * (double)alpha_b;
    }
}

/* ------------------------------------- diagnostic: exact-real reading */

/* The same rule evaluated in exact real arithmetic (no fp32 steps after
 * alpha): scale s_c = E4M3(m / (alpha * c)) and code = E2M1(x / (s * alpha))
 * decided by exact comparisons in double (all products below have <= 32
 * significant bits), error sum in long double.  Used only to count how often
 * the fp32 reading R3 differs from it. */
static int e4m3_encode_ratio(double num, double den)    /* nearest to num/den, den > 0 */
{
    int best = 0;
    for (int b = 1; b <= 126; b++) {
        /* compare |num - v_b*den| against |num - v_best*den|, exact */
        double db = fabs(num - nvo_e4m3_value(b) * den);
        double dbest = fabs(num - nvo_e4m3_value(best) * den);
        if (db < dbest || (db == dbest && (b % 2) == 0)) best = b;
    }
    return best;
}

static int e2m1_encode_ratio(double x, double d)        /* nearest to x/d, d > 0 */
{
    int sign = signbit(x) ? 8 : 0;
    double a = fabs(x);
    int best = 0;
    double bd = a;
    for (int c = 1; c < 8; c++) {
        double dd = fabs(a - kE2M1[c] * d);
        if (dd < bd || (dd == bd && (c % 2) == 0)) {
            bd = dd;
            best = c;
        }
    }
    return sign | best;
}

void nvo_quantize_exact_reading(const float *x, int64_t rows, int64_t cols, int64_t ld, int block,
                                int rule, uint8_t *codes, uint8_t *scales, float *alpha_out)
{
    float alpha = nvo_global_scale(nvo_amax(x, rows, cols, ld));
    int64_t nb = nblocks_of(block, rows, cols);
    memset(codes, 0, (size_t)(rows * cols / 2));
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t b = 0; b < nb; b++) {
        block_geo g;
        geometry(block, rows, cols, ld, b, &g);
        double m = 0.0;
        for (int i = 0; i < g.n; i++)
            if (fabs((double)x[g.x_off[i]]) > m) m = fabs((double)x[g.x_off[i]]);
        int sbs[2], cds[2][256];
        long double errs[2];
        int nc = rule == NVO_4OVER6 ? 2 : 1;
        for (int ci = 0; ci < nc; ci++) {
            double c = ci == 0 ? 6.0 : 4.0;
            int sb = e4m3_encode_ratio(m, (double)alpha * c);
            double sa = nvo_e4m3_value(sb) * (double)alpha;      /* exact */
            long double e = 0.0L;
            for (int i = 0; i < g.n; i++) {
                double xv = (double)x[g.x_off[i]];
                int code = sa > 0.0 ? e2m1_encode_ratio(xv, sa) : (signbit(xv) ? 8 : 0);
                long double d = (long double)xv - (long double)nvo_e2m1_value(code) * (long double)sa;
                e += d * d;
                cds[ci][i] = code;
            }
            sbs[ci] = sb;
            errs[ci] = e;
        }
        int pick = (nc == 2 && errs[1] < errs[0]) ? 1 : 0;
        scales[g.s_off] = (uint8_t)sbs[pick];
        for (int i = 0; i < g.n; i++) {
            uint8_t nib = (uint8_t)(cds[pick][i] & 15);
            codes[g.c_byte[i]] |= g.c_hi[i] ? (uint8_t)(nib << 4) : nib;
        }
    }
    *alpha_out = alpha;
}
