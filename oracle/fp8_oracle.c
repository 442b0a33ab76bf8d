/*
 * fp8_oracle.c -- plain, slow, CPU reference for the MoE FP8 training hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark load this file's library.  It shares no code, header, table or constant
 * generator with the GPU library, and the GPU library never calls it.
 *
 * What it follows (page titles as printed on the pages):
 *   [P1] "AMD Boosts PyTorch FP8 Training on Instinct GPUs" (latestnews.news), 3rd paragraph:
 *        the FNUZ format (finite, no NaN, unsigned zero) and grouped GEMM for MoE.
 *   [P3] "FP8 su GPU AMD ..." (ai-radar.it):
 *        intro -- rowwise scales on activations, colwise scales on expert weights, an offset
 *                 tensor that routes tokens to experts;
 *        "La correttezza del formato viene prima del tuning" -- e4m3fnuz, largest value 240,
 *                 no NaN/Inf encoding, scales must be taken against the target format's max;
 *        "Il guadagno vero e' nel movimento dei dati" -- the chain absmax per row or column,
 *                 scale, clamp, cast to FP8; the transposed colwise operand of the backward.
 *   [P4] "AMD Primus adds FP8/MXFP8 kernels, megakernel fusion and DeepSeek-V3 training at 1024
 *        GPUs" (fosswire.org), "What Primus adds for MoE training on MI355X": FP8 and MXFP8
 *        grouped GEMM.  The pages do not define MXFP8; the OCP Microscaling Formats (MX) v1.0
 *        specification does (1x32 blocks, E8M0 shared scale, e4m3 elements).
 *   OCP e4m3fn (bias 7, largest value 448, one NaN code per sign, signed zero) is from the OCP
 *   8-bit floating point specification; the pages only call it the standard (non-AMD) format.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - zero absmax: the scale uses max(absmax, 1e-12f);
 *   - cast rounding: round to nearest, ties to the even code; no stochastic rounding;
 *   - the stored scale is the quant multiplier s = FMAX / absmax (fp32, correctly rounded);
 *     dequantization multiplies by 1/s;
 *   - the chain is: fp32 product x*s (rounded), then clamp to [-FMAX, FMAX], then FP8 rounding;
 *   - e4m3fnuz never yields 0x80 (its NaN); any value that rounds to zero gives 0x00;
 *     e4m3fn keeps the sign of zero (0x80 for -0 and negative underflow);
 *   - offsets are int32 cumulative group END indices, offsets[G-1] == rows, empty groups allowed;
 *   - the colwise output is the column-major copy of the whole 2-D input, q_t[c * ld + r];
 *   - grouped GEMM output: the exact sum divided by s_a*s_b (the caller's output type, bf16 or
 *     fp32, is a rounding of it).
 *
 * Precision: the quantization chain is evaluated in IEEE fp32 (the precision in which the
 * GPU takes the same integer decisions).  GEMM sums are accumulated in fp64: every fp8 x fp8
 * product is a multiple of 2^-18 (e4m3fn) or 2^-20 (e4m3fnuz) below 2^17.7 in magnitude, so
 * every partial sum of up to 2^17 terms is exactly representable and the sum is exact (all
 * contractions here are far shorter).  The exact sum is then divided by the fp64 product of
 * the two fp32 scales and returned unrounded; it is the value the matrix cores' fp32
 * accumulation approximates.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -fPIC -shared -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OR_FNUZ 0 /* e4m3fnuz: bias 8, max 240, 0x80 = NaN, no negative zero */
#define OR_FN 1   /* OCP e4m3fn: bias 7, max 448, 0x7F/0xFF = NaN */

static const float OR_EPS = 1e-12f;

/* ---------------------------------------------------------------- bf16 helpers */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float bf16_to_f32(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp64 -> bf16, round to nearest, ties to even (directly from fp64, one rounding). */
uint16_t or_f64_to_bf16(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    int neg = v < 0;
    double a = neg ? -v : v;
    int e;
    double f = frexp(a, &e);           /* a = f * 2^e, f in [0.5, 1) */
    int ue = e - 1;                    /* a = (2f) * 2^ue, 2f in [1, 2) */
    if (ue < -126) ue = -126;          /* bf16 subnormal range: fixed quantum 2^-133 */
    double quantum = ldexp(1.0, ue - 7);
    double q = nearbyint(a / quantum); /* default rounding mode: to nearest even */
    double r = q * quantum;
    float rf = (float)r;               /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, 4);
    uint16_t out = (uint16_t)(u >> 16);
    if (neg) out |= 0x8000;
    return out;
}

/* ---------------------------------------------------------------- codec (c1) */

/* Format maximum: 240 for e4m3fnuz as the ai-radar.it page fixes it (format-correctness
 * section); 448 for OCP e4m3fn. */
float or_fmax(int fmt) { return fmt == OR_FNUZ ? 240.0f : 448.0f; }

/* Decode one byte from its bit fields: s = b>>7, e = (b>>3)&15, m = b&7. */
double or_decode(int fmt, unsigned b) {
    unsigned s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (fmt == OR_FNUZ) {
        if (b == 0x80) return NAN;                       /* the single NaN code */
        v = (e == 0) ? m * ldexp(1.0, -10) : ldexp(1.0 + m / 8.0, (int)e - 8);
    } else {
        if (e == 15 && m == 7) return NAN;               /* 0x7F, 0xFF */
        v = (e == 0) ? m * ldexp(1.0, -9) : ldexp(1.0 + m / 8.0, (int)e - 7);
    }
    return s ? -v : v;
}

/* Largest positive finite code; positive codes 0..max are increasing in value. */
static unsigned max_code(int fmt) { return fmt == OR_FNUZ ? 0x7Fu : 0x7Eu; }

/* Encode a finite fp32 y with |y| <= FMAX: the representable value nearest to y, a tie going
 * to the code whose mantissa LSB is 0.  Found by binary search over the positive codes, which
 * are sorted by value. */
unsigned or_encode(int fmt, float y) {
    int neg = signbit(y) != 0;
    double a = fabs((double)y);
    unsigned lo = 0, hi = max_code(fmt);
    /* invariant: dec(lo) <= a; find the largest code lo with dec(lo) <= a */
    while (lo < hi) {
        unsigned mid = (lo + hi + 1) / 2;
        if (or_decode(fmt, mid) <= a) lo = mid; else hi = mid - 1;
    }
    unsigned code = lo;
    if (lo < max_code(fmt)) {
        double d0 = a - or_decode(fmt, lo);         /* exact in fp64 */
        double d1 = or_decode(fmt, lo + 1) - a;
        if (d1 < d0) code = lo + 1;
        else if (d1 == d0) code = (lo & 1) ? lo + 1 : lo;
    }
    if (fmt == OR_FNUZ) return code == 0 ? 0u : (code | (neg ? 0x80u : 0u));
    return code | (neg ? 0x80u : 0u);
}

/* Vector form of or_encode for brute-force checks. */
void or_encode_array(int fmt, const float* y, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)or_encode(fmt, y[i]);
}

/* One element of the chain after the scale is known: y = RNE32(x*s), clamp, encode. */
static unsigned scale_clamp_cast(int fmt, float x, float s) {
    float fmax = or_fmax(fmt);
    float y = x * s;                      /* fp32 multiply, correctly rounded */
    if (y > fmax) y = fmax;
    if (y < -fmax) y = -fmax;
    return or_encode(fmt, y);
}

/* Scale from an absmax: s = RNE32(FMAX / max(amax, EPS)). */
float or_scale(int fmt, float amax) {
    float d = amax > OR_EPS ? amax : OR_EPS;
    return or_fmax(fmt) / d;              /* fp32 divide, correctly rounded */
}

/* ---------------------------------------------------------------- rowwise quant (c2) */

/* Rowwise scales on activations ([P3] intro) with the absmax -> scale -> clamp -> cast chain
 * ([P3] data-movement section).  x: bf16 bits [rows][ld_x]; q: [rows][ld_q]; s: [rows]. */
void or_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                      uint8_t* q, int64_t ld_q, float* s) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float amax = 0.0f;
        for (int64_t c = 0; c < cols; c++) {
            float a = fabsf(bf16_to_f32(x[r * ld_x + c]));
            if (a > amax) amax = a;
        }
        float sc = or_scale(fmt, amax);
        s[r] = sc;
        for (int64_t c = 0; c < cols; c++)
            q[r * ld_q + c] = (uint8_t)scale_clamp_cast(fmt, bf16_to_f32(x[r * ld_x + c]), sc);
    }
}

/* ---------------------------------------------------------------- colwise-grouped quant (c3) */

/* Colwise scales per token group ([P3] intro: offset tensor; data-movement section: the
 * backward's transposed operand written directly instead of through a transpose copy).
 * Group g covers rows [offsets[g-1], offsets[g]) with offsets[-1] = 0.  For every group g and
 * column c: amax over the group's rows, s[g*cols + c], and q_t[c*ld_qt + r] for each row r of
 * the group.  An empty group writes its scales (FMAX/EPS) and no bytes. */
void or_quant_colwise_grouped(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              const int32_t* offsets, int32_t groups, int fmt, uint8_t* q_t,
                              int64_t ld_qt, float* s) {
    (void)rows;
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t g = 0; g < groups; g++) {
        for (int64_t c = 0; c < cols; c++) {
            int64_t r0 = g == 0 ? 0 : offsets[g - 1];
            int64_t r1 = offsets[g];
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; r++) {
                float a = fabsf(bf16_to_f32(x[r * ld_x + c]));
                if (a > amax) amax = a;
            }
            float sc = or_scale(fmt, amax);
            s[(int64_t)g * cols + c] = sc;
            for (int64_t r = r0; r < r1; r++)
                q_t[c * ld_qt + r] = (uint8_t)scale_clamp_cast(fmt, bf16_to_f32(x[r * ld_x + c]), sc);
        }
    }
}

/* ---------------------------------------------------------------- grouped GEMM (c4) */

static int32_t group_of_row(const int32_t* offsets, int32_t groups, int64_t m) {
    for (int32_t g = 0; g < groups; g++)
        if (m < offsets[g]) return g;
    return -1;
}

/* Forward, M-grouped ([P1] grouped GEMM for MoE; [P3] intro).  For row m of group g:
 *   out[i*N + n] = sum_k dec(a[m*lda + k]) * dec(b[g*b_gs + n*ldb + k]) / (sa[m] * sb[g*N + n])
 * for each requested row m = row_idx[i].  The sum is exact in fp64 (no rounding). */
void or_gemm_fwd_rows(int fmt, const uint8_t* a, int64_t lda, const float* sa, const uint8_t* b,
                      int64_t ldb, int64_t b_gs, const float* sb, const int32_t* offsets,
                      int32_t groups, int64_t N, int64_t K, const int64_t* row_idx, int64_t nrows,
                      double* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; i++) {
        int64_t m = row_idx[i];
        int32_t g = group_of_row(offsets, groups, m);
        for (int64_t n = 0; n < N; n++) {
            if (g < 0) { out[i * N + n] = 0.0; continue; }
            const uint8_t* ar = a + m * lda;
            const uint8_t* br = b + g * b_gs + n * ldb;
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) acc += or_decode(fmt, ar[k]) * or_decode(fmt, br[k]);
            out[i * N + n] = acc / ((double)sa[m] * (double)sb[(int64_t)g * N + n]);
        }
    }
}

/* Weight gradient, K-grouped: for group g, dW_g[k][n] = sum over rows m of group g of
 * dec(xt[k*ldx + m]) * dec(dyt[n*ldd + m]) / (sx[g*K + k] * sdy[g*N + n]).
 * Computes the requested (g, k) output rows: out[i*N + n] for (g_idx[i], k_idx[i]).
 * An empty group gives zeros. */
void or_gemm_wgrad_rows(int fmt, const uint8_t* xt, int64_t ldx, const float* sx,
                        const uint8_t* dyt, int64_t ldd, const float* sdy, const int32_t* offsets,
                        int32_t groups, int64_t N, int64_t K, const int32_t* g_idx,
                        const int64_t* k_idx, int64_t nrows, double* out) {
    (void)groups;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; i++) {
        int32_t g = g_idx[i];
        int64_t k = k_idx[i];
        int64_t m0 = g == 0 ? 0 : offsets[g - 1], m1 = offsets[g];
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            for (int64_t m = m0; m < m1; m++)
                acc += or_decode(fmt, xt[k * ldx + m]) * or_decode(fmt, dyt[n * ldd + m]);
            out[i * N + n] = acc / ((double)sx[(int64_t)g * K + k] * (double)sdy[(int64_t)g * N + n]);
        }
    }
}

/* ---------------------------------------------------------------- MXFP8 (c5) */

/* E8M0 exponent of one 1x32 block (OCP MX v1.0): e = floor(log2(amax)) - 8, where 8 is the
 * exponent of e4m3's largest normal (448 = 1.75 * 2^8), clamped to [-127, 127]; an all-zero
 * block gets e = -127.  The stored byte is e + 127. */
static int mx_exponent(float amax) {
    if (amax == 0.0f) return -127;
    int ex;
    (void)frexpf(amax, &ex);      /* amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex - 1 */
    int e = (ex - 1) - 8;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* One element: y = x * 2^-e (fp32), clamp to +-448, encode as OCP e4m3fn. */
static unsigned mx_cast(float x, int e) {
    float y = (float)((double)x * ldexp(1.0, -e));
    if (y > 448.0f) y = 448.0f;
    if (y < -448.0f) y = -448.0f;
    return or_encode(OR_FN, y);
}

/* MX quant along rows: blocks of 32 consecutive columns.  cols % 32 == 0.
 * q: [rows][ld_q] bytes; e8: [rows][ld_s] E8M0 bytes, ld_s >= cols/32. */
void or_mx_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                         int64_t ld_q, uint8_t* e8, int64_t ld_s) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t kb = 0; kb < cols / 32; kb++) {
            float amax = 0.0f;
            for (int64_t j = 0; j < 32; j++) {
                float a = fabsf(bf16_to_f32(x[r * ld_x + kb * 32 + j]));
                if (a > amax) amax = a;
            }
            int e = mx_exponent(amax);
            e8[r * ld_s + kb] = (uint8_t)(e + 127);
            for (int64_t j = 0; j < 32; j++)
                q[r * ld_q + kb * 32 + j] = (uint8_t)mx_cast(bf16_to_f32(x[r * ld_x + kb * 32 + j]), e);
        }
    }
}

/* MX quant along the row dimension with a transposed output: blocks of 32 consecutive rows of
 * one column.  rows % 32 == 0.  q_t[c*ld_qt + r]; e8[c*ld_s + r/32]. */
void or_mx_quant_colwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q_t,
                         int64_t ld_qt, uint8_t* e8, int64_t ld_s) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        for (int64_t rb = 0; rb < rows / 32; rb++) {
            float amax = 0.0f;
            for (int64_t j = 0; j < 32; j++) {
                float a = fabsf(bf16_to_f32(x[(rb * 32 + j) * ld_x + c]));
                if (a > amax) amax = a;
            }
            int e = mx_exponent(amax);
            e8[c * ld_s + rb] = (uint8_t)(e + 127);
            for (int64_t j = 0; j < 32; j++)
                q_t[c * ld_qt + rb * 32 + j] =
                    (uint8_t)mx_cast(bf16_to_f32(x[(rb * 32 + j) * ld_x + c]), e);
        }
    }
}

/* MX grouped GEMM, forward.  For row m of group g:
 *   out[i*N + n] = sum_kb 2^(ea + eb) * sum_{k in kb} dec(a[m,k]) * dec(b_g[n,k])
 * with ea = ae8[m*ld_sa + kb] - 127 and eb = be8[g*bs_gs + n*ld_sb + kb] - 127. */
void or_mx_gemm_fwd_rows(const uint8_t* a, int64_t lda, const uint8_t* ae8, int64_t ld_sa,
                         const uint8_t* b, int64_t ldb, int64_t b_gs, const uint8_t* be8,
                         int64_t ld_sb, int64_t bs_gs, const int32_t* offsets, int32_t groups,
                         int64_t N, int64_t K, const int64_t* row_idx, int64_t nrows, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; i++) {
        int64_t m = row_idx[i];
        int32_t g = group_of_row(offsets, groups, m);
        for (int64_t n = 0; n < N; n++) {
            if (g < 0) { out[i * N + n] = 0.0; continue; }
            double acc = 0.0;
            for (int64_t kb = 0; kb < K / 32; kb++) {
                double part = 0.0;
                for (int64_t j = 0; j < 32; j++) {
                    int64_t k = kb * 32 + j;
                    part += or_decode(OR_FN, a[m * lda + k]) * or_decode(OR_FN, b[g * b_gs + n * ldb + k]);
                }
                int ea = (int)ae8[m * ld_sa + kb] - 127;
                int eb = (int)be8[g * bs_gs + n * ld_sb + kb] - 127;
                acc += ldexp(part, ea + eb);
            }
            out[i * N + n] = acc;
        }
    }
}

/* MX grouped GEMM, weight gradient (K-grouped): the token dimension is the contraction, in 1x32
 * blocks of absolute token rows (the blocks fp8_mx_quant_colwise forms over all M rows).  A block
 * that straddles a group boundary keeps its one scale; each group sums only its own tokens:
 *   out[i*N + n] = sum_{m in g} dec(xt[k,m]) 2^(ex[k, m/32] - 127) dec(dyt[n,m]) 2^(ed[n, m/32] - 127)
 * for (g, k) = (g_idx[i], k_idx[i]).  Products are summed exactly per block, then scaled. */
void or_mx_gemm_wgrad_rows(const uint8_t* xt, int64_t ldx, const uint8_t* xe8, int64_t ld_sx,
                           const uint8_t* dyt, int64_t ldd, const uint8_t* de8, int64_t ld_sd,
                           const int32_t* offsets, int32_t groups, int64_t N,
                           const int32_t* g_idx, const int64_t* k_idx, int64_t nrows,
                           double* out) {
    (void)groups;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; i++) {
        int32_t g = g_idx[i];
        int64_t k = k_idx[i];
        int64_t m0 = g == 0 ? 0 : offsets[g - 1], m1 = offsets[g];
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            int64_t m = m0;
            while (m < m1) {
                int64_t blk = m / 32, stop = (blk + 1) * 32 < m1 ? (blk + 1) * 32 : m1;
                double part = 0.0;
                for (; m < stop; m++)
                    part += or_decode(OR_FN, xt[k * ldx + m]) * or_decode(OR_FN, dyt[n * ldd + m]);
                int ex = (int)xe8[k * ld_sx + blk] - 127, ed = (int)de8[n * ld_sd + blk] - 127;
                acc += ldexp(part, ex + ed);
            }
            out[i * N + n] = acc;
        }
    }
}

/* Threads OpenMP will use (reported next to CPU timings), and a way to change it (the CPU
 * baseline is timed at one thread and at all threads). */
#ifdef _OPENMP
#include <omp.h>
int or_num_threads(void) { return omp_get_max_threads(); }
void or_set_num_threads(int n) { if (n > 0) omp_set_num_threads(n); }
#else
int or_num_threads(void) { return 1; }
void or_set_num_threads(int n) { (void)n; }
#endif
