/*
 * fp8_oracle.c -- plain, slow, obviously-correct CPU reference for FP8 scaled
 * quantization and the scaled FP8 GEMM it feeds.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP library is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no source, header, table or
 * helper with the HIP library, and the library never calls it.
 *
 * Built with:  gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fopenmp
 * (no FMA contraction, IEEE binary32/binary64 arithmetic, OpenMP only across
 * independent rows/groups so that every per-element result is order-free).
 *
 * Sources for what is computed (web pages; see the citations per function):
 *   [DeepL]  "DeepL bets on FP8: unified-precision training and inference"
 *            (hmyw.cn/news/121341), sections 2.1, 2.3, 4.2, 5.1.
 *   [H100]   "H100 FP8 acceleration, measured" (scrxy.com/news/908489),
 *            paragraph on the FP8 formats (OCP origin, E5M2 range +-57344).
 *   [Soup]   "FP8 training and QAT: ... with Soup on Hopper GPUs"
 *            (lbrq.cn/news/198264), table of the three FP8 scaling recipes.
 * Where the pages are silent (rounding mode, saturation, NaN codes, scale edge
 * cases, block sizes) this file takes one documented reading; each such
 * reading is marked "READING:".
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>
#include <float.h>
#include <omp.h>
#include <stdlib.h>

enum { OR_E4M3 = 0, OR_E5M2 = 1 };
enum { OR_GRAN_TENSOR = 0, OR_GRAN_ROW = 1, OR_GRAN_1x128 = 2, OR_GRAN_128x128 = 3 };
enum { OR_IN_F32 = 0, OR_IN_BF16 = 1 };

/* ------------------------------------------------------------------------ */
/* Bit-level helpers (IEEE binary32 as stored in memory).                    */
/* ------------------------------------------------------------------------ */
static inline uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 is by definition the upper half of a binary32 word. */
static inline float bf16_to_f32(uint16_t h) { return u2f(((uint32_t)h) << 16); }

static inline float load_in(const void* x, int in_dtype, int64_t idx) {
    if (in_dtype == OR_IN_F32) return ((const float*)x)[idx];
    return bf16_to_f32(((const uint16_t*)x)[idx]);
}

/* ------------------------------------------------------------------------ */
/* O1. Decode: the value of every code, from the bit split.                  */
/* [DeepL] 2.1: E4M3 = 1 sign, 4 exponent, 3 mantissa bits; E5M2 = 1 sign,   */
/* 5 exponent, 2 mantissa bits.  [H100] formats paragraph: the formats are    */
/* the jointly defined (OCP) ones and E5M2 reaches +-57344.                   */
/* READING: OCP "E4M3FN" -- bias 7, no infinities, S.1111.111 is NaN, so the  */
/* largest finite value is 448; E5M2 -- bias 15, IEEE-style Inf/NaN.          */
/* ------------------------------------------------------------------------ */
double or_decode(int fmt, uint8_t code) {
    int sign = (code >> 7) & 1;
    double mag;
    if (fmt == OR_E4M3) {
        int e = (code >> 3) & 0xF, m = code & 0x7;
        if (e == 15 && m == 7) return NAN;
        if (e == 0) mag = ldexp((double)m, -9);            /* m/8 * 2^(1-7) */
        else        mag = ldexp(1.0 + m / 8.0, e - 7);
    } else {
        int e = (code >> 2) & 0x1F, m = code & 0x3;
        if (e == 31) {
            if (m != 0) return NAN;
            mag = INFINITY;
        } else if (e == 0) mag = ldexp((double)m, -16);   /* m/4 * 2^(1-15) */
        else               mag = ldexp(1.0 + m / 4.0, e - 15);
    }
    return sign ? -mag : mag;
}

void or_decode_table(int fmt, double* out256) {
    for (int c = 0; c < 256; ++c) out256[c] = or_decode(fmt, (uint8_t)c);
}

/* Largest finite magnitude and the code that holds it. */
static double fmt_max(int fmt) { return fmt == OR_E4M3 ? 448.0 : 57344.0; }
static int fmt_max_code(int fmt) { return fmt == OR_E4M3 ? 0x7E : 0x7B; }

double or_format_max(int fmt) { return fmt_max(fmt); }

/* ------------------------------------------------------------------------ */
/* O2. Encode one binary32 value: saturating round-to-nearest-even.          */
/* READING (the pages name neither rounding nor saturation): the code of the  */
/* finite FP8 value nearest to v; on an exact tie the code with an even       */
/* mantissa (LSB 0); |v| >= max finite (Inf included) gives +-max; NaN gives  */
/* the all-ones-exponent/mantissa NaN code with v's sign; the sign of v is    */
/* kept on underflow (-tiny -> 0x80).                                         */
/* Done as a nearest-value search over the decoded positive codes, which are  */
/* monotone in the code value -- deliberately not a bit manipulation.         */
/* ------------------------------------------------------------------------ */
uint8_t or_encode(int fmt, float v) {
    uint8_t sign = (uint8_t)(signbit(v) ? 0x80 : 0x00);
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    int top = fmt_max_code(fmt);
    if (a >= fmt_max(fmt)) return (uint8_t)(sign | top);
    /* largest code lo in [0, top] with decode(lo) <= a */
    int lo = 0, hi = top;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (or_decode(fmt, (uint8_t)mid) <= a) lo = mid; else hi = mid - 1;
    }
    double vlo = or_decode(fmt, (uint8_t)lo);
    if (vlo == a) return (uint8_t)(sign | lo);
    double vhi = or_decode(fmt, (uint8_t)(lo + 1));
    double half = 0.5 * (vlo + vhi);   /* exact: one more mantissa bit */
    int pick;
    if (a < half) pick = lo;
    else if (a > half) pick = lo + 1;
    else pick = (lo % 2 == 0) ? lo : lo + 1;   /* tie: even code */
    return (uint8_t)(sign | pick);
}

void or_encode_array(int fmt, const float* v, int64_t n, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = or_encode(fmt, v[i]);
}

/* ------------------------------------------------------------------------ */
/* O3. amax = max |x| over a group ([DeepL] 4.2 names the per-layer maximum  */
/* absolute value as the statistic behind the scale).                        */
/* READING for non-finite data: any NaN makes the result NaN (the one with    */
/* the largest magnitude bits), else any Inf makes it Inf.  For non-negative  */
/* binary32 values the unsigned order of the bit patterns is the numeric     */
/* order, and NaN patterns sort above Inf, so the result is the element of    */
/* largest |bits|.                                                            */
/* ------------------------------------------------------------------------ */
static inline uint32_t abs_bits(float v) { return f2u(v) & 0x7FFFFFFFu; }

/* Group geometry for a [rows x cols] matrix with leading dimension ld.
 * READING (block sizes are not on the pages): 1x128 and 128x128 blocks
 * aligned at element (0,0); a final partial block covers the remainder.   */
static void group_dims(int gran, int64_t rows, int64_t cols,
                       int64_t* gr, int64_t* gc, int64_t* h, int64_t* w) {
    /* an empty tensor (or an empty row) is still one group, of amax 0 */
    int64_t r1 = rows > 0 ? rows : 1, c1 = cols > 0 ? cols : 1;
    switch (gran) {
    case OR_GRAN_TENSOR: *h = r1; *w = c1;  break;
    case OR_GRAN_ROW:    *h = 1;  *w = c1;  break;
    case OR_GRAN_1x128:  *h = 1;  *w = 128; break;
    default:             *h = 128; *w = 128; break;
    }
    *gr = (gran == OR_GRAN_TENSOR) ? 1 : (rows + *h - 1) / *h;
    *gc = (gran == OR_GRAN_TENSOR || gran == OR_GRAN_ROW) ? 1 : (cols + *w - 1) / *w;
}

int64_t or_num_groups(int gran, int64_t rows, int64_t cols) {
    int64_t gr, gc, h, w;
    group_dims(gran, rows, cols, &gr, &gc, &h, &w);
    return gr * gc;
}

/* amax_out[g] for every group g (row-major over the group grid). */
void or_amax(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
             int gran, float* amax_out) {
    int64_t gr, gc, h, w;
    group_dims(gran, rows, cols, &gr, &gc, &h, &w);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t g = 0; g < gr * gc; ++g) {
        int64_t r0 = (g / gc) * h, c0 = (g % gc) * w;
        int64_t r1 = r0 + h < rows ? r0 + h : rows;
        int64_t c1 = c0 + w < cols ? c0 + w : cols;
        uint32_t best = 0;
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t c = c0; c < c1; ++c) {
                uint32_t b = abs_bits(load_in(x, in_dtype, r * ld + c));
                if (b > best) best = b;
            }
        amax_out[g] = u2f(best);
    }
}

/* ------------------------------------------------------------------------ */
/* O4. Scale from amax.  [DeepL] 2.3: a scaling factor maps the raw values    */
/* into the interval FP8 can represent.  READING: multiply before the cast    */
/* by s = fl32(fmax / amax) (no margin); dequantize by s_inv = fl32(1/s).     */
/* Edge cases (silent on the pages): amax == 0 or non-finite -> s = 1; a      */
/* quotient that overflows -> FLT_MAX.                                        */
/* [Soup] recipe table: the rowwise recipe uses power-of-two scales --        */
/* READING: truncate the binary32 quotient to 2^floor(log2 s) by clearing its */
/* mantissa bits (FLT_MAX becomes 2^127).                                     */
/* ------------------------------------------------------------------------ */
void or_scale(float amax, int fmt, int pow2, float* s_out, float* s_inv_out) {
    float s;
    float fmax = (float)fmt_max(fmt);
    if (!(amax > 0.0f) || isinf(amax) || isnan(amax)) {
        s = 1.0f;
    } else {
        s = fmax / amax;                 /* one IEEE binary32 division */
        if (isinf(s)) s = FLT_MAX;
    }
    if (pow2) s = u2f(f2u(s) & 0xFF800000u);
    *s_out = s;
    *s_inv_out = 1.0f / s;
}

/* ------------------------------------------------------------------------ */
/* O5. Quantize: q = encode(fl32(x * s_group)).                               */
/* Optional counters: sat = non-NaN products with |x*s| > fmax (Inf inputs     */
/* included); nonfinite = NaN or Inf inputs; underflow = nonzero, non-NaN      */
/* inputs whose code is +-0.                                                   */
/* scales[g] supplies s for group g (row-major over the group grid).          */
/* ------------------------------------------------------------------------ */
void or_quantize_with_scales(const void* x, int in_dtype, int64_t rows, int64_t cols,
                             int64_t ld, int gran, int fmt, const float* scales,
                             uint8_t* q, int64_t ldq, int64_t* counts3) {
    int64_t gr, gc, h, w;
    group_dims(gran, rows, cols, &gr, &gc, &h, &w);
    double fmax = fmt_max(fmt);
    int64_t sat = 0, nonfinite = 0, under = 0;
    #pragma omp parallel for schedule(static) reduction(+:sat, nonfinite, under)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            int64_t g = (r / h) * gc + (c / w);
            float xv = load_in(x, in_dtype, r * ld + c);
            float v = xv * scales[g];          /* rounded once to binary32 */
            uint8_t code = or_encode(fmt, v);
            q[r * ldq + c] = code;
            if (!isnan(v) && fabs((double)v) > fmax) ++sat;
            if (isnan(xv) || isinf(xv)) ++nonfinite;
            if (!isnan(xv) && xv != 0.0f && (code & 0x7F) == 0) ++under;
        }
    }
    if (counts3) { counts3[0] = sat; counts3[1] = nonfinite; counts3[2] = under; }
}

/* Just-in-time quantize: amax per group, scale per group, cast. */
void or_quantize(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                 int gran, int fmt, int pow2, uint8_t* q, int64_t ldq,
                 float* amax_out, float* scale_out, float* scale_inv_out,
                 int64_t* counts3) {
    int64_t ng = or_num_groups(gran, rows, cols);
    or_amax(x, in_dtype, rows, cols, ld, gran, amax_out);
    for (int64_t g = 0; g < ng; ++g)
        or_scale(amax_out[g], fmt, pow2, &scale_out[g], &scale_inv_out[g]);
    or_quantize_with_scales(x, in_dtype, rows, cols, ld, gran, fmt, scale_out, q, ldq, counts3);
}

/* ------------------------------------------------------------------------ */
/* O6. Delayed scaling.  [DeepL] 2.3: the factor for this step is predicted   */
/* from statistics of the previous steps, so no synchronous per-step amax is  */
/* needed; it lags a sudden change of distribution.                           */
/* READING: per tensor; the history holds the raw amax of the last            */
/* min(count, len) steps (len <= 16); this step's scale is                    */
/* scale(max over the history), the current step excluded; with an empty      */
/* history (first step) the scale is taken just in time from this step's      */
/* amax.  After the cast this step's amax is pushed into the ring.            */
/* ------------------------------------------------------------------------ */
typedef struct {
    float amax[16];
    int32_t len, pos, count;
} or_ring;

void or_ring_init(or_ring* r, int32_t len) {
    memset(r, 0, sizeof(*r));
    r->len = len;
}

float or_ring_window_max(const or_ring* r) {
    uint32_t best = 0;
    for (int i = 0; i < r->count; ++i) {
        uint32_t b = abs_bits(r->amax[i]);
        if (b > best) best = b;
    }
    return u2f(best);
}

/* One delayed step on a whole tensor.  out4 = {s, s_inv, amax, spiked}.
 * [DeepL] 2.3 also describes the recovery from a sudden change of the
 * distribution that delayed scaling lags behind: compare the current
 * statistic with the history and recompute the scaling factor past a
 * threshold.  READING: the statistic is this step's amax, the history's is
 * the window max, "past a threshold" is amax > threshold * window_max (an
 * fp32 product), and the recomputed factor is the just-in-time scale of
 * this step's amax; the ring is updated as without the guard.  A threshold
 * <= 0 (the default) or an empty window never triggers. */
void or_delayed_step(or_ring* r, const void* x, int in_dtype, int64_t rows, int64_t cols,
                     int64_t ld, int fmt, uint8_t* q, int64_t ldq, float spike_threshold,
                     float* out4, int64_t* counts3) {
    float amax_now;
    or_amax(x, in_dtype, rows, cols, ld, OR_GRAN_TENSOR, &amax_now);
    float basis = (r->count == 0) ? amax_now : or_ring_window_max(r);
    int spiked = 0;
    if (r->count > 0 && spike_threshold > 0.0f) {
        float limit = spike_threshold * or_ring_window_max(r);
        if (amax_now > limit) {
            spiked = 1;
            basis = amax_now;
        }
    }
    float s, s_inv;
    or_scale(basis, fmt, 0, &s, &s_inv);
    or_quantize_with_scales(x, in_dtype, rows, cols, ld, OR_GRAN_TENSOR, fmt, &s, q, ldq, counts3);
    r->amax[r->pos] = amax_now;
    r->pos = (r->pos + 1) % r->len;
    if (r->count < r->len) r->count += 1;
    out4[0] = s; out4[1] = s_inv; out4[2] = amax_now; out4[3] = (float)spiked;
}

/* ------------------------------------------------------------------------ */
/* O7. Scaled GEMM, Y = X . W^T with both operands K-contiguous.             */
/* Step 1, dequantize every operand element: A_hat = fl32(decode(q) * s_inv) */
/* with the s_inv of the element's group; decode(q) is read from the table   */
/* of all 256 codes that or_decode (the closed form above) fills.            */
/* Step 2, an fp32 triple loop: Y32[m,n] = sum over k, in k order, of        */
/* fl32(A_hat[m,k] * B_hat[n,k]), one rounding per product and per add; and  */
/* P = sum_k |A_hat * B_hat| in fp64 for the error floor.                    */
/* Scale layouts: a_per_row / b_per_row select a scalar or one scale per row */
/* of A (per output row) / of B (per output column).  The block-scaled form  */
/* ([DeepL] 2.3, per-block scaling) has one scale per (row of A, 128-wide K  */
/* block), a_inv[m*(K/128)+kb], and one per (128 rows of B, 128-wide K       */
/* block), b_inv[(n/128)*(K/128)+kb]; it needs K % 128 == 0.                 */
/* OpenMP splits the outputs across threads; each output is one thread's     */
/* k-ordered chain, so the results do not depend on the thread count.        */
/* ------------------------------------------------------------------------ */
typedef struct {
    float a[256], b[256];   /* decode tables of the two formats */
} or_tables;

static void fill_tables(int fa, int fb, or_tables* t) {
    for (int c = 0; c < 256; ++c) {
        t->a[c] = (float)or_decode(fa, (uint8_t)c);   /* every FP8 value is a binary32 value */
        t->b[c] = (float)or_decode(fb, (uint8_t)c);
    }
}

/* Scale of element (r, k) of an operand: mode 0 = one scalar, 1 = one per
 * row, 2 = A's 1x128 blocks, 3 = B's 128x128 blocks (K % 128 == 0). */
enum { SC_SCALAR = 0, SC_ROW = 1, SC_A_BLOCK = 2, SC_B_BLOCK = 3 };

static inline float scale_at(const float* s, int mode, int64_t r, int64_t k, int64_t kb_n) {
    switch (mode) {
    case SC_SCALAR:  return s[0];
    case SC_ROW:     return s[r];
    case SC_A_BLOCK: return s[r * kb_n + k / 128];
    default:         return s[(r / 128) * kb_n + k / 128];
    }
}

/* Step 1 for rows [0, rows) of one operand into out[rows x K]. */
static void dequantize_rows(const uint8_t* q, int64_t ldq, int64_t rows, int64_t K, const float* tab,
                            const float* s, int mode, float* out) {
    int64_t kb_n = K / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = tab[q[r * ldq + k]] * scale_at(s, mode, r, k, kb_n);
}

/* Step 2 for one output: the k-ordered fp32 sum and the fp64 sum of |products|. */
static inline void dot_f32(const float* a, const float* b, int64_t K, float* y, double* p) {
    float acc = 0.0f;
    double pabs = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        float prod = a[k] * b[k];
        acc = acc + prod;
        pabs += fabs((double)a[k] * (double)b[k]);
    }
    *y = acc;
    *p = pabs;
}

/* Every output of an M x N problem.  B_hat is formed once; each thread
 * forms the row of A_hat it works on. */
static void gemm_full(const uint8_t* A, int fa, int64_t lda, const float* a_inv, int amode,
                      const uint8_t* B, int fb, int64_t ldb, const float* b_inv, int bmode,
                      int64_t M, int64_t N, int64_t K, float* Y32, int64_t ldy, double* P, int64_t ldp) {
    or_tables t;
    fill_tables(fa, fb, &t);
    int64_t kb_n = K / 128;
    float* Bh = (float*)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1) * (size_t)(K > 0 ? K : 1));
    dequantize_rows(B, ldb, N, K, t.b, b_inv, bmode, Bh);
    #pragma omp parallel
    {
        float* Ah = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t k = 0; k < K; ++k) Ah[k] = t.a[A[m * lda + k]] * scale_at(a_inv, amode, m, k, kb_n);
            for (int64_t nn = 0; nn < N; ++nn) {
                float y;
                double p;
                dot_f32(Ah, Bh + nn * K, K, &y, &p);
                Y32[m * ldy + nn] = y;
                if (P) P[m * ldp + nn] = p;
            }
        }
        free(Ah);
    }
    free(Bh);
}

/* The outputs (ms[i], ns[i]), each dequantizing its own row pair. */
static void gemm_sampled(const uint8_t* A, int fa, int64_t lda, const float* a_inv, int amode,
                         const uint8_t* B, int fb, int64_t ldb, const float* b_inv, int bmode, int64_t K,
                         const int64_t* ms, const int64_t* ns, int64_t n, float* y32, double* p64) {
    or_tables t;
    fill_tables(fa, fb, &t);
    int64_t kb_n = K / 128;
    #pragma omp parallel
    {
        float* ab = (float*)malloc(sizeof(float) * 2 * (size_t)(K > 0 ? K : 1));
        #pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < n; ++i) {
            int64_t m = ms[i], nn = ns[i];
            for (int64_t k = 0; k < K; ++k) {
                ab[k] = t.a[A[m * lda + k]] * scale_at(a_inv, amode, m, k, kb_n);
                ab[K + k] = t.b[B[nn * ldb + k]] * scale_at(b_inv, bmode, nn, k, kb_n);
            }
            double p;
            dot_f32(ab, ab + K, K, &y32[i], &p);
            if (p64) p64[i] = p;
        }
        free(ab);
    }
}

void or_gemm_sampled(const uint8_t* A, int fa, int64_t lda, const uint8_t* B, int fb, int64_t ldb,
                     int64_t K, const float* a_inv, int a_per_row, const float* b_inv, int b_per_row,
                     const int64_t* ms, const int64_t* ns, int64_t n, float* y32, double* p64) {
    gemm_sampled(A, fa, lda, a_inv, a_per_row ? SC_ROW : SC_SCALAR, B, fb, ldb, b_inv,
                 b_per_row ? SC_ROW : SC_SCALAR, K, ms, ns, n, y32, p64);
}

void or_gemm(const uint8_t* A, int fa, int64_t lda, const uint8_t* B, int fb, int64_t ldb,
             int64_t M, int64_t N, int64_t K, const float* a_inv, int a_per_row,
             const float* b_inv, int b_per_row, float* Y32, int64_t ldy, double* P, int64_t ldp) {
    gemm_full(A, fa, lda, a_inv, a_per_row ? SC_ROW : SC_SCALAR, B, fb, ldb, b_inv,
              b_per_row ? SC_ROW : SC_SCALAR, M, N, K, Y32, ldy, P, ldp);
}

void or_blockgemm_sampled(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, int64_t K,
                          const float* a_inv, const float* b_inv,
                          const int64_t* ms, const int64_t* ns, int64_t n, float* y32, double* p64) {
    gemm_sampled(A, OR_E4M3, lda, a_inv, SC_A_BLOCK, B, OR_E4M3, ldb, b_inv, SC_B_BLOCK, K, ms, ns, n,
                 y32, p64);
}

void or_blockgemm(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, int64_t M, int64_t N,
                  int64_t K, const float* a_inv, const float* b_inv, float* Y32, int64_t ldy, double* P,
                  int64_t ldp) {
    gemm_full(A, OR_E4M3, lda, a_inv, SC_A_BLOCK, B, OR_E4M3, ldb, b_inv, SC_B_BLOCK, M, N, K, Y32, ldy,
              P, ldp);
}

/* ------------------------------------------------------------------------ */
/* Exact pin for O7: every finite E4M3 value is an integer multiple of 2^-9   */
/* and every finite E5M2 value of 2^-16, so each product and the whole K sum  */
/* are exact integers at scale 2^-(ea+eb).  D is accumulated in __int128.     */
/* Returns Y_exact = s_a * s_b * D * 2^-(ea+eb) in fp64 (long double product  */
/* for the final scaling).  Block mode sums per K block with its own scales.  */
/* Non-finite codes are not allowed here (the caller filters them).           */
/* ------------------------------------------------------------------------ */
static void int_table(int fmt, int64_t* t) {
    /* decode(code) * 2^9 (E4M3) or * 2^16 (E5M2): an exact integer */
    for (int c = 0; c < 256; ++c) {
        double v = or_decode(fmt, (uint8_t)c) * (fmt == OR_E4M3 ? 512.0 : 65536.0);
        t[c] = isfinite(v) ? (int64_t)v : 0;
    }
}

void or_gemm_exact_sampled(const uint8_t* A, int fa, int64_t lda, const uint8_t* B, int fb,
                           int64_t ldb, int64_t K, const float* a_inv, int a_per_row,
                           const float* b_inv, int b_per_row, int block_mode,
                           const int64_t* ms, const int64_t* ns, int64_t n, double* y_exact) {
    int64_t kb_n = K / 128;
    int shift = (fa == OR_E4M3 ? 9 : 16) + (fb == OR_E4M3 ? 9 : 16);
    int64_t ta[256], tb[256];
    int_table(fa, ta);
    int_table(fb, tb);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n; ++i) {
        int64_t m = ms[i], nn = ns[i];
        long double total = 0.0L;
        if (!block_mode) {
            __int128 d = 0;
            for (int64_t k = 0; k < K; ++k)
                d += (__int128)ta[A[m * lda + k]] * (__int128)tb[B[nn * ldb + k]];
            float sa = a_per_row ? a_inv[m] : a_inv[0];
            float sb = b_per_row ? b_inv[nn] : b_inv[0];
            total = (long double)d * (long double)sa * (long double)sb;
        } else {
            for (int64_t kb = 0; kb < kb_n; ++kb) {
                __int128 d = 0;
                for (int64_t k = kb * 128; k < kb * 128 + 128; ++k)
                    d += (__int128)ta[A[m * lda + k]] * (__int128)tb[B[nn * ldb + k]];
                total += (long double)d * (long double)a_inv[m * kb_n + kb]
                         * (long double)b_inv[(nn / 128) * kb_n + kb];
            }
        }
        y_exact[i] = (double)ldexpl(total, -shift);
    }
}

/* ------------------------------------------------------------------------ */
/* O8. Output rounding to bfloat16, round-to-nearest-even (NaN stays NaN).    */
/* Done as the nearest-value rule on the two bf16 neighbours of v, ties to   */
/* the even one -- written out rather than as an add-and-shift trick.         */
/* ------------------------------------------------------------------------ */
uint16_t or_f32_to_bf16(float v) {
    uint32_t b = f2u(v);
    if (isnan(v)) return (uint16_t)((b >> 16) | 0x0040);   /* quiet NaN, sign kept */
    uint32_t down = b & 0xFFFF0000u;                        /* toward zero */
    float lo = u2f(down);
    if (lo == v) return (uint16_t)(down >> 16);
    uint32_t up = down + 0x00010000u;                       /* next magnitude */
    float hi = u2f(up);                                     /* may be Inf */
    double dv = fabs((double)v), dlo = fabs((double)lo);
    double dhi = isinf(hi) ? ldexp(1.0, 128) : fabs((double)hi);
    double half = 0.5 * (dlo + dhi);
    uint32_t pick;
    if (dv < half) pick = down;
    else if (dv > half) pick = up;
    else pick = ((down >> 16) & 1u) ? up : down;
    return (uint16_t)(pick >> 16);
}

void or_f32_to_bf16_array(const float* v, int64_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = or_f32_to_bf16(v[i]);
}

/* ------------------------------------------------------------------------ */
/* O9. FP8 KV cache.  [DeepL] 3.1: holding the attention K and V caches in    */
/* FP8 halves their memory against BF16 (longer contexts, larger batches);   */
/* K's precision drives the attention scores, V's the mixed output, and      */
/* keeping a single layer's K cache in BF16 removed a long-sequence error.    */
/* READING (the page fixes no layout, granularity or scale rule):             */
/*  - one layer's K (or V) cache is [capacity x heads x head_dim], head_dim   */
/*    contiguous.  New token t (of n, x row t at x + t*ld) goes to cache row  */
/*    slots[t]; slots == NULL means row t; a slot outside [0, capacity) is    */
/*    not stored (padding).                                                   */
/*  - PER_TOKEN_HEAD: each (token, head) vector of head_dim values is one     */
/*    group: amax (O3), scale (O4, pow2 optional), cast (O5), and             */
/*    scale_inv[slot*heads + head] is stored beside the codes.                */
/*  - PER_HEAD: a fixed, calibrated scale_inv[head] is given; the cast        */
/*    multiplies by s = fl32(1 / scale_inv[head]).                            */
/*  - BF16 storage (the per-layer fallback): the values rounded to bf16 (O8), */
/*    no scale.                                                               */
/*  - load gathers cache rows slots[t] (NULL: row t) into out row t:          */
/*    y = fl32(decode(q) * scale_inv), kept in fp32 or rounded to bf16 (O8);   */
/*    a BF16 cache returns its values.  A slot outside [0, capacity) leaves   */
/*    out row t untouched.                                                    */
/* ------------------------------------------------------------------------ */
enum { OR_KV_E4M3 = 0, OR_KV_E5M2 = 1, OR_KV_BF16 = 2 };
enum { OR_KV_PER_TOKEN_HEAD = 0, OR_KV_PER_HEAD = 1 };

void or_kv_store(const void* x, int in_dtype, int64_t n, int64_t heads, int64_t head_dim,
                 int64_t ld, const int64_t* slots, int64_t capacity, int storage, int scaling,
                 int pow2, void* cache, float* scale_inv, int64_t* counts3) {
    int64_t sat = 0, nonfinite = 0, under = 0;
    for (int64_t t = 0; t < n; ++t) {
        int64_t slot = slots ? slots[t] : t;
        if (slot < 0 || slot >= capacity) continue;
        for (int64_t h = 0; h < heads; ++h) {
            int64_t src = t * ld + h * head_dim;
            int64_t dst = (slot * heads + h) * head_dim;
            if (storage == OR_KV_BF16) {
                for (int64_t c = 0; c < head_dim; ++c)
                    ((uint16_t*)cache)[dst + c] = or_f32_to_bf16(load_in(x, in_dtype, src + c));
                continue;
            }
            float s, s_inv;
            if (scaling == OR_KV_PER_TOKEN_HEAD) {
                /* one row of one group: O3 and O4 as for row-wise scaling */
                float amax;
                or_amax((const char*)x + src * (in_dtype == OR_IN_F32 ? 4 : 2), in_dtype,
                        1, head_dim, head_dim, OR_GRAN_ROW, &amax);
                or_scale(amax, storage, pow2, &s, &s_inv);
                scale_inv[slot * heads + h] = s_inv;
            } else {
                s = 1.0f / scale_inv[h];
            }
            int64_t c3[3];
            or_quantize_with_scales((const char*)x + src * (in_dtype == OR_IN_F32 ? 4 : 2),
                                    in_dtype, 1, head_dim, head_dim, OR_GRAN_TENSOR, storage,
                                    &s, (uint8_t*)cache + dst, head_dim, c3);
            sat += c3[0]; nonfinite += c3[1]; under += c3[2];
        }
    }
    if (counts3) { counts3[0] = sat; counts3[1] = nonfinite; counts3[2] = under; }
}

void or_kv_load(const void* cache, int storage, int scaling, const float* scale_inv,
                int64_t n, int64_t heads, int64_t head_dim, const int64_t* slots,
                int64_t capacity, int out_bf16, void* out, int64_t ld_out) {
    for (int64_t t = 0; t < n; ++t) {
        int64_t slot = slots ? slots[t] : t;
        if (slot < 0 || slot >= capacity) continue;
        for (int64_t h = 0; h < heads; ++h) {
            int64_t src = (slot * heads + h) * head_dim;
            int64_t dst = t * ld_out + h * head_dim;
            float sinv = 1.0f;
            if (storage != OR_KV_BF16)
                sinv = scaling == OR_KV_PER_TOKEN_HEAD ? scale_inv[slot * heads + h] : scale_inv[h];
            for (int64_t c = 0; c < head_dim; ++c) {
                float y;
                if (storage == OR_KV_BF16)
                    y = bf16_to_f32(((const uint16_t*)cache)[src + c]);
                else
                    y = (float)or_decode(storage, ((const uint8_t*)cache)[src + c]) * sinv;
                if (out_bf16) ((uint16_t*)out)[dst + c] = or_f32_to_bf16(y);
                else ((float*)out)[dst + c] = y;
            }
        }
    }
}

/* Threads the OpenMP loops above use (reported with CPU timings). */
int or_num_threads(void) { return omp_get_max_threads(); }

/* Threads of the parallel loops above (timing only; results do not depend on it). */
void or_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
